/* Counter-based input streams for the synthetic workloads (input plumbing only).
 *
 * SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) used as a
 * counter hash: value i of stream key K is mix(K + (i+1)*GAMMA).  Uniforms on
 * (0,1) are ((x >> 11) + 0.5) * 2^-53; normals are Box-Muller pairs over
 * (u[2p], u[2p+1]): element 2p = R cos(2 pi u2), 2p+1 = R sin(2 pi u2),
 * R = sqrt(-2 ln u1).  Work is split over threads by index range; every value
 * depends only on (key, index), so the result does not depend on the split.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27; z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t tid) { return mix(seed * GAMMA + tid); }

static inline double unif(uint64_t key, uint64_t i) {
  return ((double)(mix(key + (i + 1) * GAMMA) >> 11) + 0.5) * 0x1p-53;
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unif(key, 2 * p), u2 = unif(key, 2 * p + 1);
  double rad = sqrt(-2.0 * log(u1));
  double ang = 2.0 * M_PI * u2;
  return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef struct {
  uint64_t key, start, lo, hi;
  double stdv;
  int kind;   /* 0: f32 normal, 1: bf16 normal, 2: f64 uniform */
  void* out;
} job_t;

static void* run(void* arg) {
  job_t* j = (job_t*)arg;
  for (uint64_t k = j->lo; k < j->hi; ++k) {
    uint64_t i = j->start + k;
    if (j->kind == 0) ((float*)j->out)[k] = (float)(normal_at(j->key, i) * j->stdv);
    else if (j->kind == 1) ((uint16_t*)j->out)[k] = f32_to_bf16_rne((float)(normal_at(j->key, i) * j->stdv));
    else ((double*)j->out)[k] = unif(j->key, i);
  }
  return 0;
}

static void dispatch(uint64_t key, uint64_t start, uint64_t count, double stdv, int kind, void* out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (count < 65536) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  uint64_t per = (count + nthreads - 1) / nthreads;
  int used = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t lo = per * t, hi = lo + per > count ? count : lo + per;
    if (lo >= hi) break;
    jobs[t] = (job_t){key, start, lo, hi, stdv, kind, out};
    if (pthread_create(&th[t], 0, run, &jobs[t]) != 0) { run(&jobs[t]); th[t] = 0; }
    used = t + 1;
  }
  for (int t = 0; t < used; ++t) if (th[t]) pthread_join(th[t], 0);
}

void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, double stdv, float* out, int nthreads) {
  dispatch(synth_stream_key(seed, tid), start, count, stdv, 0, out, nthreads);
}
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, double stdv, uint16_t* out, int nthreads) {
  dispatch(synth_stream_key(seed, tid), start, count, stdv, 1, out, nthreads);
}
void synth_uniform(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, double* out, int nthreads) {
  dispatch(synth_stream_key(seed, tid), start, count, 1.0, 2, out, nthreads);
}
