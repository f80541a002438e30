// ORACLE for latent causal multi-head attention -- TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, fp64 CPU statement of what the attention path computes.  Only
// the tests, the smoke check and the benchmark's CPU-baseline leg may load
// this file's library; the product path never does.  It shares no code,
// header, table or helper with the HIP library.
//
// Definition followed (POPCORNBENCH page FW-GLM-5-1 l2_p31, the latent
// attention problem, its restatement of the reference model's algorithm),
// in this file's notation: for batch b, head h and query position t, the
// keys are the positions s with 0 <= s <= t (causal, inclusive), and
//   K_s[e]  = sum_rho L[b,s,rho] * Wk[rho,h,e],   V_s[e] = sum_rho L[b,s,rho] * Wv[rho,h,e]
//   z_s     = scale * sum_e Q[b,t,h,e] * K_s[e]
//   p_s     = exp(z_s - max_s z) / sum_s' exp(z_s' - max_s z)
//   O[b,t,h,e] = sum_s p_s * V_s[e]
// with L = kv_latent [B,T,r], Wk = w_up_k and Wv = w_up_v [r,H,d], Q = q
// [B,T,H,d].  The softmax is taken in the page's three passes (the maximum,
// the sum of the exponentials, the division).  K and V are materialised
// explicitly, once per (b, h).
//
// Down-projection (POPCORNBENCH page FW-GLM-5-1 l2_p1, the KV compression
// problem: its list of shapes and operations): latent = hidden @ w_down with
// hidden [B*T, D] and w_down [D, r] row-major, no transpose.
//
// Decode: one query per sequence at position L_b - 1, attending the L_b
// cached latents 0 .. L_b - 1 (the same causal definition for its last row).
//
// Key mask (optional, [B, Tlat] bytes, 0 = masked): a masked key's logit is
// -infinity before the softmax, as the MSA page's attention fills masked
// scores with -inf ahead of its softmax (page Kimi-K2.6 l2_p29, its model
// walk-through and its analysis of rows whose every key is masked).  The
// same two-pass softmax then gives weight 0 to masked keys, and a row with no
// unmasked key gets NaN weights (-inf - -inf), hence a NaN output, which is
// what that softmax produces.
//
// Inputs are read from their stored bits (float32, bf16 or float64) and
// widened exactly to double; every sum runs in ascending index order in
// double; results are returned in double.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F64 = 2 };

// Exact widening of one stored element to double.
double load(const void* p, int dt, size_t i) {
  if (dt == DT_F32) return (double)((const float*)p)[i];
  if (dt == DT_F64) return ((const double*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;  // bf16 -> f32 is a shift
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

struct Problem {
  const void* q; int dt_q;            // query rows [n, d] (already gathered per row)
  const void* lat; int dt_lat;        // kv_latent [B, Tlat, r]
  const void* wk; const void* wv; int dt_w;  // w_up_k / w_up_v [r, H, d]
  long Tlat, H, d, r;
  double scale;
  const long* row_b; const long* row_h; const long* row_nkeys;
  double* out;                        // [n, d]
  double* probs; long pstride;        // optional [n, pstride]
  const uint8_t* key_mask;            // optional [B, Tlat], 0 = masked
};

// One (b, h) pair: materialise k and v for the key positions needed, then
// evaluate each requested query row of that pair.
void attend_group(const Problem& P, const std::vector<long>& rows) {
  const long b = P.row_b[rows[0]], h = P.row_h[rows[0]];
  long nk = 0;
  for (long i : rows) nk = std::max(nk, P.row_nkeys[i]);
  const long d = P.d, r = P.r, H = P.H;
  std::vector<double> k(nk * d), v(nk * d);
  for (long s = 0; s < nk; ++s) {
    for (long e = 0; e < d; ++e) {
      double ks = 0.0, vs = 0.0;
      for (long rho = 0; rho < r; ++rho) {
        const double lat = load(P.lat, P.dt_lat, (size_t)(b * P.Tlat + s) * r + rho);
        const size_t w = (size_t)(rho * H + h) * d + e;
        ks += lat * load(P.wk, P.dt_w, w);
        vs += lat * load(P.wv, P.dt_w, w);
      }
      k[s * d + e] = ks;
      v[s * d + e] = vs;
    }
  }
  std::vector<double> logit(nk), p(nk);
  for (long i : rows) {
    const long n = P.row_nkeys[i];  // keys s = 0 .. n-1
    for (long s = 0; s < n; ++s) {
      double dot = 0.0;
      for (long e = 0; e < d; ++e) dot += load(P.q, P.dt_q, (size_t)i * d + e) * k[s * d + e];
      logit[s] = dot * P.scale;
      if (P.key_mask && !P.key_mask[(size_t)b * P.Tlat + s]) logit[s] = -INFINITY;
    }
    double m = logit[0];
    for (long s = 1; s < n; ++s) m = std::max(m, logit[s]);
    double z = 0.0;
    for (long s = 0; s < n; ++s) z += std::exp(logit[s] - m);
    for (long s = 0; s < n; ++s) p[s] = std::exp(logit[s] - m) / z;
    for (long e = 0; e < d; ++e) {
      double acc = 0.0;
      for (long s = 0; s < n; ++s) acc += p[s] * v[s * d + e];
      P.out[(size_t)i * d + e] = acc;
    }
    if (P.probs)
      for (long s = 0; s < n; ++s) P.probs[(size_t)i * P.pstride + s] = p[s];
  }
}

int nthreads_or_default(int nthreads) {
  if (nthreads > 0) return nthreads;
  unsigned hc = std::thread::hardware_concurrency();
  return hc ? (int)hc : 1;
}

}  // namespace

extern "C" {

// Number of worker threads the oracle uses for a given request (0 = all cores).
int oracle_threads(int nthreads) { return nthreads_or_default(nthreads); }

// latent[m, j] = sum_i hidden[m, i] * w_down[i, j]; hidden [M, D], w_down [D, r].
int oracle_down_proj(const void* hidden, int dt_hidden, const void* w_down, int dt_w,
                     long M, long D, long r, double* latent) {
  if (!hidden || !w_down || !latent || M < 0 || D < 1 || r < 1) return 1;
  for (long m = 0; m < M; ++m)
    for (long j = 0; j < r; ++j) {
      double acc = 0.0;
      for (long i = 0; i < D; ++i)
        acc += load(hidden, dt_hidden, (size_t)m * D + i) * load(w_down, dt_w, (size_t)i * r + j);
      latent[(size_t)m * r + j] = acc;
    }
  return 0;
}

// Attention for an arbitrary list of query rows.  Row i is the query vector
// q_rows[i, 0:d] of batch row_b[i], head row_h[i]; it attends key positions
// 0 .. row_nkeys[i]-1 of kv_latent[row_b[i]] (row_nkeys = t + 1 for prefill
// position t, = L_b for decode).  out[i, :] receives the attention output;
// probs (optional, stride pstride >= max nkeys) the softmax weights.
int oracle_attend_rows_masked(const void* q_rows, int dt_q, long n,
                              const long* row_b, const long* row_h, const long* row_nkeys,
                              const void* kv_latent, int dt_lat, long B, long Tlat,
                              const void* w_up_k, const void* w_up_v, int dt_w,
                              long H, long d, long r, double scale, const uint8_t* key_mask,
                              double* out, double* probs, long pstride, int nthreads) {
  if (n < 0 || B < 1 || Tlat < 1 || H < 1 || d < 1 || r < 1) return 1;
  if (n == 0) return 0;
  if (!q_rows || !row_b || !row_h || !row_nkeys || !kv_latent || !w_up_k || !w_up_v || !out) return 1;
  for (long i = 0; i < n; ++i) {
    if (row_b[i] < 0 || row_b[i] >= B || row_h[i] < 0 || row_h[i] >= H) return 1;
    if (row_nkeys[i] < 1 || row_nkeys[i] > Tlat) return 1;
    if (probs && row_nkeys[i] > pstride) return 1;
  }
  Problem P{q_rows, dt_q, kv_latent, dt_lat, w_up_k, w_up_v, dt_w, Tlat, H, d, r, scale,
            row_b, row_h, row_nkeys, out, probs, pstride, key_mask};
  // group rows by (b, h): each group materialises its k and v once
  std::vector<long> order(n);
  for (long i = 0; i < n; ++i) order[i] = i;
  std::sort(order.begin(), order.end(), [&](long a, long c) {
    if (row_b[a] != row_b[c]) return row_b[a] < row_b[c];
    if (row_h[a] != row_h[c]) return row_h[a] < row_h[c];
    return a < c;
  });
  std::vector<std::vector<long>> groups;
  for (long i : order) {
    if (groups.empty() || row_b[groups.back()[0]] != row_b[i] || row_h[groups.back()[0]] != row_h[i])
      groups.emplace_back();
    groups.back().push_back(i);
  }
  std::atomic<size_t> next{0};
  auto worker = [&]() {
    for (size_t g; (g = next.fetch_add(1)) < groups.size();) attend_group(P, groups[g]);
  };
  const int nt = std::min<int>(nthreads_or_default(nthreads), (int)groups.size());
  std::vector<std::thread> pool;
  for (int t = 1; t < nt; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  return 0;
}

int oracle_attend_rows(const void* q_rows, int dt_q, long n,
                       const long* row_b, const long* row_h, const long* row_nkeys,
                       const void* kv_latent, int dt_lat, long B, long Tlat,
                       const void* w_up_k, const void* w_up_v, int dt_w,
                       long H, long d, long r, double scale,
                       double* out, double* probs, long pstride, int nthreads) {
  return oracle_attend_rows_masked(q_rows, dt_q, n, row_b, row_h, row_nkeys, kv_latent, dt_lat, B, Tlat, w_up_k,
                                   w_up_v, dt_w, H, d, r, scale, nullptr, out, probs, pstride, nthreads);
}

// Full causal prefill with a key mask (key_mask [B, T] bytes, 0 = masked;
// nullptr = none): out[b, t, h, :] for every b < B, t < T, h < H.
int oracle_latent_attn_masked(const void* q, int dt_q, const void* kv_latent, int dt_lat,
                              const void* w_up_k, const void* w_up_v, int dt_w,
                              long B, long T, long H, long d, long r, double scale,
                              const uint8_t* key_mask, double* out, int nthreads) {
  if (B < 1 || T < 1 || H < 1) return 1;
  const long n = B * T * H;
  std::vector<long> rb(n), rh(n), rk(n);
  for (long b = 0; b < B; ++b)
    for (long t = 0; t < T; ++t)
      for (long h = 0; h < H; ++h) {
        const long i = (b * T + t) * H + h;
        rb[i] = b; rh[i] = h; rk[i] = t + 1;
      }
  return oracle_attend_rows_masked(q, dt_q, n, rb.data(), rh.data(), rk.data(), kv_latent, dt_lat, B, T,
                                   w_up_k, w_up_v, dt_w, H, d, r, scale, key_mask, out, nullptr, 0, nthreads);
}

// Full causal prefill: out[b, t, h, :] for every b < B, t < T, h < H.
// q [B, T, H, d]; kv_latent [B, T, r].
int oracle_latent_attn(const void* q, int dt_q, const void* kv_latent, int dt_lat,
                       const void* w_up_k, const void* w_up_v, int dt_w,
                       long B, long T, long H, long d, long r, double scale,
                       double* out, int nthreads) {
  if (B < 1 || T < 1 || H < 1) return 1;
  const long n = B * T * H;
  std::vector<long> rb(n), rh(n), rk(n);
  for (long b = 0; b < B; ++b)
    for (long t = 0; t < T; ++t)
      for (long h = 0; h < H; ++h) {
        const long i = (b * T + t) * H + h;  // q and out rows are [B, T, H] in this order
        rb[i] = b; rh[i] = h; rk[i] = t + 1;
      }
  return oracle_attend_rows(q, dt_q, n, rb.data(), rh.data(), rk.data(), kv_latent, dt_lat, B, T,
                            w_up_k, w_up_v, dt_w, H, d, r, scale, out, nullptr, 0, nthreads);
}

// Decode: q [B, H, d] (one token per sequence), kv_latent [B, Tmax, r] with
// seq_lens[b] valid rows; out [B, H, d].
int oracle_decode(const void* q, int dt_q, const void* kv_latent, int dt_lat,
                  const int32_t* seq_lens, const void* w_up_k, const void* w_up_v, int dt_w,
                  long B, long Tmax, long H, long d, long r, double scale,
                  double* out, int nthreads) {
  if (!seq_lens || B < 1 || H < 1) return 1;
  const long n = B * H;
  std::vector<long> rb(n), rh(n), rk(n);
  for (long b = 0; b < B; ++b)
    for (long h = 0; h < H; ++h) {
      rb[b * H + h] = b; rh[b * H + h] = h; rk[b * H + h] = seq_lens[b];
    }
  return oracle_attend_rows(q, dt_q, n, rb.data(), rh.data(), rk.data(), kv_latent, dt_lat, B, Tmax,
                            w_up_k, w_up_v, dt_w, H, d, r, scale, out, nullptr, 0, nthreads);
}

}  // extern "C"
