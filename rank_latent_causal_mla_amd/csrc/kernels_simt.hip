// Vector-ALU kernels of the float32 path (also used for bf16 storage when a
// shape falls outside the matrix-core kernels' tiles): every product and sum
// in float32.  Same absorbed formulation as the matrix-core path (absorb,
// streaming-softmax attention over the latents, up-projection), plus the KV
// down-projection GEMM of POPCORNBENCH page FW-GLM-5-1 l2_p1 (latent =
// hidden @ w_down).
#include "mla_device.h"
#include "mla_kernels.h"
#include "profile.h"

namespace mla {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// q_lat[row, rho] = sum_e q[row, e] * W_uk[rho, h, e], row = n*H + h.  One block per row.
template <typename T>
__global__ void absorb_simt(const T* __restrict__ q, const T* __restrict__ wk,
                            float* __restrict__ q_lat, int H, int d, int R) {
  __shared__ float qs[256];
  const size_t row = blockIdx.x;
  const int h = (int)(row % H);
  for (int e = threadIdx.x; e < d; e += blockDim.x) qs[e] = io<T>::ld(q, row * d + e);
  __syncthreads();
  for (int rho = threadIdx.x; rho < R; rho += blockDim.x) {
    const T* w = wk + ((size_t)rho * H + h) * d;
    float acc = 0.f;
    for (int e = 0; e < d; ++e) acc += qs[e] * io<T>::ld(w, e);
    q_lat[row * R + rho] = acc;
  }
}

// Streaming-softmax attention of one query row per wave over the latents.
// Prefill: row = (b*T + t)*H + h attends keys 0..t of batch b; with kmask
//          [B, T] bytes, only the keys s whose kmask[b, s] is nonzero (a masked
//          logit is -infinity; a row with no visible key gives 0 / 0 = NaN).
// Decode:  row = b*H + h attends keys 0..L_b-1 (L_b = seq_lens[b] clamped to [1, Tl]) of a
//          padded cache [B, Tl, R]; with cu, the rows cu[b] .. cu[b+1]-1 of a packed cache
//          [Tl, R] (clamped into the cache, as the matrix-core path does).
template <typename T, bool DECODE>
__global__ void attend_simt(const float* __restrict__ q_lat, const T* __restrict__ lat,
                            const int32_t* __restrict__ lens, const int32_t* __restrict__ cu,
                            const uint8_t* __restrict__ kmask, float* __restrict__ o_lat, int Tl, int H,
                            int R, float sl2, long nrows) {
  __shared__ float qs[4][1024];
  __shared__ float ps[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + w;
  if (row >= nrows) return;  // whole wave; no block-level barrier below
  long b;
  int nkeys;
  size_t base;  // first cache row of the sequence
  if (DECODE && cu) {
    b = row / H;
    const int c0 = cu[b], c1 = cu[b + 1];
    const int rb = c0 < 0 ? 0 : (c0 > Tl - 1 ? Tl - 1 : c0);
    const int L = c1 - c0, Lmax = Tl - rb;
    nkeys = L < 1 ? 1 : (L > Lmax ? Lmax : L);
    base = (size_t)rb;
  } else if (DECODE) {
    b = row / H;
    int L = lens[b];
    nkeys = L < 1 ? 1 : (L > Tl ? Tl : L);
    base = (size_t)b * Tl;
  } else {
    b = row / ((long)Tl * H);
    nkeys = (int)((row / H) % Tl) + 1;
    base = (size_t)b * Tl;
  }
  for (int rho = lane; rho < R; rho += 64) qs[w][rho] = q_lat[row * R + rho];
  __builtin_amdgcn_wave_barrier();
  float o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const T* latb = lat + base * R;
  for (int s0 = 0; s0 < nkeys; s0 += 64) {
    const int s = s0 + lane;
    float x = -INFINITY;
    if (s < nkeys && (DECODE || !kmask || kmask[base + s])) {
      const T* lr = latb + (size_t)s * R;
      float dot = 0.f;
      for (int rho = 0; rho < R; ++rho) dot += qs[w][rho] * io<T>::ld(lr, rho);
      x = dot * sl2;
    }
    const float mn = fmaxf(m, wave_max(x));
    // no visible key yet: mn = -inf, subtract 0 so the weights are exact zeros
    const float msub = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(m - msub);
    const float p = exp2f(x - msub);
    l = l * alpha + wave_sum(p);
    m = mn;
    ps[w][lane] = p;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] *= alpha;
    const int nj = nkeys - s0 < 64 ? nkeys - s0 : 64;
    for (int j = 0; j < nj; ++j) {
      const float pj = ps[w][j];
      const T* lr = latb + (size_t)(s0 + j) * R;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rho = lane + 64 * i;
        if (rho < R) o[i] += pj * io<T>::ld(lr, rho);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rho = lane + 64 * i;
    if (rho < R) o_lat[row * R + rho] = o[i] * inv;
  }
}

// out[row, e] = sum_rho o_lat[row, rho] * W_uv[rho, h, e].  One block per row.
template <typename T>
__global__ void up_simt(const float* __restrict__ o_lat, const T* __restrict__ wv,
                        T* __restrict__ out, int H, int d, int R) {
  __shared__ float os[1024];
  const size_t row = blockIdx.x;
  const int h = (int)(row % H);
  for (int rho = threadIdx.x; rho < R; rho += blockDim.x) os[rho] = o_lat[row * R + rho];
  __syncthreads();
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float acc = 0.f;
    for (int rho = 0; rho < R; ++rho) acc += os[rho] * io<T>::ld(wv, ((size_t)rho * H + h) * d + e);
    io<T>::st(out, row * d + e, acc);
  }
}

// C[M, N] = A[M, K] B[K, N], row-major, float32 accumulation; 64x64 tiles,
// 16x16 threads with 4x4 outputs each, K staged through LDS 16 at a time.
template <typename T>
__global__ void gemm_simt(const T* __restrict__ A, const T* __restrict__ Bm, T* __restrict__ C,
                          int M, int K, int N) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int row0 = blockIdx.y * 64, col0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, k = idx & 15;
      As[k][r] = (row0 + r < M && k0 + k < K) ? io<T>::ld(A, (size_t)(row0 + r) * K + k0 + k) : 0.f;
      const int kb = idx >> 6, c = idx & 63;
      Bs[kb][c] = (k0 + kb < K && col0 + c < N) ? io<T>::ld(Bm, (size_t)(k0 + kb) * N + col0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * bb[j];
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + ty + 16 * i, c = col0 + tx + 16 * j;
      if (r < M && c < N) io<T>::st(C, (size_t)r * N + c, acc[i][j]);
    }
}

template <typename T>
static hipError_t prefill_simt_t(const T* q, const T* lat, const T* wk, const T* wv, T* out, int B,
                                 int T_, int H, int d, int r, float sl2, const uint8_t* kmask, void* ws,
                                 hipStream_t st) {
  const long rows = (long)B * T_ * H;
  float* q_lat = (float*)ws;
  float* o_lat = q_lat + (size_t)rows * r;
  {
    ProfScope ps("absorb_simt", st);
    hipLaunchKernelGGL(absorb_simt<T>, dim3(rows), dim3(256), 0, st, q, wk, q_lat, H, d, r);
  }
  {
    ProfScope ps("attend_simt", st);
    hipLaunchKernelGGL((attend_simt<T, false>), dim3((rows + 3) / 4), dim3(256), 0, st, q_lat, lat, nullptr,
                       (const int32_t*)nullptr, kmask, o_lat, T_, H, r, sl2, rows);
  }
  {
    ProfScope ps("up_simt", st);
    hipLaunchKernelGGL(up_simt<T>, dim3(rows), dim3(256), 0, st, o_lat, wv, out, H, d, r);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t decode_simt_t(const T* q, const T* lat, const int32_t* lens, const int32_t* cu, const T* wk,
                                const T* wv, T* out, int B, int Tmax, int H, int d, int r,
                                float sl2, void* ws, hipStream_t st) {
  const long rows = (long)B * H;
  float* q_lat = (float*)ws;
  float* o_lat = q_lat + (size_t)rows * r;
  {
    ProfScope ps("absorb_simt", st);
    hipLaunchKernelGGL(absorb_simt<T>, dim3(rows), dim3(256), 0, st, q, wk, q_lat, H, d, r);
  }
  {
    ProfScope ps("attend_simt", st);
    hipLaunchKernelGGL((attend_simt<T, true>), dim3((rows + 3) / 4), dim3(256), 0, st, q_lat, lat,
                       lens, cu, (const uint8_t*)nullptr, o_lat, Tmax, H, r, sl2, rows);
  }
  {
    ProfScope ps("up_simt", st);
    hipLaunchKernelGGL(up_simt<T>, dim3(rows), dim3(256), 0, st, o_lat, wv, out, H, d, r);
  }
  return hipGetLastError();
}

static constexpr float kLog2e = 1.4426950408889634f;

hipError_t prefill_simt(bool bf16, const void* q, const void* lat, const void* wk, const void* wv,
                        void* out, int B, int T, int H, int d, int r, float scale, const uint8_t* key_mask,
                        void* ws, hipStream_t st) {
  const float sl2 = scale * kLog2e;
  if (bf16)
    return prefill_simt_t((const uint16_t*)q, (const uint16_t*)lat, (const uint16_t*)wk,
                          (const uint16_t*)wv, (uint16_t*)out, B, T, H, d, r, sl2, key_mask, ws, st);
  return prefill_simt_t((const float*)q, (const float*)lat, (const float*)wk, (const float*)wv,
                        (float*)out, B, T, H, d, r, sl2, key_mask, ws, st);
}

size_t prefill_simt_workspace(int B, int T, int H, int d, int r) {
  (void)d;
  return (size_t)2 * B * T * H * r * sizeof(float);
}

hipError_t decode_simt(bool bf16, const void* q, const void* lat, const int32_t* lens, const int32_t* cu,
                       const void* wk, const void* wv, void* out, int B, int Tmax, int H, int d,
                       int r, float scale, void* ws, hipStream_t st) {
  const float sl2 = scale * kLog2e;
  if (bf16)
    return decode_simt_t((const uint16_t*)q, (const uint16_t*)lat, lens, cu, (const uint16_t*)wk,
                         (const uint16_t*)wv, (uint16_t*)out, B, Tmax, H, d, r, sl2, ws, st);
  return decode_simt_t((const float*)q, (const float*)lat, lens, cu, (const float*)wk,
                       (const float*)wv, (float*)out, B, Tmax, H, d, r, sl2, ws, st);
}

// One block per sequence: row lens[b] of kv_cache[b] takes new_latent[b], then
// lens[b] grows by one; a sequence whose cache is full (or whose length is
// outside [0, Tmax)) is left unchanged.
template <typename T>
__global__ void kv_append_kernel(T* __restrict__ kv_cache, int32_t* __restrict__ lens,
                                 const T* __restrict__ new_latent, int Tmax, int r) {
  __shared__ int pos;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) pos = lens[b];
  __syncthreads();
  const int p = pos;
  if (p < 0 || p >= Tmax) return;  // whole block
  T* dst = kv_cache + ((size_t)b * Tmax + p) * r;
  const T* src = new_latent + (size_t)b * r;
  for (int i = threadIdx.x; i < r; i += blockDim.x) dst[i] = src[i];
  if (threadIdx.x == 0) lens[b] = p + 1;
}

hipError_t kv_append(bool bf16, void* kv_cache, int32_t* lens, const void* new_latent, int B, int Tmax, int r,
                     hipStream_t st) {
  ProfScope ps("kv_append", st);
  if (bf16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(B), dim3(256), 0, st, (uint16_t*)kv_cache, lens,
                       (const uint16_t*)new_latent, Tmax, r);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(B), dim3(256), 0, st, (float*)kv_cache, lens,
                       (const float*)new_latent, Tmax, r);
  return hipGetLastError();
}

size_t decode_simt_workspace(int B, int Tmax, int H, int d, int r) {
  (void)Tmax;
  (void)d;
  return (size_t)2 * B * H * r * sizeof(float);
}

hipError_t down_proj(bool bf16, const void* hidden, const void* w_down, void* latent, int M, int D,
                     int r, hipStream_t st) {
  const dim3 grid((r + 63) / 64, (M + 63) / 64);
  if (bf16)
    {
      ProfScope ps("gemm_simt", st);
      hipLaunchKernelGGL(gemm_simt<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)hidden,
                         (const uint16_t*)w_down, (uint16_t*)latent, M, D, r);
    }
  else
    {
      ProfScope ps("gemm_simt", st);
      hipLaunchKernelGGL(gemm_simt<float>, grid, dim3(256), 0, st, (const float*)hidden,
                         (const float*)w_down, (float*)latent, M, D, r);
    }
  return hipGetLastError();
}

}  // namespace mla
