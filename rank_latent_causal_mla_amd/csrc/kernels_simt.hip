// Vector-ALU kernels of the float32 path (also used for bf16 storage when a
// shape falls outside the matrix-core kernels' tiles): every product and sum
// in float32.  Same absorbed formulation as the matrix-core path (absorb,
// streaming-softmax attention over the latents, up-projection), plus the KV
// down-projection GEMM of POPCORNBENCH page FW-GLM-5-1 l2_p1 (latent =
// hidden @ w_down).
#include "mla_device.h"
#include "mla_kernels.h"
#include "host_once.h"
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
    // a row with no visible key (l = 0, key mask) is NaN, written as such
    // (chosen in the integer domain, so no float rule can drop it)
    if (rho < R) o_lat[row * R + rho] = __uint_as_float(l > 0.f ? __float_as_uint(o[i] * inv) : 0x7fc00000u);
  }
}

// Causal prefill attention over the latents, float32, tiled: one block per
// 64 consecutive rows (t*H + h) of a batch and 64-key tiles, both staged in
// LDS and shared by the block.  Thread (rg, cg) = (tid / 16, tid % 16) owns
// rows rg + 16 i (i = 0..3): for the scores, keys cg + 16 j of the tile
// (j = 0..3); for the output, latent columns 4 (cg + 16 c) .. + 3
// (c < R / 64).  The 16 threads of a row group hold the same running max and
// sum (reduced over the group by shuffles), so the online rescale needs no
// exchange; the probabilities go through LDS to the output product.  Rows
// are padded to R + 4 floats: consecutive rows start in consecutive 16-byte
// bank groups.  R in {64, 128, 256}.
constexpr int kF32Rows = 64, kF32Keys = 64;
template <int R>
constexpr size_t attend_f32_lds_bytes() { return (size_t)(2 * 64 * (R + 4) + 64 * (kF32Keys + 4)) * 4; }

template <typename T>
__device__ __forceinline__ float4 ld4(const T* p);
template <>
__device__ __forceinline__ float4 ld4<float>(const float* p) { return *(const float4*)p; }
template <>
__device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const u32x2 v = *(const u32x2*)p;
  return float4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
                __uint_as_float(v[1] & 0xFFFF0000u)};
}

template <int R, typename T>
__global__ __launch_bounds__(256) void attend_f32_tiled(const float* __restrict__ q_lat, const T* __restrict__ lat,
                                                        float* __restrict__ o_lat, int Tn, int H, float sl2) {
  constexpr int QS = R + 4;        // row stride (floats) of the q and latent tiles
  constexpr int PS = kF32Keys + 4; // row stride of the probabilities
  constexpr int NC = R / 64;       // 4-column chunks per thread in the output
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* qs = sm;
  float* ls = qs + kF32Rows * QS;
  float* ps = ls + kF32Keys * QS;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int b = blockIdx.y;
  const long TH = (long)Tn * H;
  const long row0 = (long)blockIdx.x * kF32Rows;
  for (int idx = tid; idx < kF32Rows * (R / 4); idx += 256) {
    const int r = idx / (R / 4), c = idx % (R / 4);
    const long row = row0 + r < TH ? row0 + r : TH - 1;
    *(float4*)&qs[r * QS + 4 * c] = *(const float4*)&q_lat[((size_t)b * TH + row) * R + 4 * c];
  }
  const long last = row0 + kF32Rows - 1 < TH - 1 ? row0 + kF32Rows - 1 : TH - 1;
  const int ntiles = (int)(last / H) / kF32Keys + 1;
  int trow[4];
  float m[4], l[4];
  float4 o[4][NC];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long row = row0 + rg + 16 * i < TH ? row0 + rg + 16 * i : TH - 1;
    trow[i] = (int)(row / H);
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[i][c] = float4{0.f, 0.f, 0.f, 0.f};
  }
  const T* latb = lat + (size_t)b * Tn * R;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * kF32Keys;
    __syncthreads();  // the previous tile's products are done with ls and ps
    for (int idx = tid; idx < kF32Keys * (R / 4); idx += 256) {
      const int k = idx / (R / 4), c = idx % (R / 4);
      const int s = k0 + k < Tn ? k0 + k : Tn - 1;
      *(float4*)&ls[k * QS + 4 * c] = ld4<T>(latb + (size_t)s * R + 4 * c);
    }
    __syncthreads();
    float sc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[i][j] = 0.f;
#pragma unroll 4
    for (int rho = 0; rho < R; rho += 4) {
      float4 qv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = *(const float4*)&qs[(rg + 16 * i) * QS + rho];
#pragma unroll
      for (int j = 0; j < 4; ++j) lv[j] = *(const float4*)&ls[(cg + 16 * j) * QS + rho];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sc[i][j] += qv[i].x * lv[j].x + qv[i].y * lv[j].y + qv[i].z * lv[j].z + qv[i].w * lv[j].w;
    }
    // causal mask, then the online update of each row (keys s <= t only)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x[4], mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = k0 + cg + 16 * j <= trow[i] ? sc[i][j] * sl2 : -INFINITY;
        mx = fmaxf(mx, x[j]);
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(m[i], mx);
      const float msub = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m[i] - msub);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(x[j] - msub);
        sum += p;
        ps[(rg + 16 * i) * PS + cg + 16 * j] = p;
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      l[i] = l[i] * alpha + sum;
      m[i] = mn;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        o[i][c].x *= alpha;
        o[i][c].y *= alpha;
        o[i][c].z *= alpha;
        o[i][c].w *= alpha;
      }
    }
    __syncthreads();  // the probabilities of every row are in ps
    const int kn = Tn - k0 < kF32Keys ? Tn - k0 : kF32Keys;
    for (int k = 0; k < kn; ++k) {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = ps[(rg + 16 * i) * PS + k];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 lv = *(const float4*)&ls[k * QS + 4 * (cg + 16 * c)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i][c].x += pv[i] * lv.x;
          o[i][c].y += pv[i] * lv.y;
          o[i][c].z += pv[i] * lv.z;
          o[i][c].w += pv[i] * lv.w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long row = row0 + rg + 16 * i;
    if (row >= TH) continue;
    const float inv = 1.f / l[i];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *(float4*)&o_lat[((size_t)b * TH + row) * R + 4 * (cg + 16 * c)] =
          float4{o[i][c].x * inv, o[i][c].y * inv, o[i][c].z * inv, o[i][c].w * inv};
  }
}

template <int R, typename T>
static hipError_t attend_f32_tiled_launch(const float* q_lat, const T* lat, float* o_lat, int B, int Tn, int H,
                                          float sl2, hipStream_t st) {
  static OnceFlag attrs;
  const hipError_t e = run_once(attrs, [] {
    return hipFuncSetAttribute((const void*)attend_f32_tiled<R, T>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)attend_f32_lds_bytes<R>());
  });
  if (e != hipSuccess) return e;
  const long TH = (long)Tn * H;
  hipLaunchKernelGGL((attend_f32_tiled<R, T>), dim3((unsigned)((TH + kF32Rows - 1) / kF32Rows), B), dim3(256),
                     attend_f32_lds_bytes<R>(), st, q_lat, lat, o_lat, Tn, H, sl2);
  return hipGetLastError();
}

// Strided batched GEMM in float32: for batch z (blockIdx.z),
//   C[m*ldc + n] = sum_k A[m*lda + k] * B[k*ldbk + n*ldbn]
// with A, B, C offset by z*a_bs, z*b_bs, z*c_bs elements.  Tiles of 16 TS x
// 16 TS, 16x16 threads with TS x TS outputs each, k staged through LDS 16
// at a time; B is read along k when ldbk == 1 (k contiguous), else along n.
// TS = 4 (64x64 tiles) or 2 (32x32) when 64x64 tiles would leave compute
// units idle.
template <typename TA, typename TB, typename TC, int TS>
__global__ __launch_bounds__(256) void gemm_strided(const TA* __restrict__ A, const TB* __restrict__ Bm,
                                                    TC* __restrict__ C, int M, int K, int N, long lda, long ldbk,
                                                    long ldbn, long ldc, long a_bs, long b_bs, long c_bs) {
  constexpr int TW = 16 * TS;  // tile width
  __shared__ float As[16][TW + 1];
  __shared__ float Bs[16][TW + 1];
  A += blockIdx.z * a_bs;
  Bm += blockIdx.z * b_bs;
  C += blockIdx.z * c_bs;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int row0 = blockIdx.y * TW, col0 = blockIdx.x * TW;
  const bool bk = ldbk == 1;
  float acc[TS][TS] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = 0; i < 16 * TW / 256; ++i) {  // both 16 x TW tiles, 256 elements at a time
      const int idx = tid + 256 * i;
      const int r = idx >> 4, k = idx & 15;
      As[k][r] = (row0 + r < M && k0 + k < K) ? io<TA>::ld(A, (size_t)(row0 + r) * lda + k0 + k) : 0.f;
      const int kb = bk ? idx & 15 : idx / TW, c = bk ? idx >> 4 : idx % TW;
      Bs[kb][c] = (k0 + kb < K && col0 + c < N) ? io<TB>::ld(Bm, (size_t)(k0 + kb) * ldbk + (size_t)(col0 + c) * ldbn)
                                                  : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[TS], bb[TS];
#pragma unroll
      for (int i = 0; i < TS; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < TS; ++j) bb[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TS; ++j) acc[i][j] += a[i] * bb[j];
    }
    __syncthreads();
  }
  for (int i = 0; i < TS; ++i)
    for (int j = 0; j < TS; ++j) {
      const int r = row0 + ty + 16 * i, c = col0 + tx + 16 * j;
      if (r < M && c < N) io<TC>::st(C, (size_t)r * ldc + c, acc[i][j]);
    }
}

template <typename TA, typename TB, typename TC>
static hipError_t gemm_launch(const TA* A, const TB* Bm, TC* C, int M, int K, int N, long lda, long ldbk, long ldbn,
                              long ldc, int batches, long a_bs, long b_bs, long c_bs, hipStream_t st) {
  const long tiles64 = (long)((N + 63) / 64) * ((M + 63) / 64) * batches;
  if (tiles64 < 512) {  // 64x64 tiles would not fill the chip
    hipLaunchKernelGGL((gemm_strided<TA, TB, TC, 2>), dim3((N + 31) / 32, (M + 31) / 32, batches), dim3(256), 0, st,
                       A, Bm, C, M, K, N, lda, ldbk, ldbn, ldc, a_bs, b_bs, c_bs);
  } else {
    hipLaunchKernelGGL((gemm_strided<TA, TB, TC, 4>), dim3((N + 63) / 64, (M + 63) / 64, batches), dim3(256), 0, st,
                       A, Bm, C, M, K, N, lda, ldbk, ldbn, ldc, a_bs, b_bs, c_bs);
  }
  return hipGetLastError();
}

// Absorption, every head at once: q_lat[n, h, rho] = sum_e q[n, h, e] W_uk[rho, h, e]
// (n < Ntok; q_lat float32 [Ntok][H][R]).
template <typename T>
static hipError_t absorb_gemm(const T* q, const T* wk, float* q_lat, long Ntok, int H, int d, int R, hipStream_t st) {
  ProfScope ps("absorb_f32", st);
  return gemm_launch<T, T, float>(q, wk, q_lat, (int)Ntok, d, R, (long)H * d, 1, (long)H * d, (long)H * R, H, d, d,
                                  R, st);
}

// Up-projection, every head at once: out[n, h, e] = sum_rho o_lat[n, h, rho] W_uv[rho, h, e].
template <typename T>
static hipError_t up_gemm(const float* o_lat, const T* wv, T* out, long Ntok, int H, int d, int R, hipStream_t st) {
  ProfScope ps("up_f32", st);
  return gemm_launch<float, T, T>(o_lat, wv, out, (int)Ntok, R, d, (long)H * R, (long)H * d, 1, (long)H * d, H, R, d,
                                  d, st);
}

template <typename T>
static hipError_t prefill_simt_t(const T* q, const T* lat, const T* wk, const T* wv, T* out, int B,
                                 int T_, int H, int d, int r, float sl2, const uint8_t* kmask, void* ws,
                                 hipStream_t st) {
  const long rows = (long)B * T_ * H;
  float* q_lat = (float*)ws;
  float* o_lat = q_lat + (size_t)rows * r;
  {
    hipError_t e = absorb_gemm<T>(q, wk, q_lat, rows / H, H, d, r, st);
    if (e != hipSuccess) return e;
  }
  if (!kmask && (r == 64 || r == 128 || r == 256)) {
    ProfScope ps("attend_f32_tiled", st);
    hipError_t e = r == 64    ? attend_f32_tiled_launch<64, T>(q_lat, lat, o_lat, B, T_, H, sl2, st)
                   : r == 128 ? attend_f32_tiled_launch<128, T>(q_lat, lat, o_lat, B, T_, H, sl2, st)
                              : attend_f32_tiled_launch<256, T>(q_lat, lat, o_lat, B, T_, H, sl2, st);
    if (e != hipSuccess) return e;
  } else {
    ProfScope ps("attend_simt", st);
    hipLaunchKernelGGL((attend_simt<T, false>), dim3((rows + 3) / 4), dim3(256), 0, st, q_lat, lat, nullptr,
                       (const int32_t*)nullptr, kmask, o_lat, T_, H, r, sl2, rows);
  }
  {
    hipError_t e = up_gemm<T>(o_lat, wv, out, rows / H, H, d, r, st);
    if (e != hipSuccess) return e;
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
    hipError_t e = absorb_gemm<T>(q, wk, q_lat, rows / H, H, d, r, st);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("attend_simt", st);
    hipLaunchKernelGGL((attend_simt<T, true>), dim3((rows + 3) / 4), dim3(256), 0, st, q_lat, lat,
                       lens, cu, (const uint8_t*)nullptr, o_lat, Tmax, H, r, sl2, rows);
  }
  {
    hipError_t e = up_gemm<T>(o_lat, wv, out, rows / H, H, d, r, st);
    if (e != hipSuccess) return e;
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
  ProfScope ps("down_f32", st);
  if (bf16)
    return gemm_launch<uint16_t, uint16_t, uint16_t>((const uint16_t*)hidden, (const uint16_t*)w_down,
                                                     (uint16_t*)latent, M, D, r, D, r, 1, r, 1, 0, 0, 0, st);
  return gemm_launch<float, float, float>((const float*)hidden, (const float*)w_down, (float*)latent, M, D, r, D, r,
                                          1, r, 1, 0, 0, 0, st);
}

}  // namespace mla
