// gfx950 matrix-core kernels of the bf16 prefill path: weight absorption, the
// fused causal latent flash kernel and the per-head up-projection (the decode
// kernels are in kernels_decode.hip).
//
// The attention they compute is the latent causal attention of POPCORNBENCH
// page FW-GLM-5-1 l2_p31 (algorithm restatement), rewritten by bilinearity:
//   <q, latent_s W_uk[:,h]> = <W_uk[:,h] q, latent_s>  and
//   sum_s p_s latent_s W_uv[:,h] = (sum_s p_s latent_s) W_uv[:,h],
// so every head attends the shared r-wide latents directly (K = V = latent)
// with an r-wide query q_lat = W_uk[:,h] q, and the d-wide output is o_lat
// up-projected by W_uv[:,h].  The softmax is the streaming (online) form:
// a running max m, running sum l and running output rescaled by
// exp(m_old - m_new) whenever the max grows -- exact up to rounding.
#include "mla_device.h"
#include "mla_kernels.h"
#include "prep_blocks.h"
#include "profile.h"

namespace mla {

// ---------------------------------------------------------------------------
// Absorption (one block per 32 query rows of one head, the whole rank) and
// the W_uv transpose, as kernels around the block bodies of prep_blocks.h.
template <int R, int DK>
__global__ __launch_bounds__(256) void absorb_bf16(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ wk,
                                                   uint16_t* __restrict__ q_lat, int N, int H,
                                                   float qscale) {
  absorb_tile<R, DK, R / 128>(q, wk, q_lat, N, H, qscale, blockIdx.x, blockIdx.y, 0);
}

__global__ __launch_bounds__(256) void transpose_wv(const uint16_t* __restrict__ wv, uint16_t* __restrict__ wvT,
                                                    int R, int H, int d) {
  transpose_wv_tile(wv, wvT, R, H, d, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int R>
static hipError_t absorb_launch(const uint16_t* q, const uint16_t* wk, uint16_t* q_lat, int N, int H,
                                int d, float qscale, hipStream_t st) {
  const dim3 grid((N + 31) / 32, H);
  switch (d) {
    case 32: hipLaunchKernelGGL((absorb_bf16<R, 2>), grid, dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 64: hipLaunchKernelGGL((absorb_bf16<R, 4>), grid, dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 128: hipLaunchKernelGGL((absorb_bf16<R, 8>), grid, dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 256: hipLaunchKernelGGL((absorb_bf16<R, 16>), grid, dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t absorb_mfma(const uint16_t* q, const uint16_t* wk, uint16_t* q_lat, int N, int H, int d,
                       int R, float qscale, hipStream_t st) {
  ProfScope ps("absorb_bf16", st);
  switch (R) {
    case 128: return absorb_launch<128>(q, wk, q_lat, N, H, d, qscale, st);
    case 256: return absorb_launch<256>(q, wk, q_lat, N, H, d, qscale, st);
    case 512: return absorb_launch<512>(q, wk, q_lat, N, H, d, qscale, st);
  }
  return hipErrorInvalidValue;
}

hipError_t transpose_wv_launch(const uint16_t* wv, uint16_t* wvT, int R, int H, int d, hipStream_t st) {
  hipLaunchKernelGGL(transpose_wv, dim3((R + 31) / 32, (d + 31) / 32, H), dim3(256), 0, st, wv, wvT, R, H, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Up-projection: out[n, h, e] = sum_rho o_lat[n*H + h, rho] * W_uv[rho, h, e],
// computed as out^T = W_uv^T o_lat^T.  Block: 4 waves x 32 tokens of one head.
template <int R>
__global__ __launch_bounds__(256) void up_bf16(const uint16_t* __restrict__ o_lat,
                                               const uint16_t* __restrict__ wvT,
                                               uint16_t* __restrict__ out, int N, int H, int d) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int n = blockIdx.x * 128 + w * 32 + l32;
  if (blockIdx.x * 128 + w * 32 >= N) return;
  const int nc = min(n, N - 1);
  const int neb = d / 32;
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  const uint16_t* orow = o_lat + ((size_t)nc * H + h) * R + 8 * g;
  const uint16_t* wrow = wvT + ((size_t)h * d + l32) * R + 8 * g;
  for (int ks = 0; ks < R / 16; ++ks) {
    const bf16x8 bo = *(const bf16x8*)(orow + 16 * ks);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < neb) {
        const bf16x8 a = *(const bf16x8*)(wrow + (size_t)32 * i * R + 16 * ks);
        acc[i] = mfma32x32x16(a, bo, acc[i]);
      }
  }
  if (n >= N) return;
  uint16_t* dst = out + ((size_t)n * H + h) * d;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < neb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 32 * i + 8 * j + 4 * g;
        u32x2 v = {pack_bf16x2(acc[i][4 * j], acc[i][4 * j + 1]),
                   pack_bf16x2(acc[i][4 * j + 2], acc[i][4 * j + 3])};
        *(u32x2*)(dst + e) = v;
      }
}

// ---------------------------------------------------------------------------
// Causal latent flash attention, prefill.
//
// The two products need the latent tile in two orientations: the scores
// contract over rho (rows of L, rho-contiguous) and P * L contracts over keys
// (columns of L).  Transposing in LDS (ds_read_b64_tr_b16) is far slower than
// plain 16-byte reads, so the tile also comes pre-transposed from a per-call
// copy of the latents, latT [B][ceil(T/32)][R][32] (latent_transpose below),
// whose 32 keys per row are stored in the order the P operand holds them.
// Both orientations are copied into LDS by LDS-DMA and read with ds_read_b128.

// Transposed tiles.  The P operand built from the score accumulators gives
// lane group G (lanes 16 G .. 16 G + 15) the keys {4 G + u, 16 + 4 G + u},
// u = 0..3, as its 8 k-slots.  The transposed copy of a 32-key tile is
// therefore stored group-major, [G][rho][8]: entry u of (G, rho) holds
// latent[key(G, u)][rho] with key(G, u) = 16 (u / 4) + 4 G + u % 4, so each
// lane reads its A operand as one contiguous 16-byte chunk and the 16 lanes
// of a group read 256 contiguous bytes.
__device__ __forceinline__ int tkey(int G, int u) { return 16 * (u >> 2) + 4 * G + (u & 3); }

// lat [B][T][R] -> latT [B][nt][4][R][8], nt = ceil(T / 32); keys >= T are zero.
template <int R>
__global__ __launch_bounds__(256) void latent_transpose(const uint16_t* __restrict__ lat,
                                                        uint16_t* __restrict__ latT, int T, int nt) {
  __shared__ __attribute__((aligned(16))) uint16_t s[32][R + 8];
  const int tile = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  constexpr int NC = R / 8;
  const uint16_t* src = lat + ((size_t)b * T + 32 * tile) * R;
  for (int idx = tid; idx < 32 * NC; idx += 256) {
    const int key = idx / NC, c = idx % NC;
    const u32x4 v = 32 * tile + key < T ? *(const u32x4*)(src + (size_t)key * R + 8 * c) : u32x4{0, 0, 0, 0};
    *(u32x4*)&s[key][8 * c] = v;
  }
  __syncthreads();
  uint16_t* dst = latT + ((size_t)b * nt + tile) * R * 32;
  for (int idx = tid; idx < 4 * R; idx += 256) {
    const int G = idx / R, rho = idx % R;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)s[tkey(G, 2 * i)][rho] | ((uint32_t)s[tkey(G, 2 * i + 1)][rho] << 16);
    *(u32x4*)(dst + (size_t)idx * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Row-major LDS tile for the scores: key row s keeps 16-byte chunk c at
// position c ^ (s & 15) within its aligned group of 16, so the reads of one
// chunk by 16 consecutive key rows (one pass of a 16-byte LDS read) hit 16
// distinct 16-byte bank groups.  The copy is 32 * R * 2 / 1024 LDS-DMA
// instructions of 1 KB (lane i lands at base + 16 i); wave w (wave-uniform)
// issues instructions w, w + 4, ...  Keys past nkeys-1 re-read row nkeys-1.
template <int R>
__device__ __forceinline__ void dma_rowtile(const uint16_t* latb, int k0, int nkeys, char* tile, int w) {
  constexpr int NC = R / 8;
  constexpr int NINSTR = 32 * R * 2 / 1024;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NINSTR / 4; ++i) {
    const int k = 4 * i + w;
    const int idx = k * 64 + lane;
    const int s = idx / NC, p = idx % NC;
    const int c = (p & ~15) | ((p & 15) ^ (s & 15));
    const int key = k0 + s < nkeys ? k0 + s : nkeys - 1;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(latb + (size_t)key * R + 8 * c),
        (__attribute__((address_space(3))) void*)(uintptr_t)(tile + k * 1024), 16, 0, 0);
  }
}

// Transposed tile: a straight copy of its [4][R][8] image (R * 64 bytes).
template <int R>
__device__ __forceinline__ void dma_tileT(const uint16_t* src, char* tbuf, int w) {
  constexpr int NINSTR = R * 64 / 1024;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NINSTR / 4; ++i) {
    const int k = 4 * i + w;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)((const char*)src + k * 1024 + 16 * lane),
        (__attribute__((address_space(3))) void*)(uintptr_t)(tbuf + k * 1024), 16, 0, 0);
  }
}

// Per-wave tile math of the prefill kernel on 16x16x32 matrix instructions.
// Lane l = 16 G + n.  The wave's 32 query rows form two blocks qb (rows
// 16 qb + n); a 32-key tile forms two key blocks kb.
//   scores:  S^T[16 kb + 4 G + v][16 qb + n] in s[kb][qb][v]   (A = L rows, B = q_lat^T)
//   P:       lane keeps, per qb, the 8 probabilities of its keys
//            {16 kb + 4 G + v}: k-slot 8 G + 4 kb + v of the P^T operand.
//   output:  O^T[16 c + 4 G + v][16 qb + n] in o[c][qb][v]      (A = L^T, B = P^T)
// so each lane holds two query rows, and a row's keys sit in the four lanes
// n + 16 G'.
template <int R>
struct Flash {
  static constexpr int NKS = R / 32;  // 32-wide steps of the rho contraction
  static constexpr int NOB = R / 16;  // 16-row blocks of output columns

  // Four independent accumulator chains keep the matrix unit busy.
  static __device__ __forceinline__ void scores(const char* rowtile, const bf16x8 (*qf)[NKS],
                                                f32x4 (&s)[2][2]) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // read i = 2 ks + kb: key row 16 kb + n, chunk 4 ks + G (swizzled by the row)
    auto addr = [&](int i) {
      const int kb = i & 1, ks = i >> 1;
      const int key = 16 * kb + n, c = 4 * ks + G;
      return (const bf16x8*)(rowtile + key * (R * 2) + 16 * ((c & ~15) | ((c & 15) ^ (key & 15))));
    };
    constexpr int NR = 2 * NKS, DEPTH = 3;  // LDS reads kept in flight ahead of their use
    bf16x8 ring[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) ring[i] = *addr(i);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bf16x8 av = ring[i % DEPTH];
      if (i + DEPTH < NR) ring[i % DEPTH] = *addr(i + DEPTH);
      const int kb = i & 1, ks = i >> 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma16x16x32(av, qf[qb][ks], s[kb][qb]);
      // keep each read DEPTH steps ahead of its use; vector ops may move freely
      __builtin_amdgcn_sched_barrier(0x0002 | 0x0400);
    }
  }

  // Online-softmax update of both query rows of the lane for one tile.  The
  // scores are already in log2 units (q_lat carries scale * log2 e).
  // lim[qb]: keys with offset 16 kb + v (from k0 + 4 G) above lim are masked.
  static __device__ __forceinline__ void softmax(const f32x4 (&s)[2][2], const int (&lim)[2],
                                                 float (&m_run)[2], float (&l_run)[2], float (&alpha)[2],
                                                 bool& grow_any, bf16x8 (&P)[2]) {
    grow_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) x[4 * kb + v] = (16 * kb + v > lim[qb]) ? -INFINITY : s[kb][qb][v];
      float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mt = max_xor32(max_xor16(mt));
      const bool grow = mt > m_run[qb] + kRescaleSlack;
      alpha[qb] = grow ? exp2f(m_run[qb] - mt) : 1.f;
      m_run[qb] = grow ? mt : m_run[qb];
      grow_any |= grow;
      const float msub = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float p = exp2f(x[u] - msub);
        ps += p;
        P[qb][u] = (__bf16)p;
      }
      l_run[qb] = l_run[qb] * alpha[qb] + ps;
    }
  }

  static __device__ __forceinline__ void rescale(f32x4 (&o)[NOB][2], const float (&alpha)[2]) {
    mfma_agpr_wait();
#pragma unroll
    for (int c = 0; c < NOB; ++c)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {  // a few registers at a time
        mfma_agpr_tie(o[c][qb]);
        o[c][qb] *= alpha[qb];
        mfma_agpr_tie(o[c][qb]);
      }
  }

  // O^T += L^T P^T from the transposed tile ([4][R][8] image).
  static __device__ __forceinline__ void pv(const char* ttile, bf16x8 (&P)[2], f32x4 (&o)[NOB][2]) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n = lane & 15;
    const char* pa = ttile + G * (R * 16) + 16 * n;
    constexpr int DEPTH = 4;  // LDS reads kept in flight ahead of their use
    bf16x8 ring[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) ring[i] = *(const bf16x8*)(pa + 256 * i);
    mfma_operand_ready(P[0]);
    mfma_operand_ready(P[1]);
#pragma unroll
    for (int c = 0; c < NOB; ++c) {
      const bf16x8 av = ring[c % DEPTH];
      if (c + DEPTH < NOB) ring[c % DEPTH] = *(const bf16x8*)(pa + 256 * (c + DEPTH));
      mfma16x16x32_a(o[c][0], av, P[0]);
      mfma16x16x32_a(o[c][1], av, P[1]);
    }
  }
};

// q_lat, o_lat: [B][T*H][R] bf16 (row t*H + h of batch b; q_lat pre-scaled by
// scale * log2 e); lat: [B][T][R];
// latT: [B][ceil(T/32)][R][32] (latent_transpose).  One block = 128
// consecutive (t, h) rows of one batch = 4 waves x 32 rows; all heads in the
// block share each latent tile.  Per tile j the wave computes the softmax of
// tile j while the scores of tile j+1 run on the matrix unit, then P_j L_j.
// Row-major tiles (two buffers) and transposed tiles (three buffers) are
// both copied two tiles ahead.  Blocks are issued heaviest (largest t) first.
template <int R>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void flash_latent_bf16(const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ lat,
                       const uint16_t* __restrict__ latT, uint16_t* __restrict__ o_lat, int B,
                       int T, int H) {
  using F = Flash<R>;
  constexpr int TILE_BYTES = 32 * R * 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* rowbuf = smem;                      // [2][TILE_BYTES]
  char* tbuf = smem + 2 * TILE_BYTES;       // [3][TILE_BYTES]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int G = lane >> 4, n = lane & 15;
  const long TH = (long)T * H;
  const int nrb = (int)((TH + 127) / 128);
  const int nt = (T + 31) / 32;
  const int rb = nrb - 1 - (int)(blockIdx.x / B);
  const int b = blockIdx.x % B;
  const long row0 = (long)rb * 128;
  const long row_end = TH < row0 + 128 ? TH : row0 + 128;
  const int t_last_blk = (int)((row_end - 1) / H);
  const int ntiles = t_last_blk / 32 + 1;
  const long wrow0 = row0 + 32 * w;
  const bool wactive = wrow0 < TH;
  const int t_first_w = wactive ? (int)(wrow0 / H) : 0;
  const int t_last_w = wactive ? (int)(((TH < wrow0 + 32 ? TH : wrow0 + 32) - 1) / H) : -1;
  long my_row[2];
  int t_row[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    my_row[qb] = wrow0 + 16 * qb + n;
    const long crow = my_row[qb] < TH ? my_row[qb] : TH - 1;
    t_row[qb] = (int)(crow / H);
  }

  bf16x8 qf[2][F::NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const long crow = my_row[qb] < TH ? my_row[qb] : TH - 1;
    const uint16_t* qrow = q_lat + ((size_t)b * TH + crow) * R + 8 * G;
#pragma unroll
    for (int ks = 0; ks < F::NKS; ++ks) qf[qb][ks] = *(const bf16x8*)(qrow + 32 * ks);
  }
  f32x4 o[F::NOB][2];
#pragma unroll
  for (int c = 0; c < F::NOB; ++c) o[c][0] = o[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const uint16_t* latb = lat + (size_t)b * T * R;
  const uint16_t* latTb = latT + (size_t)b * nt * R * 32;
  dma_rowtile<R>(latb, 0, T, rowbuf, w);
  dma_tileT<R>(latTb, tbuf, w);
  if (ntiles > 1) {
    dma_rowtile<R>(latb, 32, T, rowbuf + TILE_BYTES, w);
    dma_tileT<R>(latTb + (size_t)R * 32, tbuf + TILE_BYTES, w);
  }
  wait_all_memory();
  __syncthreads();
  f32x4 s_cur[2][2];
  F::scores(rowbuf, qf, s_cur);
  __syncthreads();  // row tile 0 is refilled below
  for (int j = 0; j < ntiles; ++j) {
    // tiles j+2 (both orientations) are copied during this iteration; at
    // its end only the copies issued one iteration earlier must have landed
    const bool ahead = j + 2 < ntiles;
    if (ahead) {
      dma_tileT<R>(latTb + (size_t)(j + 2) * R * 32, tbuf + ((j + 2) % 3) * TILE_BYTES, w);
      dma_rowtile<R>(latb, 32 * (j + 2), T, rowbuf + (j & 1) * TILE_BYTES, w);
    }
    const int k0 = 32 * j;
    const bool act = k0 <= t_last_w;
    const bool need_mask = k0 + 31 > t_first_w;
    int lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) lim[qb] = need_mask ? t_row[qb] - k0 - 4 * G : 1 << 30;
    // Softmax of tile j (vector ALU) next to the scores of tile j+1 (matrix
    // unit).  Both run unconditionally: a tile past the wave's rows is fully
    // masked (p = 0, state unchanged); the scores after the last tile read a
    // stale buffer and are discarded.
    bf16x8 P[2];
    float alpha[2];
    bool grow_any;
    F::softmax(s_cur, lim, m_run, l_run, alpha, grow_any, P);
    f32x4 s_next[2][2];
    F::scores(rowbuf + ((j + 1) & 1) * TILE_BYTES, qf, s_next);
    if (act) {
      if (__builtin_amdgcn_ballot_w64(grow_any)) F::rescale(o, alpha);
      F::pv(tbuf + (j % 3) * TILE_BYTES, P, o);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s_cur[kb][qb] = s_next[kb][qb];
    if (ahead)
      wait_vmem_outstanding<2 * (32 * R * 2 / 1024 / 4)>();  // tiles j+2 may stay in flight
    else
      wait_all_memory();
    // a bare barrier: __syncthreads() would also wait for the copy still in flight
    __builtin_amdgcn_s_barrier();
  }
  if (!wactive) return;
  mfma_agpr_wait();
#pragma unroll
  for (int c = 0; c < F::NOB; ++c) {
    mfma_agpr_tie(o[c][0]);
    mfma_agpr_tie(o[c][1]);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l_run[qb] + __shfl_xor(l_run[qb], 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.f / lt;
    if (my_row[qb] >= TH) continue;
    uint16_t* orow = o_lat + ((size_t)b * TH + my_row[qb]) * R + 4 * G;
#pragma unroll
    for (int c = 0; c < F::NOB; ++c) {
      u32x2 v = {pack_bf16x2(o[c][qb][0] * inv, o[c][qb][1] * inv),
                 pack_bf16x2(o[c][qb][2] * inv, o[c][qb][3] * inv)};
      *(u32x2*)(orow + 16 * c) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
template <int R>
static hipError_t run_prefill(const uint16_t* q, const uint16_t* lat, const uint16_t* wk,
                              const uint16_t* wv, uint16_t* out, int B, int T, int H, int d,
                              float sl2, uint16_t* q_lat, uint16_t* o_lat, uint16_t* wvT,
                              uint16_t* latT, hipStream_t st) {
  const int N = B * T;
  const int nt = (T + 31) / 32;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)flash_latent_bf16<R>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)flash_lds_bytes(R));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipError_t e = absorb_mfma(q, wk, q_lat, N, H, d, R, sl2, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("transpose_wv", st);
    e = transpose_wv_launch(wv, wvT, R, H, d, st);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("latent_transpose", st);
    hipLaunchKernelGGL(latent_transpose<R>, dim3(nt, B), dim3(256), 0, st, lat, latT, T, nt);
  }
  const long TH = (long)T * H;
  const int nrb = (int)((TH + 127) / 128);
  {
    ProfScope ps("flash_latent_bf16", st);
    hipLaunchKernelGGL(flash_latent_bf16<R>, dim3(B * nrb), dim3(256), flash_lds_bytes(R), st, q_lat,
                       lat, latT, o_lat, B, T, H);
  }
  {
    ProfScope ps("up_bf16", st);
    hipLaunchKernelGGL(up_bf16<R>, dim3((N + 127) / 128, H), dim3(256), 0, st, o_lat, wvT, out, N, H, d);
  }
  return hipGetLastError();
}

hipError_t prefill_mfma(const void* q, const void* lat, const void* wk, const void* wv, void* out,
                        int B, int T, int H, int d, int r, float sl2, void* ws, hipStream_t st) {
  const size_t rows = (size_t)B * T * H;
  uint16_t* q_lat = (uint16_t*)ws;
  uint16_t* o_lat = q_lat + rows * r;
  uint16_t* wvT = o_lat + rows * r;
  uint16_t* latT = wvT + (size_t)H * d * r;
#define ARGS (const uint16_t*)q, (const uint16_t*)lat, (const uint16_t*)wk, (const uint16_t*)wv, \
             (uint16_t*)out, B, T, H, d, sl2, q_lat, o_lat, wvT, latT, st
  switch (r) {
    case 128: return run_prefill<128>(ARGS);
    case 256: return run_prefill<256>(ARGS);
    case 512: return run_prefill<512>(ARGS);
  }
#undef ARGS
  return hipErrorInvalidValue;
}

size_t prefill_mfma_workspace(int B, int T, int H, int d, int r) {
  const size_t rows = (size_t)B * T * H;
  const size_t nt = ((size_t)T + 31) / 32;
  return (2 * rows * r + (size_t)H * d * r + (size_t)B * nt * 32 * r) * 2;
}

}  // namespace mla
