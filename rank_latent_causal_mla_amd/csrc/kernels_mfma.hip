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
#include "lds_tiles.h"
#include "prep_blocks.h"
#include "profile.h"
#include "host_once.h"

namespace mla {

// ---------------------------------------------------------------------------
// Absorption (one block per 32 query rows of one head, the whole rank) and
// the W_uv transpose, as kernels around the block bodies of prep_blocks.h.
// Absorption for prefill: q_lat[n*H + h, rho] = qscale * sum_e W_uk[rho, h, e] * q[n, h, e]
// (n = b*T + t; qscale folds the softmax scale and log2 e into q_lat).
// Computed transposed, q_lat^T = W_h q_h^T.  Block: head h, the rank slice
// [128 NB blockIdx.z, +128 NB) (wave w holds its 32 NB rows of W_uk in
// registers) and kAbsorbRowBlocks row blocks of 32 queries, whose q rows are
// copied into LDS once per block by LDS-DMA (two buffers, the next copy in
// flight), chunk-swizzled so the operand reads are conflict-free.
constexpr int kAbsorbRowBlocks = 32;
template <int R, int DK>
constexpr int absorb_nb() { return R / 128 < 32 / DK ? R / 128 : 32 / DK; }

// 16-byte chunk c of q row s (d / 8 chunks per row) sits at position
// qswz(c, s): within every 256 bytes of LDS, 16 consecutive rows reading the
// same chunk hit 16 distinct slots.
template <int DK>
__device__ __forceinline__ int qswz(int c, int s) {
  constexpr int NCd = 2 * DK;  // chunks per row
  if constexpr (NCd >= 16) return (c & ~15) | ((c & 15) ^ (s & 15));
  else return c ^ ((s / (16 / NCd)) & (NCd - 1));
}

// The results of a row block (32 rows x the block's 128 NB columns) are
// staged in LDS and stored as whole row segments, 16 bytes a lane: the matrix
// layout leaves each lane four consecutive columns of one row, and storing
// those directly scatters every instruction over 32 rows.  Staged rows are
// padded by 16 bytes, so the 16 lanes of an 8-byte staging write (rows
// 0..15 of one column) fall on distinct bank pairs but for rows r and r + 8.
template <int R, int DK>
__global__ __launch_bounds__(256, 2) void absorb_bf16(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ wk,
                                                      uint16_t* __restrict__ q_lat, int N, int H,
                                                      float qscale) {
  constexpr int NB = absorb_nb<R, DK>();
  constexpr int d = 16 * DK;
  constexpr int TB = 32 * d * 2;                      // q rows of one row block
  constexpr int NCd = d / 8;                          // chunks per row
  constexpr int RPI = 64 / NCd;                       // rows per copy instruction
  constexpr int NINS = TB / 1024;                     // copy instructions per row block
  constexpr int NIW = NINS >= 4 ? NINS / 4 : 1;       // at most, per wave
  constexpr int RB = 128 * NB;                        // columns of the block
  constexpr int OS = RB * 2 + 16;                     // staged row stride, bytes
  constexpr int OCH = RB / 8;                         // 16-byte chunks of a staged row
  static_assert(NCd <= 64 && 64 % NCd == 0 && TB % 1024 == 0, "copies cover whole rows");
  static_assert((32 * OCH) % 256 == 0, "the block's threads share the staged chunks evenly");
  __shared__ __attribute__((aligned(16))) char buf[2][TB];
  __shared__ __attribute__((aligned(16))) char ostage[32 * OS];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const int rho0 = 128 * NB * blockIdx.z + w * 32 * NB;
  const int nb0 = blockIdx.x * kAbsorbRowBlocks;
  const int nrb_all = (N + 31) / 32;
  const int nbn = nrb_all - nb0 < kAbsorbRowBlocks ? nrb_all - nb0 : kAbsorbRowBlocks;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&buf[0][0]);

  bf16x8 a[NB][DK];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint16_t* wrow = wk + ((size_t)(rho0 + 32 * i + l32) * H + h) * d + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) a[i][ks] = *(const bf16x8*)(wrow + 16 * ks);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) asm volatile("" : : "v"(a[i][ks]));  // loaded before the copies start
  const int sl = lane / NCd, p = lane % NCd;
  auto copy = [&](int k) {
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      const int ins = 4 * u + w;
      if (ins < NINS) {
        const int s = ins * RPI + sl;  // row within the block
        const int n = min(32 * (nb0 + k) + s, N - 1);
        const int n0 = __builtin_amdgcn_readfirstlane(min(32 * (nb0 + k) + ins * RPI, N - 1));
        const int c = qswz<DK>(p, s);  // the swizzle is its own inverse
        dma16(q + ((size_t)n0 * H + h) * d, (uint32_t)(((size_t)(n - n0) * H) * d * 2 + 16 * c),
              lds0 + (k & 1) * TB + ins * 1024);
      }
    }
  };
  copy(0);
  for (int k = 0; k < nbn; ++k) {
    if (k + 1 < nbn) {
      copy(k + 1);
      dma_wait<NIW>();  // own part of row block k landed
    } else {
      dma_wait<0>();
    }
    __builtin_amdgcn_s_barrier();
    const char* row = &buf[k & 1][0] + l32 * (d * 2);
    bf16x8 bq[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) bq[ks] = lds_read16(row + 16 * qswz<DK>(2 * ks + g, l32));
    f32x16 acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      acc[i] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) acc[i] = mfma32x32x16(a[i][ks], bq[ks], acc[i]);
    }
    // stage: lane (g, l32) holds columns 32 i + 8 j + 4 g .. + 3 (of the
    // wave's 32 NB) of row l32
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = w * 32 * NB + 32 * i + 8 * j + 4 * g;
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(ostage + l32 * OS + 2 * col) =
            u32x2{pack_bf16x2(acc[i][4 * j] * qscale, acc[i][4 * j + 1] * qscale),
                  pack_bf16x2(acc[i][4 * j + 2] * qscale, acc[i][4 * j + 3] * qscale)};
      }
    lds_publish_barrier();  // the row block's results are staged
    // store: chunk c = tid + 256 u is row c / OCH, 16-byte piece c % OCH
#pragma unroll
    for (int u = 0; u < 32 * OCH / 256; ++u) {
      const int c = threadIdx.x + 256 * u, row = c / OCH, piece = c % OCH;
      const int n = 32 * (nb0 + k) + row;
      const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(ostage + row * OS + 16 * piece);
      if (n < N) *(u32x4*)(q_lat + ((size_t)n * H + h) * R + 128 * NB * blockIdx.z + 8 * piece) = v;
    }
    __builtin_amdgcn_s_barrier();  // buffer k & 1 is refilled and the stage rewritten next iteration
  }
}

__global__ __launch_bounds__(256) void transpose_wv(const uint16_t* __restrict__ wv, uint16_t* __restrict__ wvT,
                                                    int R, int H, int d) {
  __shared__ __attribute__((aligned(16))) TransposeRow tile[kTransposeTile];
  transpose_wv_tile(wv, wvT, R, H, d, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

template <int R>
static hipError_t absorb_launch(const uint16_t* q, const uint16_t* wk, uint16_t* q_lat, int N, int H,
                                int d, float qscale, hipStream_t st) {
  const int nrb = (N + 32 * kAbsorbRowBlocks - 1) / (32 * kAbsorbRowBlocks);
  switch (d) {
    case 32: hipLaunchKernelGGL((absorb_bf16<R, 2>), dim3(nrb, H, R / (128 * absorb_nb<R, 2>())), dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 64: hipLaunchKernelGGL((absorb_bf16<R, 4>), dim3(nrb, H, R / (128 * absorb_nb<R, 4>())), dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 128: hipLaunchKernelGGL((absorb_bf16<R, 8>), dim3(nrb, H, R / (128 * absorb_nb<R, 8>())), dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
    case 256: hipLaunchKernelGGL((absorb_bf16<R, 16>), dim3(nrb, H, R / (128 * absorb_nb<R, 16>())), dim3(256), 0, st, q, wk, q_lat, N, H, qscale); break;
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
  hipLaunchKernelGGL(transpose_wv, dim3(R / kTransposeTile, (d + kTransposeTile - 1) / kTransposeTile, H), dim3(256), 0, st,
                     wv, wvT, R, H, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Up-projection: out[n, h, e] = oscale * sum_rho src[row, rho] * W[rho, h, e]
// with row = n*H + h (per-head rows: o_lat) or, with SHARED, row = n (one
// row for all heads: the latent, when k or v are materialised), computed as
// out^T = W^T src^T from W^T [H][d][R].  Block: head h, output columns
// e = 128 blockIdx.z + 32 w .. (wave w holds that slice of W_uv^T in
// registers), and row blocks kUpRowBlocks * blockIdx.x .. of 32 rows.  The
// o_lat rows of a row block are copied once per block into LDS by LDS-DMA
// (two buffers, the next block's copy in flight), chunk-swizzled by the row
// so the four waves' operand reads are conflict-free.  Blocks with blockIdx.z
// >= zsplit compute a second product of the same rows (W2, out2, oscale2):
// k and v from the latent in one launch.
constexpr int kUpRowBlocks = 32;
template <int R>
constexpr size_t up_lds_bytes() { return (size_t)2 * 32 * R * 2; }

template <int R, bool SHARED>
__global__ __launch_bounds__(256, 2) void up_bf16(const uint16_t* __restrict__ o_lat,
                                                  const uint16_t* __restrict__ wvT1,
                                                  uint16_t* __restrict__ out1, float oscale1,
                                                  const uint16_t* __restrict__ wvT2,
                                                  uint16_t* __restrict__ out2, float oscale2, int zsplit,
                                                  int N, int H, int d) {
  constexpr int NKS = R / 16;           // contraction steps
  constexpr int TB = 32 * R * 2;        // one row block in LDS
  constexpr int NC = R / 8;             // 16-byte chunks per row
  constexpr int RPI = 64 / NC;          // rows per copy instruction
  constexpr int NI = TB / 1024 / 4;     // copy instructions per wave and row block
  static_assert(NC <= 64 && 64 % NC == 0, "a copy instruction covers whole rows");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y;
  const bool second = (int)blockIdx.z >= zsplit;
  const uint16_t* __restrict__ wvT = second ? wvT2 : wvT1;
  uint16_t* __restrict__ out = second ? out2 : out1;
  const float oscale = second ? oscale2 : oscale1;
  const int i = 4 * ((int)blockIdx.z - (second ? zsplit : 0)) + w;  // output block of 32 columns
  const bool has_cols = i < d / 32;
  const int nb0 = blockIdx.x * kUpRowBlocks;
  const int nrb_all = (N + 31) / 32;
  const int nbn = nrb_all - nb0 < kUpRowBlocks ? nrb_all - nb0 : kUpRowBlocks;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  bf16x8 a[NKS];
  if (has_cols) {
    const uint16_t* wrow = wvT + ((size_t)h * d + 32 * i + l32) * R + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const bf16x8*)(wrow + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : : "v"(a[ks]));  // loaded before the copies start
  }
  // copy of row block k (rows 32 (nb0 + k) + s, s = 0..31) into buffer k & 1
  const int sl = lane / NC, p = lane % NC;
  auto copy = [&](int k) {
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int ins = 4 * u + w;
      const int s = ins * RPI + sl;  // row within the block
      const int n = min(32 * (nb0 + k) + s, N - 1);
      const int n0 = __builtin_amdgcn_readfirstlane(min(32 * (nb0 + k) + ins * RPI, N - 1));
      const int c = (p & ~15) | ((p & 15) ^ (s & 15));
      if (SHARED)
        dma16(o_lat + (size_t)n0 * R, (uint32_t)((n - n0) * R * 2 + 16 * c), lds0 + (k & 1) * TB + ins * 1024);
      else
        dma16(o_lat + ((size_t)n0 * H + h) * R, (uint32_t)(((size_t)(n - n0) * H) * R * 2 + 16 * c),
              lds0 + (k & 1) * TB + ins * 1024);
    }
  };
  copy(0);
  for (int k = 0; k < nbn; ++k) {
    if (k + 1 < nbn) {
      copy(k + 1);
      dma_wait<NI>();  // own part of row block k landed
    } else {
      dma_wait<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (has_cols) {
      const char* buf = smem + (k & 1) * TB + l32 * (R * 2);
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ks += 2) {
        const int c0 = 2 * ks + g, c1 = c0 + 2;
        const bf16x8 b0 = lds_read16(buf + 16 * ((c0 & ~15) | ((c0 & 15) ^ (l32 & 15))));
        const bf16x8 b1 = lds_read16(buf + 16 * ((c1 & ~15) | ((c1 & 15) ^ (l32 & 15))));
        acc0 = mfma32x32x16(a[ks], b0, acc0);
        acc1 = mfma32x32x16(a[ks + 1], b1, acc1);
      }
      const int n = 32 * (nb0 + k) + l32;
      if (n < N) {
        uint16_t* dst = out + ((size_t)n * H + h) * d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 32 * i + 8 * j + 4 * g;
          u32x2 v = {pack_bf16x2((acc0[4 * j] + acc1[4 * j]) * oscale, (acc0[4 * j + 1] + acc1[4 * j + 1]) * oscale),
                     pack_bf16x2((acc0[4 * j + 2] + acc1[4 * j + 2]) * oscale,
                                 (acc0[4 * j + 3] + acc1[4 * j + 3]) * oscale)};
          *(u32x2*)(dst + e) = v;
        }
      }
    }
    __builtin_amdgcn_s_barrier();  // buffer k & 1 is refilled next iteration
  }
}

// ---------------------------------------------------------------------------
// Causal latent flash attention, prefill.
//
// One block = 128 consecutive (t, h) rows of one batch; all its rows attend
// the same latent tiles (K = V = latent), streamed through a ring of
// kFlashBufs swizzled row-major 32-key tiles (lds_tiles.h) by LDS-DMA.  The
// two products split the work differently over the four waves:
//   scores + softmax: wave w owns rows 32 w .. 32 w + 31 (q_lat in registers);
//   P * latent:       wave w owns latent columns [R w / 4, R (w + 1) / 4) of
//                     all 128 rows (the output accumulator, in AGPRs).
// Each tile's probabilities (bf16) and rescale factors go through LDS from
// the row owners to the column owners.  Compared with one wave doing both
// products for its own rows, every latent byte read from LDS by the second
// product now serves 128 rows instead of 32, and the transposed operand is
// read straight from the row tile with transpose reads, so each tile is
// copied once.  Lane l = 16 G + n.
//   scores:  S^T[16 kb + 4 G + v][16 qb + n] in s[kb][qb][v]     (16x16x32, A = L rows)
//   P:       lane keeps, per own row block qb, the 8 probabilities of keys
//            {16 kb + 4 G + v} = the P^T operand of that row block
//   output:  O^T[R w / 4 + 16 c + 4 G + v][16 q + n] in o[c][q][v], q = 0..7 (A by TileCols)
constexpr int kFlashBufs = 4;

template <int R>
struct Flash {
  static constexpr int NKS = R / 32;  // 32-wide steps of the rho contraction
  static constexpr int NCW = R / 64;  // 16-column blocks of a wave's quarter
  static constexpr int NQ = 8;        // 16-row blocks of the block's rows

  // S^T for the wave's 32 rows: four independent accumulator chains.
  static __device__ __forceinline__ void scores(const char* tile, const bf16x8 (*qf)[NKS], f32x4 (&s)[2][2]) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n = lane & 15;
    const int f = tswz(n);  // rows n and 16 + n share the swizzle
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // read i = 2 ks + kb: key row 16 kb + n, chunk 4 ks + G
    auto rd = [&](int i) {
      const int kb = i & 1, ks = i >> 1;
      const int c = 4 * ks + G;
      return lds_read16(tile + (16 * kb + n) * (R * 2) + 16 * ((c & ~15) | ((c & 15) ^ f)));
    };
    constexpr int NR = 2 * NKS, DEPTH = 3;  // LDS reads kept in flight ahead of their use
    bf16x8 ring[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) ring[i] = rd(i);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bf16x8 av = ring[i % DEPTH];
      if (i + DEPTH < NR) ring[i % DEPTH] = rd(i + DEPTH);
      const int kb = i & 1, ks = i >> 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mfma16x16x32(av, qf[qb][ks], s[kb][qb]);
      __builtin_amdgcn_sched_barrier(0x0002 | 0x0400);
    }
  }

  // S^T of the next tile (into s) with the online-softmax update of the
  // current one (scores sc) spread over its matrix ops: the update is cut
  // into 40 pieces of a few vector instructions, and piece k is issued after
  // matrix op k + kPieceLag, so it runs while the matrix unit is busy instead
  // of between the two products.  At R = 512 the pieces fill the last 40 of
  // the 64 matrix ops (a lag of 24 ran 1% faster than 8; 12, 16, 18 and 22
  // were no better than 8).  Scores are in log2 units (q_lat carries
  // scale * log2 e).  With MASK, keys 16 kb + v (from k0 + 4 G) above lim[qb]
  // are masked.  A row's reference moves when its tile maximum exceeds thr
  // (its running maximum plus the slack); the probabilities are taken
  // relative to msub, the new maximum where grow is set and mref (the
  // running maximum, or 0 before the row's first visible key) otherwise.
  // ps returns the sums of the probabilities: the caller updates the state,
  // the running sums and the rescale factors only when some row moved.
  // Returns whether any row's reference moved.
  static constexpr int kPieceLag = 4 * NKS - 40 > 8 ? 4 * NKS - 40 : 8;
  template <bool MASK>
  static __device__ __forceinline__ bool scores_softmax(const char* tile, const bf16x8 (*qf)[NKS], f32x4 (&s)[2][2],
                                                        const f32x4 (&sc)[2][2], const int (&lim)[2], const float (&thr)[2],
                                                        const float (&mref)[2], float (&msub)[2], bool (&grow)[2],
                                                        float (&ps)[2], bf16x8 (&P)[2]) {
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, n = lane & 15;
    const int f = tswz(n);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto rd = [&](int i) {
      const int kb = i & 1, ks = i >> 1;
      const int c = 4 * ks + G;
      return lds_read16(tile + (16 * kb + n) * (R * 2) + 16 * ((c & ~15) | ((c & 15) ^ f)));
    };
    float x[2][8], mm[2][4], mt[2];
    ps[0] = ps[1] = 0.f;
    uint32_t pk[2][4];
    auto piece = [&](int k) {
      if (k < 0) {
      } else if (k < 8) {  // 0..7: masking and the lane's maximum of row block k / 4
        const int qb = k >> 2, part = k & 3;
        if (part == 0) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              x[qb][4 * kb + v] = (MASK && 16 * kb + v > lim[qb]) ? -INFINITY : sc[kb][qb][v];
          mm[qb][0] = fmaxf(x[qb][0], x[qb][1]);
          mm[qb][1] = fmaxf(x[qb][2], x[qb][3]);
        } else if (part == 1) {
          mm[qb][2] = fmaxf(x[qb][4], x[qb][5]);
          mm[qb][3] = fmaxf(x[qb][6], x[qb][7]);
        } else if (part == 2) {
          mm[qb][0] = fmaxf(mm[qb][0], mm[qb][1]);
          mm[qb][2] = fmaxf(mm[qb][2], mm[qb][3]);
        } else {
          mt[qb] = fmaxf(mm[qb][0], mm[qb][2]);
        }
      } else if (k < 12) {  // 8..11: maximum over the four lanes of a row
        const int qb = k & 1;
        mt[qb] = k < 10 ? max_xor16(mt[qb]) : max_xor32(mt[qb]);
      } else if (k < 14) {  // 12, 13: does the reference move
        const int qb = k & 1;
        grow[qb] = mt[qb] > thr[qb];
      } else if (k < 16) {  // 14, 15: the reference of this tile's probabilities
        const int qb = k & 1;
        msub[qb] = grow[qb] ? mt[qb] : mref[qb];
      } else if (k < 32) {  // 16..31: probability u of row block qb, summed in pairs
        const int qb = k & 1, u = (k - 16) >> 1;
        x[qb][u] = fast_exp2(x[qb][u] - msub[qb]);
        if (u & 1) ps[qb] += x[qb][u - 1] + x[qb][u];
      } else if (k < 40) {  // 32..39: bf16 pairs, then the P operand
        const int qb = k & 1, u = (k - 32) >> 1;
        pk[qb][u] = pack_bf16x2(x[qb][2 * u], x[qb][2 * u + 1]);
        if (u == 3) P[qb] = __builtin_bit_cast(bf16x8, u32x4{pk[qb][0], pk[qb][1], pk[qb][2], pk[qb][3]});
      }
    };
    constexpr int NR = 2 * NKS, DEPTH = 3;
    bf16x8 ring[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) ring[i] = rd(i);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bf16x8 av = ring[i % DEPTH];
      if (i + DEPTH < NR) ring[i % DEPTH] = rd(i + DEPTH);
      const int kb = i & 1, ks = i >> 1;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[kb][qb] = mfma16x16x32(av, qf[qb][ks], s[kb][qb]);
        piece(2 * i + qb - kPieceLag);
        __builtin_amdgcn_sched_barrier(0);  // keep the piece after its matrix op
      }
    }
#pragma unroll
    for (int k = 2 * NR - kPieceLag; k < 40; ++k) piece(k);  // small R: fewer matrix ops than pieces
    return grow[0] || grow[1];
  }
};

// q_lat, o_lat: [B][T*H][R] bf16 (row t*H + h of batch b; q_lat pre-scaled by
// scale * log2 e); lat: [B][T][R].  Per tile j the wave computes the softmax
// of tile j while the scores of tile j+1 run on the matrix unit, posts P_j,
// then accumulates P_j L_j for its columns.  Tiles are copied three ahead;
// blocks are issued heaviest (largest t) first.
// With COMPACT (key mask), lat holds each batch's visible keys packed in
// order (zero rows after them) and cnt [B][T] the number of visible keys
// s <= t: query t then attends packed keys 0 .. cnt[b][t] - 1, which are its
// visible keys, through the same causal limit.  A row with no visible key
// (cnt = 0) masks every key and ends with l = 0; its output is written as
// NaN, the value the softmax of an all -infinity row takes.
template <int R, bool COMPACT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void flash_latent_bf16(const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ lat,
                       uint16_t* __restrict__ o_lat, int B, int T, int H, const int32_t* __restrict__ cnt) {
  using F = Flash<R>;
  constexpr int TILE = kTileKeys * R * 2;
  constexpr int NI = TILE / 1024 / 4;  // copy instructions per wave and tile
  static_assert(kFlashBufs == 4, "three tiles in flight");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* pbuf = smem + kFlashBufs * TILE;         // [8 q][64 lanes] x 16 bytes of P
  float* abuf = (float*)(pbuf + F::NQ * 1024);   // [8 q][16] rescale factors, then l
  int* fbuf = (int*)(abuf + F::NQ * 16);         // [4]: wave w's rows rescale this tile
  // COMPACT: [4 w][2 qb][64 lanes] last key of each row, read back per tile
  // by the lane that wrote it (a loaded value kept in a register would be
  // spilled, and a scratch reload inside the loop waits on the tile copies;
  // for the same reason the tile copies recompute their lane offsets there)
  int* tbuf = fbuf + 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int G = lane >> 4, n = lane & 15;
  const long TH = (long)T * H;
  const int nrb = (int)((TH + 127) / 128);
  const int rb = nrb - 1 - (int)(blockIdx.x / B);
  const int b = blockIdx.x % B;
  const long row0 = (long)rb * 128;
  const long row_end = TH < row0 + 128 ? TH : row0 + 128;
  // last key position row t attends (cnt is nondecreasing in t)
  auto last_key = [&](int t) { return COMPACT ? cnt[(size_t)b * T + t] - 1 : t; };
  const int t_last_blk = last_key((int)((row_end - 1) / H));
  const int ntiles = t_last_blk / kTileKeys + 1;  // at least 1 (-1 / 32 = 0)
  // rows owned for the scores: 32 w .. 32 w + 31 of the block
  const long wrow0 = row0 + 32 * w;
  const int t_first_w = last_key((int)((wrow0 < TH ? wrow0 : TH - 1) / H));
  long my_row[2];
  int t_row[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    my_row[qb] = wrow0 + 16 * qb + n;
    t_row[qb] = last_key((int)((my_row[qb] < TH ? my_row[qb] : TH - 1) / H));
  }
  const uint16_t* latb = lat + (size_t)b * T * R;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  if (COMPACT) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) tbuf[(2 * w + qb) * 64 + lane] = t_row[qb];
  }

  // first tiles in flight while the queries load
#pragma unroll
  for (int t = 0; t < kFlashBufs - 1; ++t)
    if (t < ntiles) dma_tile32<R>(latb, kTileKeys * t, T, lds0 + t * TILE, w);
  bf16x8 qf[2][F::NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const long crow = my_row[qb] < TH ? my_row[qb] : TH - 1;
    const uint16_t* qrow = q_lat + ((size_t)b * TH + crow) * R + 8 * G;
#pragma unroll
    for (int ks = 0; ks < F::NKS; ++ks) qf[qb][ks] = *(const bf16x8*)(qrow + 32 * ks);
  }
  // Consume the query registers before the loop: the copies are invisible to
  // the compiler's wait counting, and a query load still pending at the loop
  // head would make it wait on the vector-memory counter every iteration.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < F::NKS; ++ks) asm volatile("" : : "v"(qf[qb][ks]));

  f32x4 o[F::NCW][F::NQ];
#pragma unroll
  for (int c = 0; c < F::NCW; ++c)
#pragma unroll
    for (int q = 0; q < F::NQ; ++q) o[c][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running maximum and sum of the lane's row in each row block; thr =
  // m_run + slack and mref = m_run (0 while m_run is -inf) are kept as state
  // so that the usual tile spends no instruction on deriving them
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  float thr[2] = {-INFINITY, -INFINITY}, mref[2] = {0.f, 0.f};
  const int cw = w * (R / 4);
  const TileCols<R> cols;

  // tiles 0 and 1 landed (tile 2 may still be in flight)
  if (ntiles > 2)
    dma_wait<NI>();
  else
    dma_wait<0>();
  __builtin_amdgcn_s_barrier();
  f32x4 s_cur[2][2];
  F::scores(smem, qf, s_cur);
  for (int j = 0; j < ntiles; ++j) {
    const int k0 = kTileKeys * j;
    int lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      lim[qb] = (COMPACT ? *(const __attribute__((address_space(3))) int*)(uintptr_t)(tbuf + (2 * w + qb) * 64 + lane)
                         : t_row[qb]) - k0 - 4 * G;
    bf16x8 P[2];
    float msub[2], ps[2];
    bool growq[2];
    // scores of tile j + 1 (after the last tile: a stale buffer, discarded)
    // with the softmax of tile j between their matrix ops
    f32x4 s_next[2][2];
    const char* ntile = smem + ((j + 1) % kFlashBufs) * TILE;
    const bool grow = k0 + kTileKeys - 1 > t_first_w
                          ? F::template scores_softmax<true>(ntile, qf, s_next, s_cur, lim, thr, mref, msub, growq, ps, P)
                          : F::template scores_softmax<false>(ntile, qf, s_next, s_cur, lim, thr, mref, msub, growq, ps, P);
    // every wave passed the barrier that ended iteration j - 1: the exchange buffers are free
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(pbuf + ((2 * w + qb) * 64 + lane) * 16) = P[qb];
    // every lane votes: a ballot inside the lane-0 branch would see lane 0's row only
    const uint64_t grew = __builtin_amdgcn_ballot_w64(grow);
    if (grew != 0) {  // rare: rescale factors, posted only by a wave whose rows moved
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float alpha = growq[qb] ? fast_exp2(m_run[qb] - msub[qb]) : 1.f;
        if (growq[qb]) {
          m_run[qb] = msub[qb];
          thr[qb] = msub[qb] + kRescaleSlack;
          mref[qb] = msub[qb];
        }
        l_run[qb] = l_run[qb] * alpha + ps[qb];
        if (G == 0) abuf[(2 * w + qb) * 16 + n] = alpha;
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) l_run[qb] += ps[qb];
    }
    if (lane == 0) fbuf[w] = grew != 0;
    lds_publish_barrier();  // P and rescale factors of tile j posted
    // The flags first: the branch on them then waits for this read alone (the
    // LDS counter drains in order), while the P and latent reads behind it
    // are still in flight.
    const u32x4 f = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)fbuf;
    bf16x8 pq[F::NQ];
#pragma unroll
    for (int q = 0; q < F::NQ; ++q) pq[q] = lds_read16(pbuf + (q * 64 + lane) * 16);
    const char* tile = smem + (j % kFlashBufs) * TILE;
    bf16x8 a_next = cols(tile, cw);
    {
      if ((f[0] | f[1] | f[2] | f[3]) != 0) {  // some row of the block has a new max
        float al[F::NQ];
#pragma unroll
        for (int q = 0; q < F::NQ; ++q) al[q] = f[q >> 1] ? abuf[q * 16 + n] : 1.f;  // row block q: wave q / 2
        mfma_agpr_wait();
#pragma unroll
        for (int c = 0; c < F::NCW; ++c)
#pragma unroll
          for (int q = 0; q < F::NQ; ++q) {  // a few registers at a time
            mfma_agpr_tie(o[c][q]);
            o[c][q] *= al[q];
            mfma_agpr_tie(o[c][q]);
          }
      }
    }
    {
#pragma unroll
      for (int c = 0; c < F::NCW; ++c) {
        const bf16x8 av = a_next;
        if (c + 1 < F::NCW) a_next = cols(tile, cw + 16 * (c + 1));
#pragma unroll
        for (int q = 0; q < F::NQ; ++q) mfma16x16x32_a(o[c][q], av, pq[q]);
      }
    }
    // refill the buffer of tile j - 1 (every wave is past it) while the matrix ops run
    if (j + kFlashBufs - 1 < ntiles)
      dma_tile32<R, COMPACT>(latb, kTileKeys * (j + kFlashBufs - 1), T,
                             lds0 + ((j + kFlashBufs - 1) % kFlashBufs) * TILE, w);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s_cur[kb][qb] = s_next[kb][qb];
    // own part of tile j + 2 landed before the barrier that ends the iteration
    if (j + kFlashBufs - 1 < ntiles)
      dma_wait<NI>();
    else
      dma_wait<0>();
    __builtin_amdgcn_s_barrier();
  }

  // ---- l of every row through LDS, then the normalised rows of this wave's columns
  mfma_agpr_wait();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l_run[qb] + __shfl_xor(l_run[qb], 16);
    lt += __shfl_xor(lt, 32);
    if (G == 0) abuf[(2 * w + qb) * 16 + n] = lt;
  }
  __syncthreads();  // also: every wave is done with the ring, and no copy is in flight
  // The normalised rows are staged in LDS over the ring (rows padded by 16
  // bytes) and stored as whole rows, 16 bytes a lane: stored straight from
  // the accumulators, each store scattered 32-byte pieces over 16 rows and
  // the epilogue took about 16K clocks a block (flash 0.71 -> 0.64 ms at
  // B=8, T=2048, H=16).  The epilogue's lane values are derived afresh from
  // the thread id, so none of them is held across the tile loop.
  constexpr int OS = R * 2 + 16;   // staged row stride, bytes
  constexpr int NCH = R / 8;       // 16-byte chunks of a row
  constexpr int RPI = 64 / NCH;    // rows per store instruction
  int etid = threadIdx.x;          // lane values of the epilogue, derived afresh
  asm volatile("" : "+v"(etid));
  const int elane = etid & 63, eG = elane >> 4, en = elane & 15;
  static_assert(128 * OS <= kFlashBufs * TILE + F::NQ * 1024, "the staged rows fit the ring and the P buffer");
#pragma unroll
  for (int q = 0; q < F::NQ; ++q) {
    const float l = abuf[q * 16 + en];
    const float inv = 1.f / l;
    char* srow = smem + (16 * q + en) * OS + 2 * (cw + 4 * eG);
#pragma unroll
    for (int c = 0; c < F::NCW; ++c) {
      mfma_agpr_tie(o[c][q]);
      // a row with no visible key (l = 0) is NaN, written as such (bf16 quiet NaN bits)
      const uint32_t lo = l > 0.f ? pack_bf16x2(o[c][q][0] * inv, o[c][q][1] * inv) : 0x7fc07fc0u;
      const uint32_t hi = l > 0.f ? pack_bf16x2(o[c][q][2] * inv, o[c][q][3] * inv) : 0x7fc07fc0u;
      *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(srow + 32 * c) = u32x2{lo, hi};
    }
  }
  lds_publish_barrier();
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int rl = 32 * w + k * RPI + elane / NCH, ch = elane % NCH;
    const long row = row0 + rl;
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)(smem + rl * OS + 16 * ch);
    if (row < TH) *(u32x4*)(o_lat + ((size_t)b * TH + row) * R + 8 * ch) = v;
  }
}

// ---------------------------------------------------------------------------
// KV down-projection on the matrix cores (page FW-GLM-5-1 l2_p1, its
// operations list: latent = hidden @ w_down): lat[m, rho] =
// sum_k hid[m, k] w_down[k, rho], computed transposed, lat^T = W^T hid^T,
// from wdT = w_down^T [R][D] so that both operands are rows with contiguous k.
// Block: 128 latent columns (blockIdx.y) x 128 tokens (blockIdx.x); wave w
// owns columns 64 (w & 1) .. + 63 and tokens 64 (w >> 1) .. + 63 as 2 x 2
// tiles of 32 x 32.  k advances 32 at a time through two LDS buffers; the
// next step's operands are loaded into registers while the current step's
// matrix ops run.  Rows are padded to 40 elements (80 bytes), so the eight
// lanes of a 16-byte read hit eight distinct groups of four banks.
constexpr int kDownPad = 40;
__global__ __launch_bounds__(256, 2) void down_bf16(const uint16_t* __restrict__ hid,
                                                    const uint16_t* __restrict__ wdT, uint16_t* __restrict__ lat,
                                                    int M, int D, int R) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][128 * kDownPad];  // W^T rows (latent columns)
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][128 * kDownPad];  // hidden rows (tokens)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * 128, c0 = blockIdx.y * 128;
  u32x4 ra[2], rb[2];
  // chunk ch = tid + 256 i of a 128 x 32 tile: row ch / 4, elements 8 (ch % 4) .. + 7
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i, row = ch >> 2, part = ch & 3;
      ra[i] = *(const u32x4*)(wdT + (size_t)(c0 + row) * D + k0 + 8 * part);
      const int m = m0 + row < M ? m0 + row : M - 1;
      rb[i] = *(const u32x4*)(hid + (size_t)m * D + k0 + 8 * part);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i, row = ch >> 2, part = ch & 3;
      *(u32x4*)&sa[buf][row * kDownPad + 8 * part] = ra[i];
      *(u32x4*)&sb[buf][row * kDownPad + 8 * part] = rb[i];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) acc[i][i2] = f32x16{};
  const int nk = D / 32;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(32 * (kt + 1));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = lds_read16(&sa[buf][(64 * (w & 1) + 32 * i + l32) * kDownPad + 16 * ks + 8 * g]);
        b[i] = lds_read16(&sb[buf][(64 * (w >> 1) + 32 * i + l32) * kDownPad + 16 * ks + 8 * g]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) acc[i][i2] = mfma32x32x16(a[i], b[i2], acc[i][i2]);
    }
    // buffer buf ^ 1 was last read in step kt - 1, before the barrier that ended it
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // acc[i][i2][4 j + v] = lat^T[c0 + 64 (w & 1) + 32 i + 8 j + 4 g + v][m0 + 64 (w >> 1) + 32 i2 + l32]
#pragma unroll
  for (int i2 = 0; i2 < 2; ++i2) {
    const int m = m0 + 64 * (w >> 1) + 32 * i2 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = c0 + 64 * (w & 1) + 32 * i + 8 * j + 4 * g;
        *(u32x2*)(lat + (size_t)m * R + rho) = u32x2{pack_bf16x2(acc[i][i2][4 * j], acc[i][i2][4 * j + 1]),
                                                      pack_bf16x2(acc[i][i2][4 * j + 2], acc[i][i2][4 * j + 3])};
      }
  }
}

bool down_mfma_supported(int D, int r) { return D % 64 == 0 && r % 128 == 0 && r <= 1024; }

size_t down_mfma_workspace(int D, int r) { return ((size_t)D * r * 2 + 255) / 256 * 256; }

// w_down [D, r] -> w_down^T [r, D] in the workspace (the W_uv transpose with
// R = D, H = 1, d = r), then the matrix-core product.
hipError_t down_mfma(const uint16_t* hid, const uint16_t* wd, uint16_t* lat, int M, int D, int r, void* ws,
                     hipStream_t st) {
  uint16_t* wdT = (uint16_t*)ws;
  hipError_t e;
  {
    ProfScope ps("transpose_wv", st);
    e = transpose_wv_launch(wd, wdT, D, 1, r, st);
    if (e != hipSuccess) return e;
  }
  ProfScope ps("down_bf16", st);
  hipLaunchKernelGGL(down_bf16, dim3((M + 127) / 128, r / 128), dim3(256), 0, st, hid, wdT, lat, M, D, r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Key mask -> packed keys.  compact_scan: one block of 1024 per batch walks
// key_mask[b] [T] bytes (nonzero = visible) in chunks of 1024 and writes
// cnt[b][t] = number of visible keys s <= t and src[b][j] = the position of
// the j-th visible key.  compact_gather: one wave per packed row j copies
// latent row src[b][j] of batch b (or zeros for j >= cnt[b][T - 1]).
__global__ __launch_bounds__(1024) void compact_scan(const uint8_t* __restrict__ key_mask,
                                                     int32_t* __restrict__ cnt, int32_t* __restrict__ src, int T) {
  __shared__ int wsum[16];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint8_t* m = key_mask + (size_t)b * T;
  int32_t* cb = cnt + (size_t)b * T;
  int32_t* sb = src + (size_t)b * T;
  int run = 0;  // visible keys before this chunk (block-uniform)
  for (int c0 = 0; c0 < T; c0 += 1024) {
    const int t = c0 + threadIdx.x;
    const bool vis = t < T && m[t] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(vis);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wsum[w] = __builtin_popcountll(bal);
    __syncthreads();
    int before = run;
    for (int i = 0; i < w; ++i) before += wsum[i];
    int total = 0;
    for (int i = 0; i < 16; ++i) total += wsum[i];
    if (t < T) {
      const int k = before + below;  // visible keys before t
      cb[t] = k + (vis ? 1 : 0);
      if (vis) sb[k] = t;
    }
    run += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
}

template <int R>
__global__ __launch_bounds__(256) void compact_gather(const uint16_t* __restrict__ lat, const int32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ src, uint16_t* __restrict__ lat_c,
                                                      int T) {
  static_assert(R % 8 == 0 && R / 8 <= 64, "one 16-byte chunk per lane");
  const int b = blockIdx.y;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= T || lane >= R / 8) return;
  const int nvis = cnt[(size_t)b * T + T - 1];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (j < nvis) v = *(const u32x4*)(lat + ((size_t)b * T + src[(size_t)b * T + j]) * R + 8 * lane);
  *(u32x4*)(lat_c + ((size_t)b * T + j) * R + 8 * lane) = v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
template <int R>
static hipError_t run_prefill(const uint16_t* q, const uint16_t* lat, const uint16_t* wk,
                              const uint16_t* wv, uint16_t* out, int B, int T, int H, int d,
                              float sl2, uint16_t* q_lat, uint16_t* o_lat, uint16_t* wvT,
                              const uint8_t* key_mask, int32_t* cnt, int32_t* src, uint16_t* lat_c,
                              hipStream_t st) {
  const int N = B * T;
  static OnceFlag attrs;
  hipError_t e = run_once(attrs, [] {
    hipError_t r = hipFuncSetAttribute((const void*)flash_latent_bf16<R, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)flash_lds_bytes(R));
    if (r == hipSuccess)
      r = hipFuncSetAttribute((const void*)flash_latent_bf16<R, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)flash_lds_bytes(R));
    if (r == hipSuccess)
      r = hipFuncSetAttribute((const void*)up_bf16<R, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)up_lds_bytes<R>());
    return r;
  });
  if (e != hipSuccess) return e;
  e = absorb_mfma(q, wk, q_lat, N, H, d, R, sl2, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("transpose_wv", st);
    e = transpose_wv_launch(wv, wvT, R, H, d, st);
    if (e != hipSuccess) return e;
  }
  const long TH = (long)T * H;
  const int nrb = (int)((TH + 127) / 128);
  if (key_mask) {
    {
      ProfScope ps("compact_keys", st);
      hipLaunchKernelGGL(compact_scan, dim3(B), dim3(1024), 0, st, key_mask, cnt, src, T);
      hipLaunchKernelGGL(compact_gather<R>, dim3((T + 3) / 4, B), dim3(256), 0, st, lat, cnt, src, lat_c, T);
    }
    ProfScope ps("flash_latent_bf16_masked", st);
    hipLaunchKernelGGL((flash_latent_bf16<R, true>), dim3(B * nrb), dim3(256), flash_lds_bytes(R), st, q_lat, lat_c,
                       o_lat, B, T, H, (const int32_t*)cnt);
  } else {
    ProfScope ps("flash_latent_bf16", st);
    hipLaunchKernelGGL((flash_latent_bf16<R, false>), dim3(B * nrb), dim3(256), flash_lds_bytes(R), st, q_lat, lat,
                       o_lat, B, T, H, (const int32_t*)nullptr);
  }
  {
    ProfScope ps("up_bf16", st);
    const int zb = (d + 127) / 128;
    hipLaunchKernelGGL((up_bf16<R, false>), dim3((N + 32 * kUpRowBlocks - 1) / (32 * kUpRowBlocks), H, zb),
                       dim3(256), up_lds_bytes<R>(), st, o_lat, wvT, out, 1.0f, wvT, out, 1.0f, zb, N, H, d);
  }
  return hipGetLastError();
}

// Workspace: q_lat [B*T*H][r] | o_lat [B*T*H][r] | W_uv^T [H][d][r], all bf16;
// with a key mask, then (at a 256-byte boundary) the packed latents
// [B][T][r] bf16 | cnt [B][T] int32 | src [B][T] int32.
hipError_t prefill_mfma(const void* q, const void* lat, const void* wk, const void* wv, void* out,
                        int B, int T, int H, int d, int r, float sl2, const uint8_t* key_mask, void* ws,
                        hipStream_t st) {
  const size_t rows = (size_t)B * T * H;
  uint16_t* q_lat = (uint16_t*)ws;
  uint16_t* o_lat = q_lat + rows * r;
  uint16_t* wvT = o_lat + rows * r;
  uint16_t* lat_c = (uint16_t*)((char*)ws + prefill_mfma_workspace(B, T, H, d, r));
  int32_t* cnt = (int32_t*)(lat_c + (size_t)B * T * r);
  int32_t* src = cnt + (size_t)B * T;
#define ARGS (const uint16_t*)q, (const uint16_t*)lat, (const uint16_t*)wk, (const uint16_t*)wv, \
             (uint16_t*)out, B, T, H, d, sl2, q_lat, o_lat, wvT, key_mask, cnt, src, lat_c, st
  switch (r) {
    case 128: return run_prefill<128>(ARGS);
    case 256: return run_prefill<256>(ARGS);
    case 512: return run_prefill<512>(ARGS);
  }
#undef ARGS
  return hipErrorInvalidValue;
}

// k and v of every head from the shared latent (the unabsorbed form):
// k[n, h, :] = kscale * latent[n, :] W_uk[:, h, :], v[n, h, :] = latent[n, :] W_uv[:, h, :],
// both [N][H][d] bf16; wkT, wvT: [H][d][R] transposes in the workspace.
template <int R>
static hipError_t run_materialise(const uint16_t* lat, const uint16_t* wk, const uint16_t* wv, uint16_t* k,
                                  uint16_t* v, uint16_t* wkT, uint16_t* wvT, int N, int H, int d, float kscale,
                                  hipStream_t st) {
  static OnceFlag attrs;
  hipError_t e = run_once(attrs, [] {
    return hipFuncSetAttribute((const void*)up_bf16<R, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)up_lds_bytes<R>());
  });
  if (e != hipSuccess) return e;
  {
    ProfScope ps("transpose_wv", st);
    e = transpose_wv_launch(wk, wkT, R, H, d, st);
    if (e == hipSuccess) e = transpose_wv_launch(wv, wvT, R, H, d, st);
    if (e != hipSuccess) return e;
  }
  const int zb = (d + 127) / 128;  // column blocks of one product; k then v along z
  const dim3 grid((N + 32 * kUpRowBlocks - 1) / (32 * kUpRowBlocks), H, 2 * zb);
  {
    ProfScope ps("materialise_kv", st);
    hipLaunchKernelGGL((up_bf16<R, true>), grid, dim3(256), up_lds_bytes<R>(), st, lat, wkT, k, kscale, wvT, v, 1.0f,
                       zb, N, H, d);
  }
  return hipGetLastError();
}

hipError_t materialise_kv(const uint16_t* lat, const uint16_t* wk, const uint16_t* wv, uint16_t* k, uint16_t* v,
                          uint16_t* wkT, uint16_t* wvT, int N, int H, int d, int r, float kscale, hipStream_t st) {
  switch (r) {
    case 128: return run_materialise<128>(lat, wk, wv, k, v, wkT, wvT, N, H, d, kscale, st);
    case 256: return run_materialise<256>(lat, wk, wv, k, v, wkT, wvT, N, H, d, kscale, st);
    case 512: return run_materialise<512>(lat, wk, wv, k, v, wkT, wvT, N, H, d, kscale, st);
  }
  return hipErrorInvalidValue;
}

size_t prefill_mfma_workspace(int B, int T, int H, int d, int r) {
  const size_t rows = (size_t)B * T * H;
  return ((2 * rows * r + (size_t)H * d * r) * 2 + 255) / 256 * 256;
}

size_t key_mask_workspace(int B, int T, int r) { return (size_t)B * T * (8 + 2 * (size_t)r); }

}  // namespace mla
