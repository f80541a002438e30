// Block bodies shared by the prefill kernels and the fused decode prologue:
// weight absorption, the W_uv transpose and the prefix of the decode lengths.  Each is
// the work of one 256-thread block, given its block coordinates.
#pragma once

#include "mla_device.h"

namespace mla {

// Absorption: q_lat[n*H + h, rho] = qscale * sum_e W_uk[rho, h, e] * q[n, h, e]
// (n = b*T + t; qscale folds the softmax scale and log2 e into q_lat).
// Computed transposed, q_lat^T = W_h q_h^T, so each lane ends with 4
// consecutive rho of one query row.  The block covers head h, the rank slice
// [rho_base, rho_base + 128 NB) (wave w takes 32 NB of those rho, its slice
// of W_uk held in registers) and the row blocks nb0 .. nb0 + nbn - 1 of 32
// query rows each, so W_uk is read once per block.  DK = d / 16 steps of
// the contraction.
template <int R, int DK, int NB>
__device__ __forceinline__ void absorb_tile(const uint16_t* __restrict__ q, const uint16_t* __restrict__ wk,
                                            uint16_t* __restrict__ q_lat, int N, int H, float qscale, int nb0,
                                            int nbn, int h, int rho_base) {
  constexpr int d = 16 * DK;
  static_assert(NB * DK <= 32, "the W_uk slice fits 128 registers");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int rho0 = rho_base + w * 32 * NB;
  bf16x8 a[NB][DK];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint16_t* wrow = wk + ((size_t)(rho0 + 32 * i + l32) * H + h) * d + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) a[i][ks] = *(const bf16x8*)(wrow + 16 * ks);
  }
  for (int nb = nb0; nb < nb0 + nbn && nb * 32 < N; ++nb) {
    const int n = nb * 32 + l32;
    const int nc = min(n, N - 1);
    const uint16_t* qrow = q + ((size_t)nc * H + h) * d + 8 * g;
    bf16x8 bq[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) bq[ks] = *(const bf16x8*)(qrow + 16 * ks);
    f32x16 acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      acc[i] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) acc[i] = mfma32x32x16(a[i][ks], bq[ks], acc[i]);
    }
    if (n < N) {
      uint16_t* orow = q_lat + ((size_t)n * H + h) * R;
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rho = rho0 + 32 * i + 8 * j + 4 * g;
          u32x2 v = {pack_bf16x2(acc[i][4 * j] * qscale, acc[i][4 * j + 1] * qscale),
                     pack_bf16x2(acc[i][4 * j + 2] * qscale, acc[i][4 * j + 3] * qscale)};
          *(u32x2*)(orow + rho) = v;
        }
    }
  }
}

// W_uv [R, H, d] -> W_uv^T [H, d, R], so the up-projection reads rho-contiguous
// rows.  The block transposes the 64 x 64 tile (rho block rb, e block eb) of
// head h through the LDS array `tile` (16-byte aligned), reading and writing
// 16-byte pieces (d and R are multiples of 32 and 64 on this path; e past d
// is skipped).
constexpr int kTransposeTile = 64;
typedef uint16_t TransposeRow[kTransposeTile + 8];
__device__ __forceinline__ void transpose_wv_tile(const uint16_t* __restrict__ wv, uint16_t* __restrict__ wvT,
                                                  int R, int H, int d, int rb, int eb, int h,
                                                  TransposeRow* tile) {
  const int rho0 = rb * 64, e0 = eb * 64;
  const int tid = threadIdx.x;
  // read: 64 rho rows x 8 pieces of 8 e
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k, r = idx >> 3, c = idx & 7;
    const int e = e0 + 8 * c;
    u32x4 v = {0, 0, 0, 0};
    if (e < d) v = *(const u32x4*)(wv + ((size_t)(rho0 + r) * H + h) * d + e);
    *(u32x4*)&tile[r][8 * c] = v;
  }
  __syncthreads();
  // write: 64 e rows x 8 pieces of 8 rho
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 256 * k, er = idx >> 3, c = idx & 7;
    const int e = e0 + er;
    if (e >= d) continue;
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w4[i] = (uint32_t)tile[8 * c + 2 * i][er] | ((uint32_t)tile[8 * c + 2 * i + 1][er] << 16);
    *(u32x4*)(wvT + ((size_t)h * d + e) * R + rho0 + 8 * c) = u32x4{w4[0], w4[1], w4[2], w4[3]};
  }
}

// The same transpose for all R rho of head h and e in [64 eb, 64 eb + 64),
// every load in flight before the first LDS write, through `tile` (R x 128
// bytes of LDS, 16-byte aligned).  Piece (rho, c) of 8 e sits at chunk
// c ^ ((rho / 8) % 8) of its 128-byte row, so both the row writes and the
// column reads below are free of bank conflicts; each store instruction
// writes 8 W_uv^T rows x 128 contiguous bytes.
template <int R>
__device__ __forceinline__ void transpose_wv_strip(const uint16_t* __restrict__ wv, uint16_t* __restrict__ wvT,
                                                   int H, int d, int eb, int h, uint16_t* tile) {
  constexpr int NP = R * 8 / 256;  // 16-byte pieces per thread, R rows x 8 pieces
  const int e0 = eb * 64, tid = threadIdx.x;
  u32x4 v[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int idx = tid + 256 * k, r = idx >> 3, c = idx & 7;
    const int e = e0 + 8 * c;
    v[k] = e < d ? *(const u32x4*)(wv + ((size_t)r * H + h) * d + e) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int idx = tid + 256 * k, r = idx >> 3, c = idx & 7;
    *(u32x4*)(tile + r * 64 + 8 * (c ^ ((r >> 3) & 7))) = v[k];
  }
  __syncthreads();
  // output pieces: e row er, rho [8 c, 8 c + 8); a wave takes 8 rows x 8 pieces
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int idx = tid + 256 * k, grp = idx >> 6, l = idx & 63;
    const int er = 8 * (grp & 7) + (l >> 3), c = 8 * (grp >> 3) + (l & 7);
    const int e = e0 + er;
    if (e >= d) continue;
    const uint16_t* col = tile + 8 * ((er >> 3) ^ (c & 7)) + (er & 7);
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w4[i] = (uint32_t)col[(8 * c + 2 * i) * 64] | ((uint32_t)col[(8 * c + 2 * i + 1) * 64] << 16);
    *(u32x4*)(wvT + ((size_t)h * d + e) * R + 8 * c) = u32x4{w4[0], w4[1], w4[2], w4[3]};
  }
}

__device__ __forceinline__ int clamp_len(int L, int Tmax) { return L < 1 ? 1 : (L > Tmax ? Tmax : L); }

// Where each decode sequence's latents start and how many it has (one
// 256-thread block): RB[b] is its first cache row and S the exclusive prefix
// of the lengths (S[B] = the total).  Padded cache [B, Tmax, r]: RB[b] =
// b Tmax and the length clamp(lens[b], 1, Tmax).  Packed cache [total, r]
// (cu != nullptr, `Tmax` = total): RB[b] = clamp(cu[b], 0, total - 1) and the
// length clamp(cu[b + 1] - cu[b], 1, total - RB[b]), so every row read is a
// row of the cache whatever cu holds.
__device__ __forceinline__ void length_prefix_block(const int32_t* __restrict__ lens,
                                                    const int32_t* __restrict__ cu, int B, int Tmax,
                                                    int32_t* __restrict__ S, int32_t* __restrict__ RB) {
  auto len = [&](int b) {
    if (!cu) {
      RB[b] = b * Tmax;
      return clamp_len(lens[b], Tmax);
    }
    const int c0 = cu[b], c1 = cu[b + 1];
    const int base = c0 < 0 ? 0 : (c0 > Tmax - 1 ? Tmax - 1 : c0);
    RB[b] = base;
    return clamp_len(c1 - c0, Tmax - base);
  };
  __shared__ int scan[256];
  __shared__ int carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + tid;
    const int L = b < B ? len(b) : 0;
    scan[tid] = L;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive Hillis-Steele scan
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (b < B) S[b] = carry + scan[tid] - L;
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  if (tid == 0) S[B] = carry;
}

}  // namespace mla
