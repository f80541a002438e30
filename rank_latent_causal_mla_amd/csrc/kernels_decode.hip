// gfx950 decode path: one query per sequence against its cached latents.
//
// Same absorbed formulation as prefill (POPCORNBENCH page FW-GLM-5-1 l2_p31,
// algorithm restatement; the decode query is the last position of its
// sequence and attends keys 0..L_b-1): every head's r-wide query q_lat
// attends the shared latents, the online softmax keeps (m, l, o_lat), and
// o_lat is up-projected per head.  The cache is streamed once from HBM:
//   decode_prep      -- split plan and absorption in one launch;
//   decode_split     -- split-K over balanced chunks of every sequence; each
//                       block writes one partial state per head; blocks past
//                       the split's transpose W_uv for the merge;
//   decode_merge_up  -- log-sum-exp merge of the partial states of each
//                       (b, h), then the W_uv up-projection on the matrix unit.
#include <algorithm>

#include "mla_device.h"
#include "mla_kernels.h"
#include "host_once.h"
#include "lds_tiles.h"
#include "prep_blocks.h"
#include "profile.h"

namespace mla {

constexpr int kDecodeTileKeys = kTileKeys;  // keys per LDS tile of decode_split
constexpr int kDecodeBufs = 4;       // tiles in its LDS ring

// Wait until at most `later` tiles (NI copy instructions of this wave each)
// are still in flight.
template <int NI>
__device__ __forceinline__ void dma_wait_tiles(int later) {
  switch (later) {
    case 0: dma_wait<0>(); break;
    case 1: dma_wait<NI>(); break;
    default: dma_wait<2 * NI>(); break;
  }
}

// Split-K decode over a balanced partition of the concatenated key space.
// The keys of all sequences, one after another (sequence b owns positions
// S[b] .. S[b+1]-1 of the exclusive prefix S of the clamped lengths), are
// cut into P equal chunks of C = ceil(S[B] / P) keys; block (g, hg) takes
// chunk g for head group hg (32 heads) and processes every sequence segment
// in it, writing one partial state (normalised o, m, l) per segment into
// slot g + b.  Every compute unit thus streams the same number of keys.
//
// A segment [k0, k1) of sequence b is streamed through a ring of
// kDecodeBufs block-shared LDS buffers (three in flight while one is read):
// first the query block of sequence b, then its tiles of 32 keys.  The four
// waves share each tile: wave
// w = 2 kb + qb computes the 16 x 16 score block of keys
// 16 kb .. 16 kb + 15 and heads 16 qb .. 16 qb + 15; the row maxima and the
// probabilities P are exchanged through LDS; then wave w accumulates o_lat
// for all 32 heads over its quarter of the latent columns.  Lane l = 16 G + n.
//   scores:  S^T[16 kb + 4 G + v][16 qb + n] in sc[v]                       (16x16x32)
//   output:  O^T[rw + 16 c + 4 G + v][16 q + n] in o[c][q][v], q = 0, 1       (16x16x32, K =
//            the tile's keys in the order 16 t + 4 G + v; A by two transpose reads)
// Every wave tracks the running maxima of all 32 heads (identical in every
// wave) and the partial sum l over its own 16 keys of its 16 heads.
// Blocks 0 .. P * ceil(H / 32) - 1 are the split's (g = index mod P, head group
// index / P); each later block transposes the 64-wide e strip of one head of
// W_uv into W_uv^T for the merge.  Those blocks are dispatched after every
// split block, so they take compute units as the first split blocks finish,
// in the shadow of the slowest ones.
__device__ __forceinline__ int decode_chunk(int N, int P) {
  const int C = (N + P - 1) / P;
  return C < 1 ? 1 : C;
}

template <int R>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_split(const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ lat,
                  const int32_t* __restrict__ S, const int32_t* __restrict__ RB, uint16_t* __restrict__ part_o,
                  float* __restrict__ part_ml, int B, int H, int P, const uint16_t* __restrict__ wv,
                  uint16_t* __restrict__ wvT, int d) {
  constexpr int TILE = kDecodeTileKeys * R * 2;
  constexpr int NI = TILE / 1024 / 4;  // copy instructions per wave and tile
  constexpr int NKS = R / 32;          // contraction steps of a score block
  constexpr int NCW = R / 64;          // 16-column blocks of this wave's quarter
  static_assert(kDecodeBufs == 4, "dma_wait_tiles covers up to 2 later tiles");
  static_assert(NKS % 2 == 0, "two score chains");
  static_assert(R * 128 <= kDecodeBufs * TILE, "a W_uv strip fits the ring");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // after the ring: P [2 q][4 G][16 n][2 kb][4] bf16, maxima [2 kb][2 q][16] f32, l likewise
  char* pbuf = smem + kDecodeBufs * TILE;
  float* mxbuf = (float*)(pbuf + 2048);
  float* lbuf = mxbuf + 64;
  __shared__ int first_seq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w >> 1, qb = w & 1;
  const int G = lane >> 4, n = lane & 15;
  const int nsplit = P * ((H + 31) / 32);
  if ((int)blockIdx.x >= nsplit) {  // block-uniform: a W_uv transpose block
    const int t = blockIdx.x - nsplit, neb = (d + 63) / 64;
    transpose_wv_strip<R>(wv, wvT, H, d, t % neb, t / neb, (uint16_t*)smem);
    return;
  }
  const int g = blockIdx.x % P, hg = blockIdx.x / P;
  const int N = S[B];
  const int C = decode_chunk(N, P);
  const int x0 = (int)min((long long)g * C, (long long)N);
  const int x1 = (int)min((long long)x0 + C, (long long)N);
  if (x0 >= x1) return;  // whole block: chunk past the end
  // sequence holding key x0 (S is nondecreasing with positive steps)
  for (int i = tid; i < B; i += 256)
    if (S[i] <= x0 && x0 < S[i + 1]) first_seq = i;
  __syncthreads();
  const int b_first = __builtin_amdgcn_readfirstlane(first_seq);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  // end of sequence b's part of the chunk, in its own key positions
  auto seg_end = [&](int b) {
    const int sb = __builtin_amdgcn_readfirstlane(S[b]), se = __builtin_amdgcn_readfirstlane(S[b + 1]);
    return (x1 < se ? x1 : se) - sb;
  };
  auto seg_more = [&](int b) { return b < B && __builtin_amdgcn_readfirstlane(S[b]) < x1; };
  const int k_first = x0 - __builtin_amdgcn_readfirstlane(S[b_first]);

  // The chunk as one stream of ring items, segment after segment: the query
  // block of a segment's sequence (its 32 heads' q_lat rows, the same size as
  // a tile and copied the same way), then the segment's 32-key tiles.  The
  // copy cursor runs three items ahead of the compute cursor, across
  // segments.  The queries travel through the ring because a plain load of
  // them would be counted with the copies in flight, and waiting for it
  // would drain the stream at every segment start.
  const int qrows = H - hg * 32 < 32 ? H - hg * 32 : 32;  // heads of this group (rows past it repeat the last)
  int db = b_first, dk = k_first, dend = seg_end(b_first);
  int drb = __builtin_amdgcn_readfirstlane(RB[b_first]);  // first cache row of sequence db
  bool dq = true;  // the next item is the query block of sequence db
  bool ddone = false;
  int issued = 0;
  auto copy_next = [&]() {
    const uint32_t dst = lds0 + (issued % kDecodeBufs) * TILE;
    ++issued;
    if (dq) {
      dma_tile32<R>(q_lat + ((size_t)db * H + hg * 32) * R, 0, qrows, dst, w);
      dq = false;
      return;
    }
    dma_tile32<R, false, true>(lat + (size_t)drb * R, dk, dend, dst, w);  // each cache row is read once
    dk += kDecodeTileKeys;
    if (dk >= dend) {
      ++db;
      if (seg_more(db)) {
        dk = 0;
        dend = seg_end(db);
        drb = __builtin_amdgcn_readfirstlane(RB[db]);
        dq = true;
      } else {
        ddone = true;
      }
    }
  };
  // items 0 .. 3: the first query block is read before the loop, so all four
  // buffers can be in flight at the start
#pragma unroll
  for (int t = 0; t < kDecodeBufs; ++t)
    if (!ddone) copy_next();

  int cb = b_first, ck = k_first, cend = seg_end(b_first);  // compute cursor
  bf16x8 qf[NKS];

  f32x4 o[NCW][2];
  float m_run[2], l_part;
  auto reset = [&]() {
#pragma unroll
    for (int c = 0; c < NCW; ++c) o[c][0] = o[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[0] = m_run[1] = -INFINITY;
    l_part = 0.f;
  };
  reset();
  const int rw = w * (R / 4);

  // per-lane LDS offsets: score row 16 kb + n, transpose key 4 G + n / 4 (+16 t)
  const int fs = tswz(n);
  const int trkey = 4 * G + (n >> 2);
  const int ft = tswz(trkey);
  const int trsub = 8 * (n & 1);
  const int trh = (n & 3) >> 1;
  char* pw = pbuf + ((qb * 4 + G) * 16 + n) * 16 + kb * 8;  // this lane's 4 probabilities
  // this lane's query fragments from a landed query block: row 16 qb + n
  // (tswz(16 + n) = tswz(n)), columns 32 ks + 8 G .. + 7
  auto read_q = [&](const char* qtile) {
    const char* qrow = qtile + (16 * qb + n) * (R * 2);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int c = 4 * ks + G;
      qf[ks] = lds_read16(qrow + 16 * ((c & ~15) | ((c & 15) ^ fs)));
    }
  };

  // partial state of sequence b's segment into slot g + b: l of every head
  // from the two key halves (through LDS), o normalised, (m, l)
  auto flush = [&](int b) {
    float lsum = l_part + __shfl_xor(l_part, 16);
    lsum += __shfl_xor(lsum, 32);
    if (G == 0) lbuf[(kb * 2 + qb) * 16 + n] = lsum;
    lds_publish_barrier();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float lt = lbuf[q * 16 + n] + lbuf[(2 + q) * 16 + n];
      const int hh = hg * 32 + 16 * q + n;
      if (hh >= H) continue;
      const float inv = 1.f / lt;
      const size_t prow = (size_t)(g + b) * H + hh;
      uint16_t* po = part_o + prow * R + rw + 4 * G;
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        const u32x2 v = {pack_bf16x2(o[c][q][0] * inv, o[c][q][1] * inv),
                         pack_bf16x2(o[c][q][2] * inv, o[c][q][3] * inv)};
        *(u32x2*)(po + 16 * c) = v;
      }
      if (w == 0 && G == 0) {
        part_ml[prow * 2] = m_run[q];
        part_ml[prow * 2 + 1] = lt;
      }
    }
  };

  // items 0 (the first query block) and 1 (the first tile) landed; 2 <= issued
  // <= 4 since a segment is never empty
  dma_wait_tiles<NI>(issued - 2);
  __builtin_amdgcn_s_barrier();
  read_q(smem);
  for (int tau = 1;; ++tau) {
    const char* tile = smem + (tau % kDecodeBufs) * TILE;
    const int kt = ck;

    // ---- scores of this wave's block, two interleaved chains
    f32x4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
    {
      const char* arow = tile + (16 * kb + n) * (R * 2);
#pragma unroll
      for (int ks = 0; ks < NKS; ks += 2) {
        const int c0 = 4 * ks + G, c1 = c0 + 4;
        const bf16x8 a0 = lds_read16(arow + 16 * ((c0 & ~15) | ((c0 & 15) ^ fs)));
        const bf16x8 a1 = lds_read16(arow + 16 * ((c1 & ~15) | ((c1 & 15) ^ fs)));
        sc0 = mfma16x16x32(a0, qf[ks], sc0);
        sc1 = mfma16x16x32(a1, qf[ks + 1], sc1);
      }
    }
    // keys >= cend masked: key 16 kb + 4 G + v valid iff v <= lim
    const int lim = cend - 1 - kt - 16 * kb - 4 * G;
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = v > lim ? -INFINITY : sc0[v] + sc1[v];
    {
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = max_xor32(max_xor16(mt));
      if (G == 0) mxbuf[(kb * 2 + qb) * 16 + n] = mt;
    }
    lds_publish_barrier();  // X: maxima posted; every wave is done with item tau - 1
    // refill the buffer of item tau - 1
    if (!ddone) copy_next();
    float m_new[2];
    bool grow_any = false;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float mt = fmaxf(mxbuf[q * 16 + n], mxbuf[(2 + q) * 16 + n]);
      const bool grow = mt > m_run[q] + kRescaleSlack;
      m_new[q] = grow ? mt : m_run[q];
      grow_any |= grow;
    }
    float psum;
    {
      const float mq = qb ? m_new[1] : m_new[0];
      const float msub = mq == -INFINITY ? 0.f : mq;
      const float p0 = fast_exp2(x[0] - msub), p1 = fast_exp2(x[1] - msub);
      const float p2 = fast_exp2(x[2] - msub), p3 = fast_exp2(x[3] - msub);
      psum = (p0 + p1) + (p2 + p3);
      *(u32x2*)pw = u32x2{pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
    }
    // own part of tile tau + 1 landed before the barrier that publishes P
    if (tau + 1 < issued) dma_wait_tiles<NI>(issued - tau - 2);
    lds_publish_barrier();  // Y: P of tile tau complete; tile tau + 1 landed
    if (__builtin_amdgcn_ballot_w64(grow_any)) {  // rare: rescale factors only now
      float alpha[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        alpha[q] = m_new[q] == m_run[q] ? 1.f : fast_exp2(m_run[q] - m_new[q]);
        m_run[q] = m_new[q];
      }
      l_part = l_part * (qb ? alpha[1] : alpha[0]) + psum;
#pragma unroll
      for (int c = 0; c < NCW; ++c)
#pragma unroll
        for (int q = 0; q < 2; ++q) o[c][q] *= alpha[q];
    } else {
      l_part += psum;
    }
    // ---- O^T += L^T P^T over this wave's columns.  Transpose read t of lane
    // (G, n): key 16 t + 4 G + n / 4, columns rw + 16 c + 4 (n % 4) .. + 3.
    bf16x8 Pq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) Pq[q] = lds_read16(pbuf + ((q * 4 + G) * 16 + n) * 16);
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int ch = (rw >> 3) + 2 * c + trh;
      i16x4 a2[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        a2[t] = lds_read_tr16(tile + (16 * t + trkey) * (R * 2) + 16 * ((ch & ~15) | ((ch & 15) ^ ft)) + trsub);
      const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, a2[0])[0],
                                                         __builtin_bit_cast(u32x2, a2[0])[1],
                                                         __builtin_bit_cast(u32x2, a2[1])[0],
                                                         __builtin_bit_cast(u32x2, a2[1])[1]});
      o[c][0] = mfma16x16x32(av, Pq[0], o[c][0]);
      o[c][1] = mfma16x16x32(av, Pq[1], o[c][1]);
    }
    // ---- advance; at the end of a segment, its partial state, then the next
    // segment's query block (item tau + 1) and first tile (item tau + 2)
    ck += kDecodeTileKeys;
    if (ck >= cend) {
      flush(cb);  // its barrier: every wave is done with tile tau
      ++cb;
      if (!seg_more(cb)) break;
      ck = 0;
      cend = seg_end(cb);
      reset();
      if (!ddone) copy_next();  // refill the buffer of tile tau
      // items tau + 1 and tau + 2 exist, so issued >= tau + 3
      dma_wait_tiles<NI>(issued - tau - 3);
      __builtin_amdgcn_s_barrier();
      read_q(smem + ((tau + 1) % kDecodeBufs) * TILE);
      ++tau;
    }
  }
}

// Prologue of a decode call in one launch (independent block roles):
//   block 0          -- the prefix S of the clamped lengths and the row bases RB;
//   the other blocks -- absorption, 32 sequences x 128 rho of one head each.
// (The W_uv transpose runs in the tail of decode_split.)
template <int R, int DK>
__global__ __launch_bounds__(256) void decode_prep(const uint16_t* __restrict__ q, const uint16_t* __restrict__ wk,
                                                   uint16_t* __restrict__ q_lat, const int32_t* __restrict__ lens,
                                                   const int32_t* __restrict__ cu, int B, int Tmax, int H,
                                                   float qscale, int32_t* __restrict__ S, int32_t* __restrict__ RB) {
  constexpr int NQ = R / 128;
  const int bid = blockIdx.x;
  if (bid == 0) {
    length_prefix_block(lens, cu, B, Tmax, S, RB);
  } else {
    const int t = bid - 1;
    absorb_tile<R, DK, 1>(q, wk, q_lat, B, H, qscale, t / (H * NQ), 1, (t / NQ) % H, 128 * (t % NQ));
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Merge + up-projection.  Block (h, group of 16 sequences), 16 waves:
//   o_b = sum_i w_i o_i,  w_i = l_i 2^(m_i - m*) / sum_k l_k 2^(m_k - m*),  m* = max_i m_i
// over the partial states i of sequence b (o_i normalised), then
//   out[b, h, :] = o_b W_uv[:, h, :]   (16 x R times R x d on the matrix unit,
//   W_uv^T [H][d][R] from the prologue).
// Wave v merges sequence b0 + v with lane l owning rho [8 l, 8 l + 8) of
// each 512-wide slice.  Every load of the block -- the partial states, their
// (m, l) and the up-projection operands -- is issued at the start, so the
// kernel costs about one memory round trip.
constexpr int kMergePrefetch = 8;  // partial states of a sequence loaded up front
template <int R>
__global__ __launch_bounds__(1024) void decode_merge_up(const uint16_t* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        const int32_t* __restrict__ S,
                                                        const uint16_t* __restrict__ wvT,
                                                        uint16_t* __restrict__ out, int B, int H, int d, int P) {
  constexpr int NKS = R / 32;   // contraction steps of the up-projection
  constexpr int NC = R / 512 > 0 ? R / 512 : 1;  // 8-wide rho chunks per lane
  constexpr int LANES = R / (8 * NC);            // lanes that hold rho (R < 512: fewer)
  __shared__ __attribute__((aligned(16))) uint16_t ob[16][R + 8];
  const int h = blockIdx.x, b0 = blockIdx.y * 16;
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, n = lane & 15;
  const int neb = d / 16;

  // up-projection operands of this wave's output block
  bf16x8 wa[NKS];
  if (v < neb) {
    const uint16_t* wrow = wvT + ((size_t)h * d + 16 * v + n) * R + 8 * G;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wa[ks] = *(const bf16x8*)(wrow + 32 * ks);
  }
  // partial slots of sequence b: g + b for the chunks g that hold its keys
  const int b = b0 + v;
  int base = 0, cnt = 0;
  if (b < B) {
    const int C = decode_chunk(S[B], P);
    const int sb = S[b], se = S[b + 1];
    const int g0 = sb / C, g1 = (se - 1) / C;
    base = g0 + b;
    cnt = g1 - g0 + 1;
  }
  base = __builtin_amdgcn_readfirstlane(base);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  // partial states 0 .. kMergePrefetch - 1 and the (m, l) of splits lane, lane + 64, ...
  u32x4 po[kMergePrefetch][NC];
#pragma unroll
  for (int j = 0; j < kMergePrefetch; ++j)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      po[j][c] = j < cnt && lane < LANES
                     ? *(const u32x4*)(part_o + ((size_t)(base + j) * H + h) * R + 8 * (lane + 64 * c))
                     : u32x4{0, 0, 0, 0};
  float2 ml0 = lane < cnt ? *(const float2*)(part_ml + ((size_t)(base + lane) * H + h) * 2) : float2{-INFINITY, 0.f};
  float m = ml0.x;
  for (int j = lane + 64; j < cnt; j += 64) m = fmaxf(m, part_ml[((size_t)(base + j) * H + h) * 2]);
  m = wave_max(m);
  float ls = lane < cnt ? ml0.y * exp2f(ml0.x - m) : 0.f;
  for (int j = lane + 64; j < cnt; j += 64) {
    const float2 ml = *(const float2*)(part_ml + ((size_t)(base + j) * H + h) * 2);
    ls += ml.y * exp2f(ml.x - m);
  }
  ls = wave_sum(ls);
  const float inv = ls > 0.f ? 1.f / ls : 0.f;
  const float wl = lane < cnt ? ml0.y * exp2f(ml0.x - m) * inv : 0.f;  // weight of split `lane`
  float acc[8 * NC];
#pragma unroll
  for (int i = 0; i < 8 * NC; ++i) acc[i] = 0.f;
  auto add = [&](float wt, const u32x4 (&x)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[8 * c + 2 * e] += wt * __uint_as_float(x[c][e] << 16);
        acc[8 * c + 2 * e + 1] += wt * __uint_as_float(x[c][e] & 0xFFFF0000u);
      }
  };
#pragma unroll
  for (int j = 0; j < kMergePrefetch; ++j)
    if (j < cnt) add(__shfl(wl, j), po[j]);
  for (int j = kMergePrefetch; j < cnt; ++j) {  // rare: more partial states than prefetched
    const float2 ml = *(const float2*)(part_ml + ((size_t)(base + j) * H + h) * 2);
    u32x4 x[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      x[c] = lane < LANES ? *(const u32x4*)(part_o + ((size_t)(base + j) * H + h) * R + 8 * (lane + 64 * c))
                          : u32x4{0, 0, 0, 0};
    add(ml.y * exp2f(ml.x - m) * inv, x);
  }
  if (lane < LANES)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *(u32x4*)&ob[v][8 * (lane + 64 * c)] =
          u32x4{pack_bf16x2(acc[8 * c], acc[8 * c + 1]), pack_bf16x2(acc[8 * c + 2], acc[8 * c + 3]),
                pack_bf16x2(acc[8 * c + 4], acc[8 * c + 5]), pack_bf16x2(acc[8 * c + 6], acc[8 * c + 7])};
  __syncthreads();
  // out^T[e][b] = sum_rho W_uv^T[e][rho] o[b][rho]: A = W_uv^T (e rows), B = o^T
  if (v < neb) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ks += 2) {
      a0 = mfma16x16x32(wa[ks], *(const bf16x8*)&ob[n][32 * ks + 8 * G], a0);
      a1 = mfma16x16x32(wa[ks + 1], *(const bf16x8*)&ob[n][32 * ks + 32 + 8 * G], a1);
    }
    // (a0 + a1)[u] = out^T[e = 16 v + 4 G + u][b = b0 + n]
    if (b0 + n < B) {
      uint16_t* dst = out + ((size_t)(b0 + n) * H + h) * d + 16 * v + 4 * G;
      *(u32x2*)dst = u32x2{pack_bf16x2(a0[0] + a1[0], a0[1] + a1[1]), pack_bf16x2(a0[2] + a1[2], a0[3] + a1[3])};
    }
  }
}

// ---------------------------------------------------------------------------
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::atomic<int>* slot = dev >= 0 && dev < kMaxDevices ? &cache[dev] : nullptr;
  if (slot) {
    const int c = slot->load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (slot) slot->store(cus, std::memory_order_relaxed);  // racing callers store the same value
  return cus;
}

namespace {
std::atomic<int> g_decode_splits{0};
}  // namespace
int decode_splits_override() { return g_decode_splits.load(std::memory_order_relaxed); }
void set_decode_splits(int p) { g_decode_splits.store(p, std::memory_order_relaxed); }

size_t decode_max_splits(int B) { return (size_t)decode_split_cap() + B; }

int decode_chunks(int H) {
  // one chunk of keys per compute unit over all head groups (or the count set
  // by mla_decode_set_splits)
  const int nhg = (H + 31) / 32;
  const int forced = decode_splits_override();
  const int P = forced > 0 ? forced : device_cus() / nhg;
  return P < 1 ? 1 : (P > decode_split_cap() ? decode_split_cap() : P);
}

template <int R>
static hipError_t run_decode(const uint16_t* q, const uint16_t* lat, const int32_t* lens, const int32_t* cu,
                             const uint16_t* wk, const uint16_t* wv, uint16_t* out, int B, int Tmax,
                             int H, int d, float sl2, uint16_t* q_lat, uint16_t* part_o, float* part_ml,
                             uint16_t* wvT, int32_t* S, int32_t* RB, int P, hipStream_t st) {
  const int nhg = (H + 31) / 32;
  const size_t lds = decode_lds_bytes(R);
  static OnceFlag attrs;
  const hipError_t e = run_once(attrs, [lds] {
    return hipFuncSetAttribute((const void*)decode_split<R>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (e != hipSuccess) return e;
  {
    ProfScope ps("decode_prep", st);
    const int nabs = ((B + 31) / 32) * H * (R / 128);
    const dim3 grid(1 + nabs);
#define PREP(DK)                                                                                               \
  hipLaunchKernelGGL((decode_prep<R, DK>), grid, dim3(256), 0, st, q, wk, q_lat, lens, cu, B, Tmax, H, sl2, S, \
                     RB)
    switch (d) {
      case 32: PREP(2); break;
      case 64: PREP(4); break;
      case 128: PREP(8); break;
      case 256: PREP(16); break;
      default: return hipErrorInvalidValue;
    }
#undef PREP
  }
  {
    ProfScope ps("decode_split", st);
    const int ntr = ((d + 63) / 64) * H;  // one W_uv transpose block per head and 64-wide e strip
    hipLaunchKernelGGL(decode_split<R>, dim3(P * nhg + ntr), dim3(256), lds, st, q_lat, lat, S, RB, part_o, part_ml,
                       B, H, P, wv, wvT, d);
  }
  {
    ProfScope ps("decode_merge_up", st);
    hipLaunchKernelGGL(decode_merge_up<R>, dim3(H, (B + 15) / 16), dim3(1024), 0, st, part_o, part_ml, S, wvT, out,
                       B, H, d, P);
  }
  return hipGetLastError();
}

// Workspace: q_lat [B*H][r] bf16 | W_uv^T [H][d][r] | partial o [M][H][r] bf16 |
// partial (m, l) [M][H][2] f32 | length prefix [B + 1] int32 | row bases [B] int32, with
// M partial slots (chunk g of sequence b writes slot g + b, so M >= chunks + B);
// each part 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_mfma_bytes(int B, int H, int d, int r, size_t slots) {
  const size_t M = slots;
  size_t bytes = align256((size_t)B * H * r * 2);
  bytes = align256(bytes + (size_t)H * d * r * 2);
  bytes = align256(bytes + M * H * r * 2);
  bytes = align256(bytes + M * H * 2 * 4);
  bytes += (size_t)(B + 1) * 4 + (size_t)B * 4;
  return bytes;
}

size_t decode_mfma_workspace(int B, int Tmax, int H, int d, int r) {
  (void)Tmax;
  return decode_mfma_bytes(B, H, d, r, decode_max_splits(B));
}

hipError_t decode_mfma(const void* q, const void* lat, const int32_t* lens, const int32_t* cu, const void* wk,
                       const void* wv, void* out, int B, int Tmax, int H, int d, int r, float sl2,
                       void* ws, size_t slots, hipStream_t st) {
  const size_t M = slots;
  // chunks per head group, within the slots the workspace was laid out for
  const int P = (int)std::min<size_t>((size_t)decode_chunks(H), slots - (size_t)B);
  char* p = (char*)ws;
  uint16_t* q_lat = (uint16_t*)p;
  size_t off = align256((size_t)B * H * r * 2);
  uint16_t* wvT = (uint16_t*)(p + off);
  off = align256(off + (size_t)H * d * r * 2);
  uint16_t* part_o = (uint16_t*)(p + off);
  off = align256(off + M * H * r * 2);
  float* part_ml = (float*)(p + off);
  off = align256(off + M * H * 2 * 4);
  int32_t* S = (int32_t*)(p + off);
  int32_t* RB = S + B + 1;
#define ARGS (const uint16_t*)q, (const uint16_t*)lat, lens, cu, (const uint16_t*)wk, (const uint16_t*)wv, \
             (uint16_t*)out, B, Tmax, H, d, sl2, q_lat, part_o, part_ml, wvT, S, RB, P, st
  switch (r) {
    case 128: return run_decode<128>(ARGS);
    case 256: return run_decode<256>(ARGS);
    case 512: return run_decode<512>(ARGS);
  }
#undef ARGS
  return hipErrorInvalidValue;
}

}  // namespace mla
