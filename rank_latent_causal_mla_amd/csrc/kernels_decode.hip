// gfx950 decode path: one query per sequence against its cached latents.
//
// Same absorbed formulation as prefill (POPCORNBENCH page FW-GLM-5-1 l2_p31,
// algorithm restatement; the decode query is the last position of its
// sequence and attends keys 0..L_b-1): every head's r-wide query q_lat
// attends the shared latents, the online softmax keeps (m, l, o_lat), and
// o_lat is up-projected per head.  The cache is streamed once from HBM:
//   decode_split     -- split-K over balanced chunks of every sequence; each
//                       block writes one partial state per head;
//   decode_merge_up  -- log-sum-exp merge of the partial states of each
//                       (b, h), then the W_uv up-projection on the matrix unit.
#include "mla_device.h"
#include "mla_kernels.h"
#include "profile.h"

namespace mla {

constexpr int kDecodeTileKeys = 32;  // keys per LDS tile of decode_split
constexpr int kDecodeBufs = 4;       // tiles in its LDS ring

// Balanced split of the ragged cache, computed on the device from the
// device-resident lengths (one block): chunk C (a multiple of the 32-key
// tile) is the smallest with sum_b ceil(L_b / C) <= target + B.  Sequence b
// owns splits base_b .. base_b + cnt_b - 1; split s covers keys [k0, k1) of
// sequence table[s].x (-1 past the last split).
__device__ __forceinline__ int clamp_len(int L, int Tmax) { return L < 1 ? 1 : (L > Tmax ? Tmax : L); }

__global__ __launch_bounds__(1024) void decode_plan(const int32_t* __restrict__ lens, int B, int Tmax,
                                                    int target, int max_splits, int4* __restrict__ table,
                                                    int2* __restrict__ seqinfo) {
  __shared__ long long red[1024];
  __shared__ int scan[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  long long part = 0;
  for (int b = tid; b < B; b += 1024) part += clamp_len(lens[b], Tmax);
  red[tid] = part;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  long long C = (red[0] + target - 1) / target;
  C = (C + kDecodeTileKeys - 1) / kDecodeTileKeys * kDecodeTileKeys;
  if (C < kDecodeTileKeys) C = kDecodeTileKeys;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 1024) {
    const int b = b0 + tid;
    const int L = b < B ? clamp_len(lens[b], Tmax) : 0;
    const int n = b < B ? (int)((L + C - 1) / C) : 0;
    scan[tid] = n;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int base = carry + scan[tid] - n;
    if (b < B) {
      seqinfo[b] = int2{base, n};
      for (int i = 0; i < n; ++i) {
        const int k0 = (int)(i * C);
        const int k1 = (int)((i + 1) * C) < L ? (int)((i + 1) * C) : L;
        table[base + i] = int4{b, k0, k1, 0};
      }
    }
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  for (int s2 = carry + tid; s2 < max_splits; s2 += 1024) table[s2] = int4{-1, 0, 0, 0};
}

// LDS-DMA copy of 16 bytes per lane (lane l: gptr -> LDS byte lds_base + 16 l).
// Issued as inline assembly: the compiler then cannot pair every later LDS
// transpose read with a wait for all copies in flight (it cannot tell which
// LDS bytes a copy writes), which would serialise the prefetch.  The kernel
// orders copies and reads itself with dma_wait<n>().
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
// Wait until at most n of this wave's vector-memory operations are outstanding.
template <int n>
__device__ __forceinline__ void dma_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(n) : "memory");
}

// Block-shared tile of 32 keys, row-major, 16-byte chunks XOR-swizzled by
// tswz(key) inside every 16-chunk group:
//   - score reads (16 lanes = 16 consecutive keys, one chunk each) hit 16
//     distinct slots because tswz is a permutation of 0..15 on key % 16;
//   - transpose reads (32 lanes = 8 consecutive keys x one chunk pair) hit 16
//     distinct slots because tswz(key) >> 1 is a permutation of key % 8.
__device__ __forceinline__ int tswz(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }

// Wave w's share of the LDS-DMA copy of one tile: instructions i = w, w + 4, ...
// of the tile's 32 R * 2 / 1024, each 64 lanes x 16 bytes.  The swizzle is
// applied on the global side: LDS-DMA writes lane l to byte 16 l of its
// 1 KB destination, so lane l fetches the chunk that belongs there.
template <int R>
__device__ __forceinline__ void dma_tile32(const uint16_t* latb, int k0, int kend, uint32_t tile, int w) {
  constexpr int NC = R / 8;                                   // chunks per key row
  constexpr int NI = kDecodeTileKeys * R * 2 / 1024 / 4;      // instructions per wave
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ins = 4 * i + w;
    const int idx = ins * 64 + lane;
    const int s = idx / NC, p = idx % NC;
    const int c = (p & ~15) | ((p & 15) ^ tswz(s));
    const int key = k0 + s < kend ? k0 + s : kend - 1;
    dma16(latb + (size_t)key * R + 8 * c, tile + ins * 1024);
  }
}

template <int NI>
__device__ __forceinline__ void dma_wait_tiles(int later) {
  // at most `later` tiles (NI instructions each) of this wave still in flight
  switch (later) {
    case 0: dma_wait<0>(); break;
    case 1: dma_wait<NI>(); break;
    case 2: dma_wait<2 * NI>(); break;
    default: dma_wait<3 * NI>(); break;
  }
}

// Split-K decode.  Block (split s, head group hg of 32 heads); the split is a
// contiguous key range [k0, k1) of one sequence b, streamed through a ring of
// kDecodeBufs block-shared LDS tiles of 32 keys.  The four waves share each
// tile: wave w = 2 kb + qb computes the 16 x 16 score block of keys
// 16 kb .. 16 kb + 15 and heads 16 qb .. 16 qb + 15; the row maxima and the
// probabilities P are exchanged through LDS; then wave w accumulates o_lat
// for all 32 heads over its quarter of the latent columns.  Lane l = 16 G + n.
//   scores:  S^T[16 kb + 4 G + v][16 qb + n] in sc[v]                       (16x16x32)
//   output:  O^T[rw + 16 c + 4 G + v][16 q + n] in o[c][q][v], q = 0, 1       (16x16x32, K =
//            the tile's keys in the order 16 t + 4 G + v; A by two transpose reads)
// Every wave tracks the running maxima of all 32 heads (identical in every
// wave) and the partial sum l over its own 16 keys of its 16 heads.
template <int R>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_split(const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ lat,
                  const int4* __restrict__ table, uint16_t* __restrict__ part_o,
                  float* __restrict__ part_ml, int Tmax, int H) {
  constexpr int TILE = kDecodeTileKeys * R * 2;
  constexpr int NI = TILE / 1024 / 4;
  constexpr int NKS = R / 32;       // contraction steps of a score block
  constexpr int NCW = R / 64;       // 16-column blocks of this wave's quarter
  static_assert(kDecodeBufs - 2 <= 3, "dma_wait_tiles covers up to 3 later tiles");
  static_assert(NKS % 2 == 0, "two score chains");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // after the ring: P [2 q][4 G][16 n][2 kb][4] bf16, maxima [2 kb][2 q][16] f32
  char* pbuf = smem + kDecodeBufs * TILE;
  float* mxbuf = (float*)(pbuf + 2048);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w >> 1, qb = w & 1;
  const int G = lane >> 4, n = lane & 15;
  const int s = blockIdx.x, hg = blockIdx.y;
  const int4 sp = table[s];
  const int b = __builtin_amdgcn_readfirstlane(sp.x);
  if (b < 0) return;  // whole block: no split left
  const int k0 = __builtin_amdgcn_readfirstlane(sp.y), k1 = __builtin_amdgcn_readfirstlane(sp.z);
  const int ntile = (k1 - k0 + kDecodeTileKeys - 1) / kDecodeTileKeys;
  const uint16_t* latb = lat + (size_t)b * Tmax * R;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  // first tiles in flight while the queries load
#pragma unroll
  for (int t = 0; t < kDecodeBufs - 1; ++t)
    if (t < ntile) dma_tile32<R>(latb, k0 + kDecodeTileKeys * t, k1, lds0 + t * TILE, w);
  bf16x8 qf[NKS];
  {
    const int hh = hg * 32 + 16 * qb + n;
    const uint16_t* qrow = q_lat + ((size_t)b * H + (hh < H ? hh : H - 1)) * R + 8 * G;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qrow + 32 * ks);
  }
  // Consume the query registers before the loop: the copies are invisible
  // to the compiler's wait counting, and a query load still pending at the
  // loop head would make it wait on the vector-memory counter every iteration.
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : : "v"(qf[ks]));

  f32x4 o[NCW][2];
#pragma unroll
  for (int c = 0; c < NCW; ++c) o[c][0] = o[c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_part = 0.f;
  const int rw = w * (R / 4);

  // per-lane LDS offsets: score row 16 kb + n, transpose key 4 G + n / 4 (+16 t)
  const int fs = tswz(n);
  const int trkey = 4 * G + (n >> 2);
  const int ft = tswz(trkey);
  const int trsub = 8 * (n & 1);
  const int trh = (n & 3) >> 1;
  char* pw = pbuf + ((qb * 4 + G) * 16 + n) * 16 + kb * 8;  // this lane's 4 probabilities

  if (ntile > 0) {
    dma_wait_tiles<NI>(ntile - 1 < kDecodeBufs - 2 ? ntile - 1 : kDecodeBufs - 2);
    __builtin_amdgcn_s_barrier();  // tile 0 landed for every wave
  }
  for (int j = 0; j < ntile; ++j) {
    const char* tile = smem + (j % kDecodeBufs) * TILE;
    const int kt = k0 + kDecodeTileKeys * j;

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
    // keys >= k1 masked: key 16 kb + 4 G + v valid iff v <= lim
    const int lim = k1 - 1 - kt - 16 * kb - 4 * G;
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = v > lim ? -INFINITY : sc0[v] + sc1[v];
    {
      float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mt = max_xor32(max_xor16(mt));
      if (G == 0) mxbuf[(kb * 2 + qb) * 16 + n] = mt;
    }
    __builtin_amdgcn_s_barrier();  // X: maxima posted; every wave is done with tile j - 1
    // refill the buffer of tile j - 1
    if (j + kDecodeBufs - 1 < ntile)
      dma_tile32<R>(latb, k0 + kDecodeTileKeys * (j + kDecodeBufs - 1), k1,
                    lds0 + ((j + kDecodeBufs - 1) % kDecodeBufs) * TILE, w);
    float alpha[2];
    bool grow_any = false;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float mt = fmaxf(mxbuf[q * 16 + n], mxbuf[(2 + q) * 16 + n]);
      const bool grow = mt > m_run[q] + kRescaleSlack;
      alpha[q] = grow ? fast_exp2(m_run[q] - mt) : 1.f;
      m_run[q] = grow ? mt : m_run[q];
      grow_any |= grow;
    }
    {
      const float mq = qb ? m_run[1] : m_run[0];
      const float msub = mq == -INFINITY ? 0.f : mq;
      const float p0 = fast_exp2(x[0] - msub), p1 = fast_exp2(x[1] - msub);
      const float p2 = fast_exp2(x[2] - msub), p3 = fast_exp2(x[3] - msub);
      l_part = l_part * (qb ? alpha[1] : alpha[0]) + ((p0 + p1) + (p2 + p3));
      *(u32x2*)pw = u32x2{pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
    }
    // own part of tile j + 1 landed before the barrier that publishes P
    if (j + 1 < ntile) {
      const int last = j + kDecodeBufs - 1 < ntile - 1 ? j + kDecodeBufs - 1 : ntile - 1;
      dma_wait_tiles<NI>(last - (j + 1));
    }
    __builtin_amdgcn_s_barrier();  // Y: P of tile j complete; tile j + 1 landed
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
      mfma_agpr_wait();
#pragma unroll
      for (int c = 0; c < NCW; ++c)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          mfma_agpr_tie(o[c][q]);
          o[c][q] *= alpha[q];
          mfma_agpr_tie(o[c][q]);
        }
    }
    // ---- O^T += L^T P^T over this wave's columns.  Transpose read t of lane
    // (G, n): key 16 t + 4 G + n / 4, columns rw + 16 c + 4 (n % 4) .. + 3.
    bf16x8 P[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) P[q] = lds_read16(pbuf + ((q * 4 + G) * 16 + n) * 16);
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
      mfma16x16x32_a(o[c][0], av, P[0]);
      mfma16x16x32_a(o[c][1], av, P[1]);
    }
  }

  // ---- l of every head: partial sums of the two key halves through LDS
  float lsum = l_part + __shfl_xor(l_part, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with the P and maxima buffers
  if (G == 0) mxbuf[(kb * 2 + qb) * 16 + n] = lsum;
  __syncthreads();
  mfma_agpr_wait();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float lt = mxbuf[q * 16 + n] + mxbuf[(2 + q) * 16 + n];
    const int hh = hg * 32 + 16 * q + n;
    if (hh >= H) continue;
    const float inv = 1.f / lt;
    const size_t prow = (size_t)s * H + hh;
    uint16_t* po = part_o + prow * R + rw + 4 * G;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      mfma_agpr_tie(o[c][q]);
      const u32x2 v = {pack_bf16x2(o[c][q][0] * inv, o[c][q][1] * inv),
                       pack_bf16x2(o[c][q][2] * inv, o[c][q][3] * inv)};
      *(u32x2*)(po + 16 * c) = v;
    }
    if (w == 0 && G == 0) {
      part_ml[prow * 2] = m_run[q];
      part_ml[prow * 2 + 1] = lt;
    }
  }
}

// Merge + up-projection.  Block (h, group of 16 sequences):
//   o_b = sum_i w_i o_i / sum_i w_i,  w_i = l_i 2^(m_i - m*),  m* = max_i m_i
// over the splits i of sequence b (o_i normalised), then
//   out[b, h, :] = o_b W_uv[:, h, :]   (16 x R times R x d on the matrix unit,
//   W_uv^T [H][d][R] from transpose_wv).
template <int R>
__global__ __launch_bounds__(256) void decode_merge_up(const uint16_t* __restrict__ part_o,
                                                       const float* __restrict__ part_ml,
                                                       const int2* __restrict__ seqinfo,
                                                       const uint16_t* __restrict__ wvT,
                                                       uint16_t* __restrict__ out, int B, int H, int d) {
  __shared__ __attribute__((aligned(16))) uint16_t ob[16][R + 8];
  __shared__ float mst[16], winv[16];
  const int h = blockIdx.x, b0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  // per-sequence max and weight sum: one lane group of 16 per sequence
  if (tid < 256) {
    const int i = tid >> 4, k = tid & 15;  // sequence b0 + i, splits k, k + 16, ...
    const int b = b0 + i;
    float mx = -INFINITY;
    int2 si = int2{0, 0};
    if (b < B) si = seqinfo[b];
    for (int j = k; j < si.y; j += 16) mx = fmaxf(mx, part_ml[((size_t)(si.x + j) * H + h) * 2]);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float ws = 0.f;
    for (int j = k; j < si.y; j += 16) {
      const size_t pr = (size_t)(si.x + j) * H + h;
      ws += part_ml[pr * 2 + 1] * exp2f(part_ml[pr * 2] - mx);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
    if (k == 0) {
      mst[i] = mx;
      winv[i] = ws > 0.f ? 1.f / ws : 0.f;
    }
  }
  __syncthreads();
  // merged o_b (bf16) into LDS; thread t owns columns 2t, 2t+1 (R / 2 threads per sequence)
  constexpr int TPS = R / 2;               // threads per sequence row
  constexpr int SPP = 256 / TPS;           // sequences per pass
  for (int i0 = 0; i0 < 16; i0 += SPP) {
    const int i = i0 + tid / TPS, rho = 2 * (tid % TPS);
    const int b = b0 + i;
    float a0 = 0.f, a1 = 0.f;
    if (b < B) {
      const int2 si = seqinfo[b];
      const float mx = mst[i];
#pragma unroll 4
      for (int j = 0; j < si.y; ++j) {
        const size_t pr = (size_t)(si.x + j) * H + h;
        const float wgt = part_ml[pr * 2 + 1] * exp2f(part_ml[pr * 2] - mx);
        const uint32_t pv = *(const uint32_t*)(part_o + pr * R + rho);
        a0 += wgt * bf16_to_f32((uint16_t)(pv & 0xFFFF));
        a1 += wgt * bf16_to_f32((uint16_t)(pv >> 16));
      }
      a0 *= winv[i];
      a1 *= winv[i];
    }
    *(uint32_t*)&ob[i][rho] = pack_bf16x2(a0, a1);
  }
  __syncthreads();
  // out^T[e][b] = sum_rho W_uv^T[e][rho] o[b][rho]: A = W_uv^T (e rows), B = o^T
  const int G = lane >> 4, n = lane & 15;
  const int neb = d / 16;
  for (int eb = w; eb < neb; eb += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* wrow = wvT + ((size_t)h * d + 16 * eb + n) * R + 8 * G;
#pragma unroll 4
    for (int ks = 0; ks < R / 32; ++ks) {
      const bf16x8 a = *(const bf16x8*)(wrow + 32 * ks);
      const bf16x8 bo = *(const bf16x8*)&ob[n][32 * ks + 8 * G];
      acc = mfma16x16x32(a, bo, acc);
    }
    // acc[v] = out^T[e = 16 eb + 4 G + v][b = b0 + n]
    const int b = b0 + n;
    if (b < B) {
      uint16_t* dst = out + ((size_t)b * H + h) * d + 16 * eb + 4 * G;
      const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *(u32x2*)dst = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Splits are sized so that about two blocks land on every compute unit.
static int decode_target(int B) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
  }
  const int t = 2 * cus - B;
  return t > cus ? t : cus;
}

size_t decode_max_splits(int B) { return (size_t)decode_split_cap() + B; }

template <int R>
static hipError_t run_decode(const uint16_t* q, const uint16_t* lat, const int32_t* lens,
                             const uint16_t* wk, const uint16_t* wv, uint16_t* out, int B, int Tmax,
                             int H, int d, float sl2, uint16_t* q_lat, uint16_t* part_o, float* part_ml,
                             uint16_t* wvT, int4* table, int2* seqinfo, hipStream_t st) {
  const int target = decode_target(B) < decode_split_cap() ? decode_target(B) : decode_split_cap();
  const int max_splits = target + B;
  const size_t lds = decode_lds_bytes(R);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_split<R>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  {
    ProfScope ps("decode_plan", st);
    hipLaunchKernelGGL(decode_plan, dim3(1), dim3(1024), 0, st, lens, B, Tmax, target, max_splits, table, seqinfo);
  }
  hipError_t e = absorb_mfma(q, wk, q_lat, B, H, d, R, sl2, st);
  if (e != hipSuccess) return e;
  {
    ProfScope ps("transpose_wv", st);
    e = transpose_wv_launch(wv, wvT, R, H, d, st);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps("decode_split", st);
    hipLaunchKernelGGL(decode_split<R>, dim3(max_splits, (H + 31) / 32), dim3(256), lds, st, q_lat, lat, table,
                       part_o, part_ml, Tmax, H);
  }
  {
    ProfScope ps("decode_merge_up", st);
    hipLaunchKernelGGL(decode_merge_up<R>, dim3(H, (B + 15) / 16), dim3(256), 0, st, part_o, part_ml, seqinfo,
                       wvT, out, B, H, d);
  }
  return hipGetLastError();
}

// Workspace: q_lat [B*H][r] bf16 | W_uv^T [H][d][r] | partial o [S][H][r] bf16 |
// partial (m, l) [S][H][2] f32 | split table [S] int4 | per-sequence (base, count) [B] int2,
// with S = decode_split_cap() + B; each part 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_mfma_workspace(int B, int Tmax, int H, int d, int r) {
  (void)Tmax;
  const size_t S = decode_max_splits(B);
  size_t bytes = align256((size_t)B * H * r * 2);
  bytes = align256(bytes + (size_t)H * d * r * 2);
  bytes = align256(bytes + S * H * r * 2);
  bytes = align256(bytes + S * H * 2 * 4);
  bytes = align256(bytes + S * 16);
  bytes += (size_t)B * 8;
  return bytes;
}

hipError_t decode_mfma(const void* q, const void* lat, const int32_t* lens, const void* wk,
                       const void* wv, void* out, int B, int Tmax, int H, int d, int r, float sl2,
                       void* ws, hipStream_t st) {
  const size_t S = decode_max_splits(B);
  char* p = (char*)ws;
  uint16_t* q_lat = (uint16_t*)p;
  size_t off = align256((size_t)B * H * r * 2);
  uint16_t* wvT = (uint16_t*)(p + off);
  off = align256(off + (size_t)H * d * r * 2);
  uint16_t* part_o = (uint16_t*)(p + off);
  off = align256(off + S * H * r * 2);
  float* part_ml = (float*)(p + off);
  off = align256(off + S * H * 2 * 4);
  int4* table = (int4*)(p + off);
  off = align256(off + S * 16);
  int2* seqinfo = (int2*)(p + off);
#define ARGS (const uint16_t*)q, (const uint16_t*)lat, lens, (const uint16_t*)wk, (const uint16_t*)wv, \
             (uint16_t*)out, B, Tmax, H, d, sl2, q_lat, part_o, part_ml, wvT, table, seqinfo, st
  switch (r) {
    case 128: return run_decode<128>(ARGS);
    case 256: return run_decode<256>(ARGS);
    case 512: return run_decode<512>(ARGS);
  }
#undef ARGS
  return hipErrorInvalidValue;
}

}  // namespace mla
