// Unabsorbed prefill: causal multi-head flash attention over k and v
// materialised from the latent (k = latent W_uk[:, h], v = latent W_uv[:, h]),
// the form the KV-compression page writes out before attention.  At r > d it
// does r / d times fewer matrix FLOPs than the absorbed form.
#include <type_traits>

#include "lds_tiles.h"
#include "mla_device.h"
#include "mla_kernels.h"
#include "host_once.h"
#include "profile.h"

namespace mla {

// LDS-DMA of 32 consecutive rows of D bf16 (global row stride `stride`
// elements, rows >= kend clamped to kend - 1) into a swizzled 32-row tile
// (the layout of lds_tiles.h): wave w issues instructions w, w + 4, ...
template <int D>
__device__ __forceinline__ void dma_rows32(const uint16_t* base, size_t stride, int k0, int kend, uint32_t tile,
                                           int w) {
  constexpr int NC = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / NC;  // rows per instruction
  constexpr int NI = 32 * D * 2 / 1024 / 4;
  static_assert(NC == 16, "rows of 16 chunks: one swizzle group per row");
  const int lane = threadIdx.x & 63;
  const int sl = lane / NC, p = lane % NC;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ins = 4 * i + w;
    const int r0 = ins * RPI;
    const int kb = __builtin_amdgcn_readfirstlane(k0 + r0 < kend ? k0 + r0 : kend - 1);
    const int s = r0 + sl;
    const int key = k0 + s < kend ? k0 + s : kend - 1;
    dma16(base + (size_t)kb * stride, (uint32_t)((size_t)(key - kb) * stride * 2 + 16 * (p ^ tswz(s))),
          tile + ins * 1024);
  }
}

// v = x, written into v's own register (an asm with a tied operand).
__device__ __forceinline__ void set_in_place(float& v, float x) { asm volatile("v_mov_b32 %0, %1" : "+v"(v) : "v"(x)); }

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled by construction
// (a loop this large is not fully unrolled by the compiler, and the softmax
// pieces need compile-time indices to stay in registers).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// One block = 256 consecutive query rows t0 .. t0 + 255 of one (b, h); wave
// w owns rows t0 + 64 w .. + 63 (four 16-row blocks qb) and computes both
// products for them, so probabilities never leave its registers.  K and V
// stream through a ring of kMhaBufs tiles of 32 keys (K tile then V tile,
// each the swizzled row-major layout of lds_tiles.h), copied kMhaAhead tiles
// ahead.  Lane l = 16 G + n:
//   scores: S^T[16 kb + 4 G + v][16 qb + n] in s[kb][qb][v] (A = K rows, B = q^T)
//   P:      per qb the 8 probabilities of keys {16 kb + 4 G + v}: the P^T operand
//   output: O^T[16 c + 4 G + v][16 qb + n] in o[c][qb][v]   (A = V^T by TileCols)
// The row sums come from the matrix unit too: a ninth output block o[NCB]
// multiplies P^T by an all-ones A operand, so every element of o[NCB][qb]
// holds the sum of row 16 qb + n's bf16 probabilities, rescaled with O.
// Per tile j the 32 score ops of tile j+1 alternate with the P*V ops of tile
// j-1 (whose P is ready), and the online softmax of tile j runs as NPIECE
// pieces between them; after them O is rescaled for tile j's maxima.  k
// carries scale * log2 e, so scores are in log2 units.
//
// A single wave per SIMD issues one instruction at a time, so the loop is
// written for instruction count: the ring has a power-of-two size, whole
// tiles are copied with loop-invariant lane offsets, the four row maxima of
// a lane are reduced and broadcast across its four 16-lane rows together
// (twelve cross-lane instructions for all four), the rescale factor is only computed in
// the (rare) rescale branch, and the loop runs two tiles per trip with the
// score and probability registers swapping roles instead of being copied.
constexpr int kMhaBufs = 8;
constexpr int kMhaAhead = 6;
constexpr int kMhaRows = 256;
static_assert((kMhaBufs & (kMhaBufs - 1)) == 0, "ring slots by masking");
// tile j + kMhaAhead reuses the slot of tile j + kMhaAhead - kMhaBufs, whose
// last reader (P*V in iteration j + kMhaAhead - kMhaBufs + 1) finished before
// the barrier that ends iteration j - 1
static_assert(kMhaAhead <= kMhaBufs - 2 && kMhaAhead >= 3, "ring reuse distance");

template <int D>
struct Mha {
  static constexpr int NKS = D / 32;          // 32-wide steps of the scores' d contraction
  static constexpr int NCB = D / 16;          // 16-column blocks of the output
  static constexpr int NQB = 4;               // 16-row blocks of a wave
  static constexpr int NSO = 2 * NKS * NQB;   // score ops per tile
  static constexpr int NPV = NCB * NQB;       // P*V ops per tile (plus NQB row-sum ops)
  static constexpr int KT = 32 * D * 2;       // bytes of one K (or V) tile
  static constexpr int TILE = 2 * KT;
  static constexpr int NPIECE = 80;
  static_assert(NSO == NPV, "one score op and one P*V op per slot");
};

template <int D>
constexpr size_t mha_lds_bytes() { return (size_t)kMhaBufs * Mha<D>::TILE; }

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void flash_mha_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, int B, int T, int H, int grp) {
  using M = Mha<D>;
  constexpr int NKS = M::NKS, NCB = M::NCB, NQB = M::NQB, KT = M::KT, TILE = M::TILE;
  constexpr int NIK = KT / 1024 / 4;  // copy instructions per wave for one K (or V) tile
  constexpr int NI = 2 * NIK;         // ... for K and V
  static_assert(NIK == 2 && D / 8 == 16, "whole-tile copies: two instructions of four rows per wave");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, n = lane & 15;
  const int nqb = (T + kMhaRows - 1) / kMhaRows;
  const int BH = B * H;
  // Block i runs on XCD i % 8 (round-robin dispatch).  With grp > 0 (B * H
  // a multiple of 8, nqb a multiple of grp) XCD x takes the heads bh = x
  // (mod 8) and walks grp row blocks of one head, heaviest first, then the
  // same levels of its next head, and so on, before the next grp levels: the
  // blocks an XCD runs at a time then stream fewer heads' K and V, close
  // together, through its L2, while the order stays heaviest first in steps
  // of grp levels.  Otherwise all heads' heaviest row blocks go first.
  int qidx, bh;  // qidx 0 = the heaviest row block
  if (grp > 0) {
    const int m = (int)(blockIdx.x >> 3), hx = BH >> 3;
    const int lvl = m / (grp * hx), r = m % (grp * hx);
    qidx = grp * lvl + r % grp;
    bh = 8 * (r / grp) + (int)(blockIdx.x & 7);
  } else {
    qidx = (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
  }
  const int qblk = nqb - 1 - qidx;
  const int b = bh / H, h = bh % H;
  const int t0 = qblk * kMhaRows;
  const int t_last = t0 + kMhaRows - 1 < T - 1 ? t0 + kMhaRows - 1 : T - 1;
  const int ntiles = t_last / kTileKeys + 1;
  const int tw0 = t0 + 64 * w;  // first row of the wave
  const size_t stride = (size_t)H * D;
  const uint16_t* kbase = k + ((size_t)b * T * H + h) * D;
  const uint16_t* vbase = v + ((size_t)b * T * H + h) * D;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  // Whole-tile copies: copy instruction i of wave w moves key rows 16 i + 4 w
  // .. + 3 (lane: row sl = lane / 16, chunk p = lane % 16, fetched for LDS
  // chunk slot p, i.e. from chunk p ^ tswz(row)); tswz has period 16 in the
  // row, so both instructions share the lane offset, the second 16 rows on.
  const uint32_t voff0 = (uint32_t)((lane >> 4) * stride * 2 + 16 * ((lane & 15) ^ tswz(4 * w + (lane >> 4))));
  const uint32_t voff1 = voff0 + (uint32_t)(16 * stride * 2);
  const uint16_t* kw = kbase + 4 * w * stride;
  const uint16_t* vw = vbase + 4 * w * stride;
  auto copy_tile = [&](int t) {
    const uint32_t dst = lds0 + (uint32_t)(t & (kMhaBufs - 1)) * TILE;
    if (kTileKeys * t + kTileKeys <= T) {
      const uint16_t* kt = kw + (size_t)kTileKeys * t * stride;
      const uint16_t* vt = vw + (size_t)kTileKeys * t * stride;
      dma16_m0(kt, voff0, dst + w * 1024);
      dma16_m0(kt, voff1, dst + (4 + w) * 1024);
      dma16_m0(vt, voff0, dst + KT + w * 1024);
      dma16_m0(vt, voff1, dst + KT + (4 + w) * 1024);
    } else {  // the ragged last tile: rows clamped to T - 1
      dma_rows32<D>(kbase, stride, kTileKeys * t, T, dst, w);
      dma_rows32<D>(vbase, stride, kTileKeys * t, T, dst + KT, w);
    }
  };

  const int npro = ntiles < kMhaAhead ? ntiles : kMhaAhead;
  for (int t = 0; t < npro; ++t) copy_tile(t);
  // q rows of the lane: t = tw0 + 16 qb + n; B operand q^T[32 ks + 8 G ..][n]
  int t_row[NQB];
  bf16x8 qf[NQB][NKS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int t = tw0 + 16 * qb + n;
    t_row[qb] = t < T ? t : T - 1;
    const uint16_t* qrow = q + (((size_t)b * T + t_row[qb]) * H + h) * D + 8 * G;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] = *(const bf16x8*)(qrow + 32 * ks);
  }
  // Consume the query registers before the loop: the copies are invisible to
  // the compiler's wait counting, and a query load still pending at the loop
  // head would make it wait on the vector-memory counter every iteration.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : : "v"(qf[qb][ks]));

  f32x4 o[NCB + 1][NQB];
#pragma unroll
  for (int c = 0; c <= NCB; ++c)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) o[c][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The all-ones A operand of the row-sum ops, produced by an asm so that the
  // compiler keeps it in registers instead of re-creating it next to a matrix
  // op (a VALU write just before a matrix op reads it is a hazard the
  // compiler does not see inside inline asm).
  uint32_t one2;
  asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(one2));
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{one2, one2, one2, one2});

  // LDS read offsets, loop-invariant: K rows 16 kb + n, chunk 4 ks + G
  // (kb = 1 is 16 rows on, an immediate offset); V^T columns by TileCols.
  uint32_t koff[NKS];
  {
    const int f = tswz(n);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = (uint32_t)(n * (D * 2) + 16 * ((4 * ks + G) ^ f));
  }
  uint32_t vcol[NCB];
  {
    const int key = 4 * G + (n >> 2), fk = tswz(key), sub = 8 * (n & 1), half = (n & 3) >> 1;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int ch = 2 * c + half;
      vcol[c] = (uint32_t)(KT + key * (D * 2) + 16 * ((ch & ~15) | ((ch & 15) ^ fk)) + sub);
    }
  }
  auto rd_k = [&](uint32_t slot, int r) {  // read r = 2 ks + kb
    return lds_read16(smem + slot + koff[r >> 1] + (r & 1) * 16 * (D * 2));
  };
  auto rd_v = [&](uint32_t slot, int c) {  // A operand V^T rows 16 c .., keys 4 G + u and 16 + 4 G + u
    const char* p = smem + slot + vcol[c];
    const i16x4 a0 = lds_read_tr16(p);
    const i16x4 a1 = lds_read_tr16(p + 16 * (D * 2));
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                                            __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]});
  };

  // Softmax state of the lane's row in each row block.  Every score chain
  // starts from cb[qb] = -m_run instead of 0, so the scores arrive relative
  // to the running maximum and the usual tile needs no subtraction before
  // its exponentials.
  //   m_run  the running maximum (absolute; set from tile 0 in the prologue,
  //          finite from then on since tile 0 holds key 0, visible to every row);
  //   base   m_run - the reference the scores of the tile being normalised
  //          started from: 0 except in the tile after a new reference;
  //   thr    base + slack: a tile maximum above it moves the reference.
  float m_run[NQB], base[NQB], thr[NQB], cb[NQB][4];
  bool moved = false;  // wave-uniform: some row moved its reference in the previous tile
  bool refix = false;  // wave-uniform: the previous tile's probabilities are to be computed again

  // tiles 0 and 1 landed (own part), then everyone's
  if (ntiles >= kMhaAhead)
    dma_wait<(kMhaAhead - 2) * NI>();
  else
    dma_wait<0>();
  __builtin_amdgcn_s_barrier();
  f32x4 sA[2][NQB], sB[2][NQB];
  bf16x8 PA[NQB], PB[NQB];
  {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) sA[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2 * NKS; ++r) {
      const bf16x8 a = rd_k(0, r);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) sA[r & 1][qb] = mfma16x16x32(a, qf[qb][r >> 1], sA[r & 1][qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) PA[qb] = bf16x8{};
  }

  // tiles below every row of the wave need no mask
  const int jm = tw0 / kTileKeys < ntiles ? tw0 / kTileKeys : ntiles;
  // keys of tile j above a row's position to -inf (the caller tests j >= jm)
  auto mask_tile = [&](int j, f32x4 (&sc)[2][NQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int lim = t_row[qb] - kTileKeys * j - 4 * G;  // last visible key offset 16 kb + u
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (16 * (e >> 2) + (e & 3) > lim) sc[e >> 2][qb][e & 3] = -INFINITY;
    }
  };
  // The probabilities of tile jp again, from its K tile (still in its slot
  // until the copy two iterations after jp's), relative to the references
  // jp's iteration moved to (-cb): for the rare tile after which some row's
  // reference moved or whose scores started from an older reference.
  auto reprob = [&](int jp, bf16x8 (&P)[NQB]) __attribute__((always_inline)) {
    f32x4 s2[2][NQB];
    const uint32_t tslot = (uint32_t)(jp & (kMhaBufs - 1)) * TILE;
#pragma unroll
    for (int r = 0; r < 2 * NKS; ++r) {
      const bf16x8 a = rd_k(tslot, r);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s2[r & 1][qb] = mfma16x16x32(a, qf[qb][r >> 1],
                                     r < 2 ? f32x4{cb[qb][0], cb[qb][1], cb[qb][2], cb[qb][3]} : s2[r & 1][qb]);
    }
    if (jp >= jm) mask_tile(jp, s2);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      uint32_t pk2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pk2[u] = pack_bf16x2(fast_exp2(s2[u >> 1][qb][2 * (u & 1)]), fast_exp2(s2[u >> 1][qb][2 * (u & 1) + 1]));
      P[qb] = __builtin_bit_cast(bf16x8, u32x4{pk2[0], pk2[1], pk2[2], pk2[3]});
    }
  };
  // Tile 0 sets the first references: its row maxima (over the four lanes of
  // a row), its scores made relative to them, and the chains of tile 1 start
  // from them.
  if (0 >= jm) mask_tile(0, sA);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float m = fmaxf(fmaxf(fmaxf(sA[0][qb][0], sA[0][qb][1]), fmaxf(sA[0][qb][2], sA[0][qb][3])),
                    fmaxf(fmaxf(sA[1][qb][0], sA[1][qb][1]), fmaxf(sA[1][qb][2], sA[1][qb][3])));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    m_run[qb] = m;
    base[qb] = 0.f;
    thr[qb] = kRescaleSlack;
#pragma unroll
    for (int k = 0; k < 4; ++k) cb[qb][k] = -m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sA[kb][qb][v] -= m;
  }
  // Iteration j: softmax of tile j (scores in sc, probabilities out in Pn),
  // scores of tile j + 1 into sn, P*V of tile j - 1 from Pp.  Tiles that
  // reach past the wave's first row first get keys above a row's position
  // masked, in a branch of their own ahead of the slots.
  auto body = [&](int j, f32x4 (&sc)[2][NQB], f32x4 (&sn)[2][NQB], bf16x8 (&Pp)[NQB],
                  bf16x8 (&Pn)[NQB]) __attribute__((always_inline)) {
    const uint32_t kslot = (uint32_t)((j + 1) & (kMhaBufs - 1)) * TILE;                 // scores of tile j + 1
    const uint32_t vslot = (uint32_t)((j > 0 ? j - 1 : 0) & (kMhaBufs - 1)) * TILE;     // P*V of tile j - 1
    if (__builtin_expect(refix, 0)) reprob(j - 1, Pp);
    if (j >= jm) mask_tile(j, sc);

    float mt[NQB];
    bool grow[NQB];
    uint32_t pk[NQB][4];
    // element e = 4 kb + u of row block qb: sc[kb][qb][u]
    float x[NQB][8];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[qb][e] = sc[e >> 2][qb][e & 3];
    auto piece = [&](int kp) __attribute__((always_inline)) {
      if (kp < 16) {  // the lane's maximum of row block kp / 4
        const int qb = kp >> 2, part = kp & 3;
        if (part == 0) {
          mt[qb] = fmaxf(fmaxf(x[qb][0], x[qb][1]), x[qb][2]);
        } else if (part == 1) {
          mt[qb] = fmaxf(fmaxf(mt[qb], x[qb][3]), x[qb][4]);
        } else if (part == 2) {
          mt[qb] = fmaxf(fmaxf(mt[qb], x[qb][5]), x[qb][6]);
        } else {
          mt[qb] = fmaxf(mt[qb], x[qb][7]);
        }
      } else if (kp < 28) {
        // Row maxima over the four 16-lane rows, all four row blocks at once:
        // after the pair swaps and the 32-lane swap, row g of mt[0] holds the
        // maximum of row block g; three more swaps broadcast it to every row.
        switch (kp) {
          case 16: swap16(mt[0], mt[1]); break;
          case 17: mt[0] = fmaxf(mt[0], mt[1]); break;
          case 18: swap16(mt[2], mt[3]); break;
          case 19: mt[2] = fmaxf(mt[2], mt[3]); break;
          case 20: swap32(mt[0], mt[2]); break;
          case 21: mt[0] = fmaxf(mt[0], mt[2]); break;
          case 22: mt[2] = mt[0]; break;
          case 23: swap32(mt[0], mt[2]); break;  // mt[0]: rows (0, 1, 0, 1); mt[2]: (2, 3, 2, 3)
          case 24: mt[1] = mt[0]; break;
          case 25: swap16(mt[0], mt[1]); break;  // block 0 everywhere in mt[0], block 1 in mt[1]
          case 26: mt[3] = mt[2]; break;
          default: swap16(mt[2], mt[3]); break;  // blocks 2 and 3
        }
      } else if (kp < 32) {  // lazy rescale: a new reference only if the max moved past the slack
        const int qb = kp & 3;
        grow[qb] = mt[qb] > thr[qb];
      } else if (kp < 64) {  // probability e of row block qb
        const int qb = kp & 3, e = (kp - 32) >> 2;
        x[qb][e] = fast_exp2(x[qb][e]);
        pin(x[qb][e]);
      } else if (kp < 80) {  // bf16 pairs, then the P operand
        const int qb = kp & 3, u = (kp - 64) >> 2;
        pk[qb][u] = pack_bf16x2(x[qb][2 * u], x[qb][2 * u + 1]);
        pin(pk[qb][u]);
        if (u == 3) Pn[qb] = __builtin_bit_cast(bf16x8, u32x4{pk[qb][0], pk[qb][1], pk[qb][2], pk[qb][3]});
      }
    };

    // slot i: score op i of tile j + 1, then P*V op i of tile j - 1 (and, in
    // the last slot of each column step pair, a row-sum op); pieces between
    constexpr int NSLOT = M::NSO, NR = 2 * NKS;
    bf16x8 kr[3], vr[3];
    kr[0] = rd_k(kslot, 0);
    kr[1] = rd_k(kslot, 1);
    vr[0] = rd_v(vslot, 0);
    vr[1] = rd_v(vslot, 1);
    static_for<NSLOT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      {
        constexpr int r = i / NQB, qb = i % NQB;
        if constexpr (qb == 0 && r + 2 < NR) kr[(r + 2) % 3] = rd_k(kslot, r + 2);
        if constexpr (r < 2)
          sn[r & 1][qb] = mfma16x16x32(kr[r % 3], qf[qb][r >> 1], f32x4{cb[qb][0], cb[qb][1], cb[qb][2], cb[qb][3]});  // from -ref
        else
          sn[r & 1][qb] = mfma16x16x32(kr[r % 3], qf[qb][r >> 1], sn[r & 1][qb]);
      }
#pragma unroll
      for (int kp = (2 * i) * M::NPIECE / (2 * NSLOT); kp < (2 * i + 1) * M::NPIECE / (2 * NSLOT); ++kp) piece(kp);
      __builtin_amdgcn_sched_barrier(0);
      {
        constexpr int c = i / NQB, qb = i % NQB;
        if constexpr (qb == 0 && c + 2 < NCB) vr[(c + 2) % 3] = rd_v(vslot, c + 2);
        mfma16x16x32_a(o[c][qb], vr[c % 3], Pp[qb]);
        if constexpr (i % 8 == 7) mfma16x16x32_a(o[NCB][i / 8], ones, Pp[i / 8]);
      }
#pragma unroll
      for (int kp = (2 * i + 1) * M::NPIECE / (2 * NSLOT); kp < (2 * i + 2) * M::NPIECE / (2 * NSLOT); ++kp)
        piece(kp);
      __builtin_amdgcn_sched_barrier(0);
    });

    // The probabilities above are right when every shift is 0: no row of
    // this tile moved its reference and none did in the previous tile (the
    // usual case).  Otherwise the state moves to the new references and this
    // tile's scores are computed again from its K tile (still in its slot,
    // which is refilled two iterations later), now relative to them.  The
    // chains of tile j + 1 started from the old cb.
    bool g = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) g |= grow[qb];
    const bool grew = __builtin_amdgcn_ballot_w64(g) != 0;
    float alpha[NQB];
    refix = false;
    if (__builtin_expect(grew || moved, 0)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float nm = grow[qb] ? mt[qb] + m_run[qb] - base[qb] : m_run[qb];  // the new reference
        const float nb = nm + cb[qb][0];                                         // tile j + 1 started from cb
        alpha[qb] = grow[qb] ? fast_exp2(m_run[qb] - nm) : 1.f;
        // the state is rewritten in place (tied operands): with plain
        // assignments the compiler kept it in other registers on this path
        // and copied it back on the usual one
        set_in_place(m_run[qb], nm);
        set_in_place(base[qb], nb);
        set_in_place(thr[qb], nb + kRescaleSlack);
#pragma unroll
        for (int k = 0; k < 4; ++k) set_in_place(cb[qb][k], -nm);
      }
      refix = true;
    }
    moved = grew;
    // O and the row sums hold tile j - 1 now: move them to tile j's maxima
    if (grew) {
      mfma_agpr_wait();
#pragma unroll
      for (int c = 0; c <= NCB; ++c)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          mfma_agpr_tie(o[c][qb]);
          o[c][qb] *= alpha[qb];
          mfma_agpr_tie(o[c][qb]);
        }
    }
    // refill the slot of tile j + kMhaAhead - kMhaBufs; tile j + 2 (own part) landed before the barrier
    if (j + kMhaAhead < ntiles) {
      copy_tile(j + kMhaAhead);
      dma_wait<(kMhaAhead - 2) * NI>();
    } else {
      dma_wait<0>();
    }
    __builtin_amdgcn_s_barrier();
  };
  // Two tiles per trip, the registers swapping roles.  An odd count runs one
  // phantom tile j = ntiles at the end: every key of it lies above every row
  // of the block, so the mask branch turns its (stale) scores into -inf and
  // its probabilities into 0, and its iteration does the P*V of the real
  // last tile; the epilogue then has no P*V left to do.
  for (int j = 0; j < ntiles; j += 2) {
    body(j, sA, sB, PA, PB);
    body(j + 1, sB, sA, PB, PA);
  }

  // P*V and row sums of the last tile (even counts)
  if (!(ntiles & 1)) {
    if (refix) reprob(ntiles - 1, PA);
    const uint32_t vslot = (uint32_t)((ntiles - 1) & (kMhaBufs - 1)) * TILE;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const bf16x8 a = rd_v(vslot, c);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) mfma16x16x32_a(o[c][qb], a, PA[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mfma16x16x32_a(o[NCB][qb], ones, PA[qb]);
  }
  mfma_agpr_wait();
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int t = tw0 + 16 * qb + n;
    mfma_agpr_tie(o[NCB][qb]);
    const float inv = 1.f / o[NCB][qb][0];
    if (t >= T) continue;
    uint16_t* orow = out + (((size_t)b * T + t) * H + h) * D + 4 * G;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      mfma_agpr_tie(o[c][qb]);
      const u32x2 val = {pack_bf16x2(o[c][qb][0] * inv, o[c][qb][1] * inv),
                         pack_bf16x2(o[c][qb][2] * inv, o[c][qb][3] * inv)};
      *(u32x2*)(orow + 16 * c) = val;
    }
  }
}

// Workspace: k [B*T][H][d] | v [B*T][H][d] | W_uk^T [H][d][r] | W_uv^T [H][d][r], bf16.
size_t prefill_unabsorbed_workspace(int B, int T, int H, int d, int r) {
  const size_t rows = (size_t)B * T * H;
  return (2 * rows * d + 2 * (size_t)H * d * r) * 2;
}

bool unabsorbed_supported(int d, int r) { return d == 128 && (r == 128 || r == 256 || r == 512); }

size_t unabsorbed_lds_bytes(int d) { return d == 128 ? mha_lds_bytes<128>() : 0; }

hipError_t prefill_unabsorbed(const void* q, const void* lat, const void* wk, const void* wv, void* out, int B,
                              int T, int H, int d, int r, float sl2, void* ws, hipStream_t st) {
  if (!unabsorbed_supported(d, r)) return hipErrorInvalidValue;
  const size_t rows = (size_t)B * T * H;
  uint16_t* kk = (uint16_t*)ws;
  uint16_t* vv = kk + rows * d;
  uint16_t* wkT = vv + rows * d;
  uint16_t* wvT = wkT + (size_t)H * d * r;
  hipError_t e = materialise_kv((const uint16_t*)lat, (const uint16_t*)wk, (const uint16_t*)wv, kk, vv, wkT, wvT,
                                B * T, H, d, r, sl2, st);
  if (e != hipSuccess) return e;
  static OnceFlag attrs;
  e = run_once(attrs, [] {
    return hipFuncSetAttribute((const void*)flash_mha_bf16<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)mha_lds_bytes<128>());
  });
  if (e != hipSuccess) return e;
  const int nqb = (T + kMhaRows - 1) / kMhaRows;
  {
    ProfScope ps("flash_mha_bf16", st);
    // Whole heads per XCD when every compute unit runs many blocks (the
    // heaviest block is then a small part of a unit's work, and a late start
    // of it costs little): at bf16_long_prefill (32 blocks per unit) 9.27 ->
    // 8.48 ms.  With few blocks per unit, heaviest first: at bf16_prefill (4
    // per unit) whole heads took 0.187 -> 0.253 ms.
    int grp = 0;
    if ((B * H) % 8 == 0) grp = (long)B * H * nqb >= 16L * device_cus() ? nqb : 1;
    hipLaunchKernelGGL(flash_mha_bf16<128>, dim3(B * H * nqb), dim3(256), mha_lds_bytes<128>(), st,
                       (const uint16_t*)q, kk, vv, (uint16_t*)out, B, T, H, grp);
  }
  return hipGetLastError();
}

}  // namespace mla
