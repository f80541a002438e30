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
// Per tile j the 32 score ops of tile j+1 alternate with the 32 P*V ops of
// tile j-1 (whose P is ready), and the online softmax of tile j runs as 80
// pieces between them; after them O is rescaled for tile j's maxima.  k
// carries scale * log2 e, so scores are in log2 units.
constexpr int kMhaBufs = 6;
constexpr int kMhaAhead = 4;
constexpr int kMhaRows = 256;

template <int D>
struct Mha {
  static constexpr int NKS = D / 32;          // 32-wide steps of the scores' d contraction
  static constexpr int NCB = D / 16;          // 16-column blocks of the output
  static constexpr int NQB = 4;               // 16-row blocks of a wave
  static constexpr int NSO = 2 * NKS * NQB;   // score ops per tile
  static constexpr int NPV = NCB * NQB;       // P*V ops per tile
  static constexpr int KT = 32 * D * 2;       // bytes of one K (or V) tile
  static constexpr int TILE = 2 * KT;
  static constexpr int NPIECE = 80;
  static_assert(NSO == NPV, "one score op and one P*V op per slot");
};

// Keeps the computation of v at this point of the instruction stream: the
// compiler otherwise sinks softmax values that are only read after the
// rescale branch into the block behind it, out of the matrix-op slots.
template <class T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

template <int D>
constexpr size_t mha_lds_bytes() { return (size_t)kMhaBufs * Mha<D>::TILE; }

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void flash_mha_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, int B, int T, int H) {
  using M = Mha<D>;
  constexpr int NKS = M::NKS, NCB = M::NCB, NQB = M::NQB, KT = M::KT, TILE = M::TILE;
  constexpr int NI = 2 * (KT / 1024 / 4);  // copy instructions per wave and tile (K and V)
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, n = lane & 15;
  const int nqb = (T + kMhaRows - 1) / kMhaRows;
  const int BH = B * H;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);  // heaviest first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / H, h = bh % H;
  const int t0 = qblk * kMhaRows;
  const int t_last = t0 + kMhaRows - 1 < T - 1 ? t0 + kMhaRows - 1 : T - 1;
  const int ntiles = t_last / kTileKeys + 1;
  const int tw0 = t0 + 64 * w;  // first row of the wave
  const size_t stride = (size_t)H * D;
  const uint16_t* kbase = k + ((size_t)b * T * H + h) * D;
  const uint16_t* vbase = v + ((size_t)b * T * H + h) * D;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  auto copy_tile = [&](int j) {
    const uint32_t dst = lds0 + (j % kMhaBufs) * TILE;
    dma_rows32<D>(kbase, stride, kTileKeys * j, T, dst, w);
    dma_rows32<D>(vbase, stride, kTileKeys * j, T, dst + KT, w);
  };
  // wait until the own part of tile `need` landed (tiles are issued in order, each NI copies)
  auto wait_tile = [&](int need, int issued) {
    const int later = issued - 1 - need;  // tiles issued after it
    if (later >= 3)
      dma_wait<3 * NI>();
    else if (later == 2)
      dma_wait<2 * NI>();
    else if (later == 1)
      dma_wait<NI>();
    else
      dma_wait<0>();
  };

  int issued = 0;
#pragma unroll
  for (int t = 0; t < kMhaAhead; ++t)
    if (t < ntiles) {
      copy_tile(t);
      ++issued;
    }
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

  f32x4 o[NCB][NQB];
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) o[c][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NQB], l_run[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const TileCols<D> cols;
  const int f = tswz(n);  // score reads: key rows n and 16 + n
  auto rd_k = [&](const char* kt, int r) {  // read r = 2 ks + kb: key row 16 kb + n, chunk 4 ks + G
    const int kb = r & 1, ks = r >> 1;
    const int c = 4 * ks + G;
    return lds_read16(kt + (16 * kb + n) * (D * 2) + 16 * (c ^ f));
  };

  // scores of tile 0
  wait_tile(ntiles > 1 ? 1 : 0, issued);
  __builtin_amdgcn_s_barrier();
  f32x4 s_cur[2][NQB];
  {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s_cur[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2 * NKS; ++r) {
      const bf16x8 a = rd_k(smem, r);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s_cur[r & 1][qb] = mfma16x16x32(a, qf[qb][r >> 1], s_cur[r & 1][qb]);
    }
  }
  bf16x8 P_prev[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) P_prev[qb] = bf16x8{};

  // Iteration j; with MASK, keys above a row's position are masked (only
  // tiles that reach past the wave's first row need it).
  auto body = [&](int j, auto maskc) __attribute__((always_inline)) {
    constexpr bool mask = decltype(maskc)::value;
    const int k0 = kTileKeys * j;
    const char* ktile = smem + ((j + 1) % kMhaBufs) * TILE;                   // scores of tile j + 1
    const char* vtile = smem + ((j > 0 ? j - 1 : 0) % kMhaBufs) * TILE + KT;  // P*V of tile j - 1
    int lim[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) lim[qb] = t_row[qb] - k0 - 4 * G;

    // softmax state of this tile
    float x[NQB][8], mm[NQB][4], mt[NQB], ps[NQB], msub[NQB], alpha[NQB];
    bool grow[NQB];
    uint32_t pk[NQB][4];
    bf16x8 P[NQB];
    auto piece = [&](int kp) __attribute__((always_inline)) {
      if (kp < 16) {  // masking and the lane's maximum of row block kp / 4
        const int qb = kp >> 2, part = kp & 3;
        if (part == 0) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 4; ++u)
              x[qb][4 * kb + u] = (mask && 16 * kb + u > lim[qb]) ? -INFINITY : s_cur[kb][qb][u];
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
      } else if (kp < 24) {  // maximum over the four lanes of a row
        const int qb = kp & 3;
        mt[qb] = kp < 20 ? max_xor16(mt[qb]) : max_xor32(mt[qb]);
      } else if (kp < 28) {  // rescale factor
        const int qb = kp & 3;
        grow[qb] = mt[qb] > m_run[qb] + kRescaleSlack;
        alpha[qb] = grow[qb] ? fast_exp2(m_run[qb] - mt[qb]) : 1.f;
      } else if (kp < 32) {  // running max
        const int qb = kp & 3;
        m_run[qb] = grow[qb] ? mt[qb] : m_run[qb];
        // finite from tile 0 on: key 0 is unmasked for every row, so the
        // first tile always moves the running max off -infinity
        msub[qb] = m_run[qb];
        ps[qb] = 0.f;
      } else if (kp < 64) {  // probability u of row block qb, summed in pairs
        const int qb = kp & 3, u = (kp - 32) >> 2;
        x[qb][u] = fast_exp2(x[qb][u] - msub[qb]);
        pin(x[qb][u]);
        if (u & 1) ps[qb] += x[qb][u - 1] + x[qb][u];
      } else if (kp < 80) {  // bf16 pairs, then the running sum and the P operand
        const int qb = kp & 3, u = (kp - 64) >> 2;
        pk[qb][u] = pack_bf16x2(x[qb][2 * u], x[qb][2 * u + 1]);
        pin(pk[qb][u]);
        if (u == 3) {
          l_run[qb] = l_run[qb] * alpha[qb] + ps[qb];
          pin(l_run[qb]);
          P[qb] = __builtin_bit_cast(bf16x8, u32x4{pk[qb][0], pk[qb][1], pk[qb][2], pk[qb][3]});
        }
      }
    };

    // slot i: score op i of tile j + 1, then P*V op i of tile j - 1; pieces between
    f32x4 s_next[2][NQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s_next[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NSLOT = M::NSO, NR = 2 * NKS;
    bf16x8 kr[3], vr[3];
    kr[0] = rd_k(ktile, 0);
    kr[1] = rd_k(ktile, 1);
    vr[0] = cols(vtile, 0);
    vr[1] = cols(vtile, 16);
    static_for<NSLOT>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      {
        constexpr int r = i / NQB, qb = i % NQB;
        if constexpr (qb == 0 && r + 2 < NR) kr[(r + 2) % 3] = rd_k(ktile, r + 2);
        s_next[r & 1][qb] = mfma16x16x32(kr[r % 3], qf[qb][r >> 1], s_next[r & 1][qb]);
      }
#pragma unroll
      for (int kp = (2 * i) * M::NPIECE / (2 * NSLOT); kp < (2 * i + 1) * M::NPIECE / (2 * NSLOT); ++kp) piece(kp);
      __builtin_amdgcn_sched_barrier(0);
      {
        constexpr int c = i / NQB, qb = i % NQB;
        if constexpr (qb == 0 && c + 2 < NCB) vr[(c + 2) % 3] = cols(vtile, 16 * (c + 2));
        mfma16x16x32_a(o[c][qb], vr[c % 3], P_prev[qb]);
      }
#pragma unroll
      for (int kp = (2 * i + 1) * M::NPIECE / (2 * NSLOT); kp < (2 * i + 2) * M::NPIECE / (2 * NSLOT); ++kp)
        piece(kp);
      __builtin_amdgcn_sched_barrier(0);
    });

    // O holds tile j - 1 now: move it to tile j's maxima
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) any |= grow[qb];
    if (__builtin_amdgcn_ballot_w64(any)) {
      mfma_agpr_wait();
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          mfma_agpr_tie(o[c][qb]);
          o[c][qb] *= alpha[qb];
          mfma_agpr_tie(o[c][qb]);
        }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) P_prev[qb] = P[qb];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s_cur[kb][qb] = s_next[kb][qb];
    // refill the buffer of tile j - 2 (its last reader, P*V of j - 2, ended last iteration)
    if (j + kMhaAhead < ntiles) {
      copy_tile(j + kMhaAhead);
      ++issued;
    }
    // own part of tile j + 2 landed before the barrier that ends the iteration
    if (j + 2 < ntiles) wait_tile(j + 2, issued);
    __builtin_amdgcn_s_barrier();
  };
  const int jm = tw0 / kTileKeys < ntiles ? tw0 / kTileKeys : ntiles;  // tiles below every row of the wave
  for (int j = 0; j < jm; ++j) body(j, std::false_type{});
  for (int j = jm; j < ntiles; ++j) body(j, std::true_type{});

  // P*V of the last tile
  {
    const char* vtile = smem + ((ntiles - 1) % kMhaBufs) * TILE + KT;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const bf16x8 a = cols(vtile, 16 * c);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) mfma16x16x32_a(o[c][qb], a, P_prev[qb]);
    }
  }
  // l of each row from its four lanes, then the normalised rows
  float inv[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float l = l_run[qb] + __shfl_xor(l_run[qb], 16);
    l += __shfl_xor(l, 32);
    inv[qb] = 1.f / l;
  }
  mfma_agpr_wait();
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int t = tw0 + 16 * qb + n;
    if (t >= T) continue;
    uint16_t* orow = out + (((size_t)b * T + t) * H + h) * D + 4 * G;
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      mfma_agpr_tie(o[c][qb]);
      const u32x2 val = {pack_bf16x2(o[c][qb][0] * inv[qb], o[c][qb][1] * inv[qb]),
                         pack_bf16x2(o[c][qb][2] * inv[qb], o[c][qb][3] * inv[qb])};
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
    hipLaunchKernelGGL(flash_mha_bf16<128>, dim3(B * H * nqb), dim3(256), mha_lds_bytes<128>(), st,
                       (const uint16_t*)q, kk, vv, (uint16_t*)out, B, T, H);
  }
  return hipGetLastError();
}

}  // namespace mla
