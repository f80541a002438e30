// Latent tiles in LDS, shared by the prefill and decode kernels: LDS-DMA
// copies issued as inline assembly, and the swizzled row-major 32-key tile
// that serves both the score reads (16-byte rows) and the transpose reads
// of the P * latent product.
#pragma once

#include "mla_device.h"

namespace mla {

constexpr int kTileKeys = 32;  // keys per latent tile

// LDS-DMA copy of 16 bytes per lane: lane l copies global byte
// gbase + voff(l) to LDS byte lds_base + 16 l (gbase and lds_base
// wave-uniform).  Issued as inline assembly: the compiler then cannot pair
// every later LDS transpose read with a wait for all copies in flight (it
// cannot tell which LDS bytes a copy writes), which would serialise the
// prefetch.  The kernel orders copies and reads itself with dma_wait<n>().
// M0 carries the LDS address; its previous value is restored.  With NT the
// load carries the non-temporal hint, for data read once (the decode's
// cache stream): a streaming probe read 302 MB at 6.6 TB/s with it against
// 5.9 without, and re-reading one 134 MB buffer was no slower with it.
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory");
}
// The same copy with M0 declared clobbered instead of saved and restored
// (the compiler then keeps nothing in M0 across it): two scalar
// instructions fewer per copy on the tile loops' issue path.
template <bool NT = false>
__device__ __forceinline__ void dma16_m0(const void* gbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory", "m0");
}
// Wait until at most n of this wave's vector-memory operations are outstanding.
template <int n>
__device__ __forceinline__ void dma_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(n) : "memory");
}

// Barrier that publishes this wave's LDS writes to the other waves of the
// block: the LDS serves the waves through several request queues, so a
// write is only known to precede another wave's later read once the writer's
// LDS counter has drained.  (A bare s_barrier orders instruction issue only;
// the compiler adds no wait before it on this target.)
__device__ __forceinline__ void lds_publish_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// Block-shared tile of 32 keys, row-major (R * 2 bytes a row, a multiple of
// 128), 16-byte chunks XOR-swizzled by tswz(key) inside every 16-chunk
// group.  The LDS has 32 four-byte banks (128 bytes): a 16-byte read is
// served 8 lanes at a time, an 8-byte transpose read 16 lanes at a time, and
// lanes of one group conflict when their addresses share a bank.
//   - score reads (lanes n = 0..15 of a 16-lane group: key row n, one chunk
//     each): each 8-lane half needs 8 distinct chunk slots mod 8, so
//     tswz(key) & 7 is a permutation of key & 7;
//   - transpose reads (16 lanes: keys 4 g .. 4 g + 3, two adjacent chunks
//     each, 32 bytes a key): the four keys need distinct 32-byte slots mod 4,
//     so (tswz(key) >> 1) & 3 is a permutation of key & 3.
// tswz(key + 16) = tswz(key), so rows n and 16 + n share the swizzle.
__device__ __forceinline__ int tswz(int key) { return ((key & 3) << 1) | ((key >> 2) & 1) | (key & 8); }

// Wave w's share of the LDS-DMA copy of one tile: instructions i = w, w + 4, ...
// of the tile's 32 R * 2 / 1024, each 64 lanes x 16 bytes.  The swizzle is
// applied on the global side: LDS-DMA writes lane l to byte 16 l of its
// 1 KB destination, so lane l fetches the chunk that belongs there.
// With REMAT the per-lane offsets are recomputed at every call instead of
// being kept as loop invariants (eight registers at R = 512), for kernels
// that are out of registers: a spilled offset is reloaded from scratch with
// a wait for every copy in flight.
template <int R, bool REMAT = false, bool NT = false>
__device__ __forceinline__ void dma_tile32(const uint16_t* latb, int k0, int kend, uint32_t tile, int w) {
  constexpr int NC = R / 8;    // 16-byte chunks per key row
  constexpr int RPI = 64 / NC;  // key rows per instruction
  constexpr int NI = kTileKeys * R * 2 / 1024 / 4;  // instructions per wave
  static_assert(NC <= 64 && 64 % NC == 0, "a copy instruction covers whole rows");
  unsigned lane = threadIdx.x & 63;
  if (REMAT) asm volatile("" : "+v"(lane));
  // with one row per instruction (R = 512) the row is wave-uniform
  const int sl = RPI == 1 ? 0 : (int)(lane / NC), p = (int)(lane % NC);
  if (k0 + kTileKeys <= kend) {
    // the whole tile is in range: no clamp; the same lane offsets as below
    const uint16_t* tb = latb + (size_t)(k0 + w * RPI) * R;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s = (4 * i + w) * RPI + sl;
      const int c = (p & ~15) | ((p & 15) ^ tswz(s));
      dma16_m0<NT>(tb + (size_t)4 * i * RPI * R, (uint32_t)(sl * R * 2 + 16 * c), tile + (4 * i + w) * 1024);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ins = 4 * i + w;       // wave-uniform
    const int r0 = ins * RPI;        // first row of the instruction
    const int kb = __builtin_amdgcn_readfirstlane(k0 + r0 < kend ? k0 + r0 : kend - 1);
    const int s = r0 + sl;           // row within the tile
    const int c = (p & ~15) | ((p & 15) ^ tswz(s));
    const int key = k0 + s < kend ? k0 + s : kend - 1;
    dma16<NT>(latb + (size_t)kb * R, (uint32_t)((key - kb) * R * 2 + 16 * c), tile + ins * 1024);
  }
}

// A operand of O^T += L^T P^T (16x16x32) for tile columns [c0, c0 + 16),
// c0 a multiple of 16: lane (G, n) receives L^T[c0 + n][key] for the keys
// 4 G + u and 16 + 4 G + u, u = 0..3 (the k-slot order of the P operand),
// from two transpose reads.  Transpose read t of lane (G, n) addresses key
// 16 t + 4 G + n / 4, columns c0 + 4 (n % 4) .. + 3.
template <int R>
struct TileCols {
  int key_off, fk, sub, half;
  __device__ __forceinline__ TileCols() {
    const int lane = threadIdx.x & 63, G = lane >> 4, n = lane & 15;
    const int key = 4 * G + (n >> 2);
    key_off = key * (R * 2);
    fk = tswz(key);  // equal for key + 16
    sub = 8 * (n & 1);
    half = (n & 3) >> 1;
  }
  __device__ __forceinline__ bf16x8 operator()(const char* tile, int c0) const {
    const int ch = (c0 >> 3) + half;
    const int off = key_off + 16 * ((ch & ~15) | ((ch & 15) ^ fk)) + sub;
    const i16x4 a0 = lds_read_tr16(tile + off);
    const i16x4 a1 = lds_read_tr16(tile + off + 16 * (R * 2));
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                                            __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]});
  }
};

}  // namespace mla
