// Device-side building blocks shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Operand and accumulator vectors of the CDNA4 bf16 matrix instructions.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// D[32x32] += A[32x16] * B[16x32] in fp32, bf16 operands.  Lane l supplies
// A[l%32][8(l/32)+0..7] and B[8(l/32)+0..7][l%32]; element v of the result
// is D[8(v/4) + 4(l/32) + v%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same instruction with the accumulator pinned to arch VGPRs (inline
// asm, so the compiler cannot choose the AGPR form for it).  The caller must
// call mfma_vgpr_drain() on the result before any VALU reads it: the
// compiler does not model the matrix-unit latency of an asm block.
__device__ __forceinline__ void mfma32x32x16_v(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// First step of a chain: accumulator input is the inline constant 0.
__device__ __forceinline__ void mfma32x32x16_v0(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a), "v"(b));
}
// Wait out the result latency of a 16-pass matrix instruction (>= 18 wait
// states) before a VALU op reads its destination; the operand ties the wait
// to the value.
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(c));
}

// Accumulator pinned to AGPRs.  Operand registers written by VALU need a
// few wait states before a matrix instruction reads them: call
// mfma_operand_ready() on such operands first.  Before VALU reads the
// accumulator, call mfma_agpr_drain() on it.
__device__ __forceinline__ void mfma32x32x16_a(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_operand_ready(bf16x8& v) {
  asm volatile("s_nop 4" : "+v"(v));
}
__device__ __forceinline__ void mfma_agpr_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4"); }
__device__ __forceinline__ void mfma_agpr_tie(f32x16& c) { asm volatile("" : "+a"(c)); }

// D[16x16] += A[16x32] * B[32x16] in fp32, bf16 operands.  Lane l supplies
// A[l%16][8(l/16)+0..7] and B[8(l/16)+0..7][l%16]; element v of the result
// is D[4(l/16) + v][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Accumulator pinned to AGPRs (same rules as mfma32x32x16_a).
// Not volatile: a side-effect-free asm lets loads be scheduled across it.
__device__ __forceinline__ void mfma16x16x32_a(f32x4& c, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr_tie(f32x4& c) { asm volatile("" : "+a"(c)); }

// Max of v over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max of v over lanes l and l ^ 16 (v_permlane16_swap exchanges 16-lane rows).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Keeps the computation of v at this point of the instruction stream: the
// compiler otherwise sinks softmax values that are only read after a
// rescale branch into the block behind it, out of the matrix-op slots.
template <class T>
__device__ __forceinline__ void pin(T& v) { asm volatile("" : "+v"(v)); }

// permlane16_swap(a, b): the odd 16-lane rows of a trade places with the even
// rows of b.
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// permlane32_swap(a, b): the upper 32 lanes of a trade places with the lower 32 of b.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// 2^x by the hardware exponential alone (no range reduction for results
// below the smallest normal float, which flush to zero): softmax weights are
// 2^(x - m) with x - m <= 8, where such results are negligible.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte read of LDS through an explicit LDS pointer: a generic pointer
// whose address space the compiler cannot infer becomes a flat load, which
// also waits on every outstanding global load.
__device__ __forceinline__ bf16x8 lds_read16(const void* lds_byte_addr) {
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)lds_byte_addr;
}

// LDS transpose read: within each group of 16 lanes, element k of lane i is
// element i%4 of the 8 bytes addressed by lane 4k + i/4.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lds_byte_addr);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Wait until every memory operation this wave issued has completed
// (including LDS-DMA writes from global_load_lds).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most n of this wave's vector-memory operations (here: the
// LDS-DMA copies, in issue order) are still outstanding.
template <int n>
__device__ __forceinline__ void wait_vmem_outstanding() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Slack (log2 units) the online-softmax reference max may lag the running
// max before the accumulators are rescaled; probabilities then stay <= 2^8.
// The normalised result does not depend on it.
constexpr float kRescaleSlack = 8.f;

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct io<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

}  // namespace mla
