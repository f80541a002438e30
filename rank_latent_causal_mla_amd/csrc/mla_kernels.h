// Host-visible entry points of the device code (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Decode split: each of the 4 waves of a block streams this many 32-key tiles.
constexpr int kDecodeTilesPerWave = 8;

// LDS of the decode split kernel: four wave-private 32-key tiles, reused at
// the end for two wave states plus their (m, l).
constexpr size_t decode_lds_bytes(int R) { return (size_t)4 * 32 * R * 2 + 2 * 64 * 2 * 4; }

// LDS of the prefill flash kernel: two row-major and three transposed 32-key tiles.
constexpr size_t flash_lds_bytes(int R) { return (size_t)5 * 32 * R * 2; }

// ---- bf16 matrix-core path (r in {128, 256, 512}, d % 32 == 0, d <= 256)
bool mfma_supported(int d, int r);
hipError_t prefill_mfma(const void* q, const void* lat, const void* wk, const void* wv, void* out,
                        int B, int T, int H, int d, int r, float sl2, void* ws, hipStream_t st);
size_t prefill_mfma_workspace(int B, int T, int H, int d, int r);
int decode_nsplit(int Tmax);
size_t decode_mfma_workspace(int B, int Tmax, int H, int d, int r);
hipError_t decode_mfma(const void* q, const void* lat, const int32_t* lens, const void* wk,
                       const void* wv, void* out, int B, int Tmax, int H, int d, int r, float sl2,
                       void* ws, hipStream_t st);

// ---- SIMT path: float32 (or bf16 storage) with float32 arithmetic, any r <= 1024, d <= 256
// dt_bf16: inputs and outputs stored as bf16 (else float32).
hipError_t prefill_simt(bool dt_bf16, const void* q, const void* lat, const void* wk,
                        const void* wv, void* out, int B, int T, int H, int d, int r,
                        float scale, void* ws, hipStream_t st);
size_t prefill_simt_workspace(int B, int T, int H, int d, int r);
hipError_t decode_simt(bool dt_bf16, const void* q, const void* lat, const int32_t* lens,
                       const void* wk, const void* wv, void* out, int B, int Tmax, int H, int d,
                       int r, float scale, void* ws, hipStream_t st);
size_t decode_simt_workspace(int B, int Tmax, int H, int d, int r);

// ---- down-projection (any sizes), float32 accumulation
hipError_t down_proj(bool dt_bf16, const void* hidden, const void* w_down, void* latent, int M,
                     int D, int r, hipStream_t st);

}  // namespace mla
