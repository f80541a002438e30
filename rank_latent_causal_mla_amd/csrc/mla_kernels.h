// Host-visible entry points of the device code (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Decode: at most this many equal chunks of the concatenated cache per head
// group; a chunk holds one partial state per sequence segment, so a call
// has at most decode_split_cap() + B - 1 partial slots (workspace sized for it).
constexpr int decode_split_cap() { return 1024; }
size_t decode_max_splits(int B);
// Chunks per head group for later decode calls: 0 = one per compute unit
// (the default), else 1 .. decode_split_cap() (mla_decode_set_splits).
void set_decode_splits(int p);

// LDS of the decode split kernel: a ring of four 32-key latent tiles, the
// probabilities of one tile (2 KB), 64 row maxima and 64 partial sums.
constexpr size_t decode_lds_bytes(int R) { return (size_t)4 * 32 * R * 2 + 2048 + 512; }

// LDS of the prefill flash kernel: a ring of four 32-key latent tiles, one
// tile's probabilities for 128 rows (8 KB), 128 rescale factors, 4 flags and
// (key-masked form) the last visible key of the 512 (row, lane) slots.
constexpr size_t flash_lds_bytes(int R) { return (size_t)4 * 32 * R * 2 + 8 * 1024 + 8 * 16 * 4 + 16 + 2048; }

// ---- bf16 matrix-core path (r in {128, 256, 512}, d in {32, 64, 128, 256})
bool mfma_supported(int d, int r);
// key_mask [B][T] bytes (nonzero = visible) or null; with it the workspace holds
// prefill_mfma_workspace() + key_mask_workspace() bytes (the visible keys are
// packed there before the attention).
hipError_t prefill_mfma(const void* q, const void* lat, const void* wk, const void* wv, void* out,
                        int B, int T, int H, int d, int r, float sl2, const uint8_t* key_mask, void* ws,
                        hipStream_t st);
size_t prefill_mfma_workspace(int B, int T, int H, int d, int r);
size_t key_mask_workspace(int B, int T, int r);
size_t decode_mfma_workspace(int B, int Tmax, int H, int d, int r);
// Decode workspace bytes with `slots` partial slots (>= decode_chunks(H) + B).
size_t decode_mfma_bytes(int B, int H, int d, int r, size_t slots);
// Chunks per head group the decode split takes (the CU count, or mla_decode_set_splits).
int decode_chunks(int H);
// lens (padded cache [B, Tmax, r]) or cu (packed cache [Tmax = total rows, r]; lens unused); ws laid out
// with `slots` partial slots (decode_mfma_bytes)
hipError_t decode_mfma(const void* q, const void* lat, const int32_t* lens, const int32_t* cu, const void* wk,
                       const void* wv, void* out, int B, int Tmax, int H, int d, int r, float sl2,
                       void* ws, size_t slots, hipStream_t st);
// q_lat[n*H + h, :] = qscale * W_uk[:, h, :] q[n, h, :] for N tokens (bf16).
hipError_t absorb_mfma(const uint16_t* q, const uint16_t* wk, uint16_t* q_lat, int N, int H, int d,
                       int R, float qscale, hipStream_t st);
// W_uv [R, H, d] -> W_uv^T [H, d, R].
hipError_t transpose_wv_launch(const uint16_t* wv, uint16_t* wvT, int R, int H, int d, hipStream_t st);

// ---- unabsorbed prefill (bf16, d = 128, r in {128, 256, 512}): k and v
// materialised in the workspace, then causal flash attention over them
bool unabsorbed_supported(int d, int r);
size_t unabsorbed_lds_bytes(int d);
size_t prefill_unabsorbed_workspace(int B, int T, int H, int d, int r);
hipError_t prefill_unabsorbed(const void* q, const void* lat, const void* wk, const void* wv, void* out, int B,
                              int T, int H, int d, int r, float sl2, void* ws, hipStream_t st);
// k [N][H][d] = kscale * latent W_uk, v [N][H][d] = latent W_uv (wkT, wvT: [H][d][r] scratch)
hipError_t materialise_kv(const uint16_t* lat, const uint16_t* wk, const uint16_t* wv, uint16_t* k, uint16_t* v,
                          uint16_t* wkT, uint16_t* wvT, int N, int H, int d, int r, float kscale, hipStream_t st);

// ---- SIMT path: float32 (or bf16 storage) with float32 arithmetic, any r <= 1024, d <= 256
// dt_bf16: inputs and outputs stored as bf16 (else float32).
// key_mask [B][T] bytes (nonzero = visible) or null.
hipError_t prefill_simt(bool dt_bf16, const void* q, const void* lat, const void* wk,
                        const void* wv, void* out, int B, int T, int H, int d, int r,
                        float scale, const uint8_t* key_mask, void* ws, hipStream_t st);
size_t prefill_simt_workspace(int B, int T, int H, int d, int r);
hipError_t decode_simt(bool dt_bf16, const void* q, const void* lat, const int32_t* lens, const int32_t* cu,
                       const void* wk, const void* wv, void* out, int B, int Tmax, int H, int d,
                       int r, float scale, void* ws, hipStream_t st);
size_t decode_simt_workspace(int B, int Tmax, int H, int d, int r);

// ---- cache append: kv_cache[b, lens[b], :] = new_latent[b, :], lens[b] += 1 while lens[b] < Tmax
hipError_t kv_append(bool dt_bf16, void* kv_cache, int32_t* lens, const void* new_latent, int B, int Tmax, int r,
                     hipStream_t st);

// ---- bf16 down-projection on the matrix cores (D % 64 == 0, r % 128 == 0):
// latent [M, r] = hid [M, D] w_down [D, r]; ws holds down_mfma_workspace() bytes (w_down^T)
bool down_mfma_supported(int D, int r);
size_t down_mfma_workspace(int D, int r);
hipError_t down_mfma(const uint16_t* hid, const uint16_t* wd, uint16_t* lat, int M, int D, int r, void* ws,
                     hipStream_t st);

// ---- down-projection (any sizes), float32 accumulation
hipError_t down_proj(bool dt_bf16, const void* hidden, const void* w_down, void* latent, int M,
                     int D, int r, hipStream_t st);

}  // namespace mla
