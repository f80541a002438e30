// C ABI of the library: argument checks, workspace sizing, path selection
// and launch sequencing.  Declarations and the contract are in include/mla.h.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/mla.h"
#include "mla_kernels.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr double kLog2e = 1.4426950408889634;

// Shared size checks of the attention entry points.
mla_status check_dims(int B, int T, int H, int d, int r, mla_dtype dt, const char* tname) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || r < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d %s=%d H=%d d=%d r=%d)", B,
                tname, T, H, d, r);
  if (dt != MLA_DTYPE_F32 && dt != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  if (r > MLA_MAX_RANK) return fail(MLA_ERR_UNSUPPORTED, "r=%d exceeds %d", r, MLA_MAX_RANK);
  if (d > MLA_MAX_HEAD_DIM) return fail(MLA_ERR_UNSUPPORTED, "d=%d exceeds %d", d, MLA_MAX_HEAD_DIM);
  // element counts are indexed with 64-bit offsets, block counts must fit the grid
  const double rows = (double)B * T * H;
  if ((double)B * T >= 2147483647.0 || rows * (r > d ? r : d) >= 9.0e15)
    return fail(MLA_ERR_UNSUPPORTED, "problem too large (B*T*H=%.0f)", rows);
  return MLA_OK;
}

bool use_mfma(mla_dtype dt, int d, int r) { return dt == MLA_DTYPE_BF16 && mla::mfma_supported(d, r); }

std::atomic<size_t> g_lds_limit_override{0};  // mla_set_lds_limit_override(); 0 = query the device

mla_status device_lds_limit(size_t* bytes) {
  const size_t forced = g_lds_limit_override.load(std::memory_order_relaxed);
  if (forced > 0) {
    *bytes = forced;
    return MLA_OK;
  }
  int dev = 0, v = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  *bytes = (size_t)v;
  return MLA_OK;
}

mla_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_down_proj(const void* hidden, const void* w_down, void* kv_latent, int B, int T,
                         int D, int r, mla_dtype dt, void* stream) {
  if (!hidden || !w_down || !kv_latent) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (B < 1 || T < 1 || D < 1 || r < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d T=%d D=%d r=%d)", B, T, D, r);
  if (dt != MLA_DTYPE_F32 && dt != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  if (!aligned16(hidden) || !aligned16(w_down) || !aligned16(kv_latent))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (r > MLA_MAX_RANK) return fail(MLA_ERR_UNSUPPORTED, "r=%d exceeds %d", r, MLA_MAX_RANK);
  if ((double)B * T >= 2147483647.0 / 64 || (double)B * T * D >= 9.0e15)
    return fail(MLA_ERR_UNSUPPORTED, "problem too large");
  return launched(mla::down_proj(dt == MLA_DTYPE_BF16, hidden, w_down, kv_latent, B * T, D, r,
                                 (hipStream_t)stream),
                  "down_proj launch");
}

size_t mla_latent_attn_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || r < 1) return 0;
  if (dt != MLA_DTYPE_F32 && dt != MLA_DTYPE_BF16) return 0;
  return use_mfma(dt, d, r) ? mla::prefill_mfma_workspace(B, T, H, d, r)
                            : mla::prefill_simt_workspace(B, T, H, d, r);
}

size_t mla_latent_attn_masked_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt) {
  const size_t base = mla_latent_attn_workspace_size(B, T, H, d, r, dt);
  if (base == 0) return 0;
  return use_mfma(dt, d, r) ? base + mla::key_mask_workspace(B, T, r) : base;
}

size_t mla_latent_attn_full_workspace_size(int B, int T, int D, int H, int d, int r, mla_dtype dt) {
  if (D < 1) return 0;
  const size_t attn = mla_latent_attn_workspace_size(B, T, H, d, r, dt);
  if (attn == 0) return 0;
  const size_t a = (attn + 255) / 256 * 256;
  return dt == MLA_DTYPE_BF16 && mla::down_mfma_supported(D, r) ? a + mla::down_mfma_workspace(D, r) : a;
}

}  // extern "C"

namespace {

// The producer of kv_latent in the full path: kv_latent = hidden @ w_down.
struct DownProj {
  const void* hidden;
  const void* w_down;
  int D;
};

// Prefill with (key_mask) or without a key mask; with `down`, kv_latent is
// first written by the down-projection.  Every check runs before the first
// launch.
mla_status prefill_common(const void* q, const void* kv_latent, const uint8_t* key_mask, const void* w_up_k,
                          const void* w_up_v, void* out, int B, int T, int H, int d, int r, float scale,
                          mla_dtype dt, void* workspace, size_t workspace_bytes, void* stream,
                          const DownProj* down = nullptr) {
  if (!q || !kv_latent || !w_up_k || !w_up_v || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  mla_status s = check_dims(B, T, H, d, r, dt, "T");
  if (s != MLA_OK) return s;
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!aligned16(q) || !aligned16(kv_latent) || !aligned16(w_up_k) || !aligned16(w_up_v) ||
      !aligned16(out) || !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (down) {
    if (!down->hidden || !down->w_down) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
    if (down->D < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "D must be positive (got %d)", down->D);
    if (!aligned16(down->hidden) || !aligned16(down->w_down))
      return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if ((double)B * T * down->D >= 9.0e15) return fail(MLA_ERR_UNSUPPORTED, "problem too large");
  }
  const size_t need = down ? mla_latent_attn_full_workspace_size(B, T, down->D, H, d, r, dt)
                      : key_mask ? mla_latent_attn_masked_workspace_size(B, T, H, d, r, dt)
                                 : mla_latent_attn_workspace_size(B, T, H, d, r, dt);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  if (use_mfma(dt, d, r)) {
    size_t limit = 0;
    s = device_lds_limit(&limit);
    if (s != MLA_OK) return s;
    if (mla::flash_lds_bytes(r) > limit)
      return fail(MLA_ERR_UNSUPPORTED, "prefill needs %zu bytes of LDS per block, device allows %zu",
                  mla::flash_lds_bytes(r), limit);
  }
  if (down) {
    hipError_t e;
    if (dt == MLA_DTYPE_BF16 && mla::down_mfma_supported(down->D, r)) {
      const size_t a = (mla_latent_attn_workspace_size(B, T, H, d, r, dt) + 255) / 256 * 256;
      e = mla::down_mfma((const uint16_t*)down->hidden, (const uint16_t*)down->w_down, (uint16_t*)kv_latent, B * T,
                         down->D, r, (char*)workspace + a, st);
    } else {
      e = mla::down_proj(dt == MLA_DTYPE_BF16, down->hidden, down->w_down, (void*)kv_latent, B * T, down->D, r, st);
    }
    if (e != hipSuccess) return launched(e, "down-projection launch");
  }
  if (use_mfma(dt, d, r))
    return launched(mla::prefill_mfma(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r,
                                      (float)(scale * kLog2e), key_mask, workspace, st),
                    "prefill launch");
  return launched(mla::prefill_simt(dt == MLA_DTYPE_BF16, q, kv_latent, w_up_k, w_up_v, out, B, T,
                                    H, d, r, scale, key_mask, workspace, st),
                  "prefill launch");
}

}  // namespace

extern "C" {

mla_status mla_latent_attn_fwd(const void* q, const void* kv_latent, const void* w_up_k,
                               const void* w_up_v, void* out, int B, int T, int H, int d, int r,
                               float scale, mla_dtype dt, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return prefill_common(q, kv_latent, nullptr, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, workspace,
                        workspace_bytes, stream);
}

mla_status mla_latent_attn_fwd_full(const void* hidden, const void* w_down, const void* q, const void* w_up_k,
                                    const void* w_up_v, void* kv_latent, void* out, int B, int T, int D, int H,
                                    int d, int r, float scale, mla_dtype dt, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const DownProj down{hidden, w_down, D};
  return prefill_common(q, kv_latent, nullptr, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, workspace,
                        workspace_bytes, stream, &down);
}

mla_status mla_latent_attn_fwd_masked(const void* q, const void* kv_latent, const uint8_t* key_mask,
                                      const void* w_up_k, const void* w_up_v, void* out, int B, int T, int H,
                                      int d, int r, float scale, mla_dtype dt, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!key_mask) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  return prefill_common(q, kv_latent, key_mask, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, workspace,
                        workspace_bytes, stream);
}

size_t mla_latent_attn_unabsorbed_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt) {
  if (B < 1 || T < 1 || H < 1 || d < 1 || r < 1) return 0;
  if (dt != MLA_DTYPE_BF16 || !mla::unabsorbed_supported(d, r)) return 0;
  return mla::prefill_unabsorbed_workspace(B, T, H, d, r);
}

mla_status mla_latent_attn_fwd_unabsorbed(const void* q, const void* kv_latent, const void* w_up_k,
                                          const void* w_up_v, void* out, int B, int T, int H, int d, int r,
                                          float scale, mla_dtype dt, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  if (!q || !kv_latent || !w_up_k || !w_up_v || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  mla_status s = check_dims(B, T, H, d, r, dt, "T");
  if (s != MLA_OK) return s;
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!aligned16(q) || !aligned16(kv_latent) || !aligned16(w_up_k) || !aligned16(w_up_v) ||
      !aligned16(out) || !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (dt != MLA_DTYPE_BF16 || !mla::unabsorbed_supported(d, r))
    return fail(MLA_ERR_UNSUPPORTED, "unabsorbed prefill covers bf16 with d = 128, r in {128, 256, 512} "
                "(got %s, d=%d, r=%d)", dt == MLA_DTYPE_BF16 ? "bf16" : "float32", d, r);
  const size_t need = mla_latent_attn_unabsorbed_workspace_size(B, T, H, d, r, dt);
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  size_t limit = 0;
  s = device_lds_limit(&limit);
  if (s != MLA_OK) return s;
  if (mla::unabsorbed_lds_bytes(d) > limit)
    return fail(MLA_ERR_UNSUPPORTED, "unabsorbed prefill needs %zu bytes of LDS per block, device allows %zu",
                mla::unabsorbed_lds_bytes(d), limit);
  return launched(mla::prefill_unabsorbed(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r,
                                          (float)(scale * kLog2e), workspace, (hipStream_t)stream),
                  "unabsorbed prefill launch");
}

int mla_latent_attn_auto_form(int B, int T, int H, int d, int r, mla_dtype dt) {
  (void)B;
  (void)T;
  (void)H;
  return dt == MLA_DTYPE_BF16 && mla::unabsorbed_supported(d, r) && r > d ? 1 : 0;
}

size_t mla_latent_attn_auto_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt) {
  return mla_latent_attn_auto_form(B, T, H, d, r, dt) ? mla_latent_attn_unabsorbed_workspace_size(B, T, H, d, r, dt)
                                                      : mla_latent_attn_workspace_size(B, T, H, d, r, dt);
}

mla_status mla_latent_attn_fwd_auto(const void* q, const void* kv_latent, const void* w_up_k, const void* w_up_v,
                                    void* out, int B, int T, int H, int d, int r, float scale, mla_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (mla_latent_attn_auto_form(B, T, H, d, r, dt))
    return mla_latent_attn_fwd_unabsorbed(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, workspace,
                                          workspace_bytes, stream);
  return mla_latent_attn_fwd(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, workspace,
                             workspace_bytes, stream);
}

size_t mla_decode_workspace_size(int B, int Tmax, int H, int d, int r, mla_dtype dt) {
  if (B < 1 || Tmax < 1 || H < 1 || d < 1 || r < 1) return 0;
  if (dt != MLA_DTYPE_F32 && dt != MLA_DTYPE_BF16) return 0;
  return use_mfma(dt, d, r) ? mla::decode_mfma_workspace(B, Tmax, H, d, r)
                            : mla::decode_simt_workspace(B, Tmax, H, d, r);
}

}  // extern "C"

// The fixed decode scratch of mla_decode_fwd_noalloc: device memory the
// library holds from load to process end (one copy per device, at its own
// address), so that call allocates nothing.  Host code never uses this name
// as an address: it is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

// The device address of `scratch` on the calling thread's current device,
// looked up on the first call on each device and kept.
mla_status scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return MLA_OK;
}

// Decode over a padded cache (lens, rows = Tmax per sequence) or a packed one
// (cu, rows = the cache's total row count).  With `noalloc` the workspace is
// the library's fixed scratch (workspace and workspace_bytes are ignored),
// laid out with the partial slots this call's chunk count needs.
mla_status decode_common(const void* q, const void* kv_latent, const int32_t* seq_lens, const int32_t* cu,
                         const void* w_up_k, const void* w_up_v, void* out, int B, int rows, int H, int d, int r,
                         float scale, mla_dtype dt, void* workspace, size_t workspace_bytes, void* stream,
                         bool noalloc = false) {
  if (!q || !kv_latent || !(seq_lens || cu) || !w_up_k || !w_up_v || !out || !(workspace || noalloc))
    return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  const int32_t* ints = cu ? cu : seq_lens;
  if (cu && rows < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "total must be positive (got %d)", rows);
  // B * rows < 2^31 for both layouts: the device prefix of the per-sequence
  // lengths (each clamped to at most `rows`) is int32
  mla_status s = check_dims(B, rows, H, d, r, dt, cu ? "total" : "Tmax");
  if (s != MLA_OK) return s;
  if (!std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!aligned16(q) || !aligned16(kv_latent) || !aligned16(w_up_k) || !aligned16(w_up_v) ||
      !aligned16(out) || (!noalloc && !aligned16(workspace)) || ((uintptr_t)ints & 3u))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned (lengths 4-byte)");
  // partial slots of the matrix-core path: the caller's workspace is sized
  // for the most chunks a call can take, the fixed scratch for this call's
  size_t slots = mla::decode_max_splits(B);
  if (noalloc) {
    slots = (size_t)mla::decode_chunks(H) + B;
    const size_t need = use_mfma(dt, d, r) ? mla::decode_mfma_bytes(B, H, d, r, slots)
                                           : mla::decode_simt_workspace(B, rows, H, d, r);
    if (need > MLA_NOALLOC_SCRATCH_BYTES)
      return fail(MLA_ERR_UNSUPPORTED, "decode needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                  (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  } else {
    const size_t need = mla_decode_workspace_size(B, rows, H, d, r, dt);
    if (workspace_bytes < need)
      return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  }
  hipStream_t st = (hipStream_t)stream;
  if (use_mfma(dt, d, r)) {
    size_t limit = 0;
    s = device_lds_limit(&limit);
    if (s != MLA_OK) return s;
    if (mla::decode_lds_bytes(r) > limit)
      return fail(MLA_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS per block, device allows %zu",
                  mla::decode_lds_bytes(r), limit);
  }
  if (noalloc) {
    s = scratch_address(&workspace);
    if (s != MLA_OK) return s;
  }
  if (use_mfma(dt, d, r)) {
    return launched(mla::decode_mfma(q, kv_latent, seq_lens, cu, w_up_k, w_up_v, out, B, rows, H, d, r,
                                     (float)(scale * kLog2e), workspace, slots, st),
                    "decode launch");
  }
  return launched(mla::decode_simt(dt == MLA_DTYPE_BF16, q, kv_latent, seq_lens, cu, w_up_k, w_up_v,
                                   out, B, rows, H, d, r, scale, workspace, st),
                  "decode launch");
}

}  // namespace

extern "C" {

mla_status mla_decode_fwd(const void* q, const void* kv_latent, const int32_t* seq_lens,
                          const void* w_up_k, const void* w_up_v, void* out, int B, int Tmax,
                          int H, int d, int r, float scale, mla_dtype dt, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!seq_lens) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  return decode_common(q, kv_latent, seq_lens, nullptr, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt,
                       workspace, workspace_bytes, stream);
}

mla_status mla_decode_fwd_noalloc(const void* q, const void* kv_latent, const int32_t* seq_lens, const void* w_up_k,
                                  const void* w_up_v, void* out, int B, int Tmax, int H, int d, int r, float scale,
                                  mla_dtype dt, void* stream) {
  if (!seq_lens) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  return decode_common(q, kv_latent, seq_lens, nullptr, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt, nullptr,
                       0, stream, /*noalloc=*/true);
}

size_t mla_decode_varlen_workspace_size(int B, int total, int H, int d, int r, mla_dtype dt) {
  return mla_decode_workspace_size(B, total, H, d, r, dt);
}

mla_status mla_decode_varlen_fwd(const void* q, const void* kv_latent, const int32_t* cu_seqlens,
                                 const void* w_up_k, const void* w_up_v, void* out, int B, int total,
                                 int H, int d, int r, float scale, mla_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  return decode_common(q, kv_latent, nullptr, cu_seqlens, w_up_k, w_up_v, out, B, total, H, d, r, scale, dt,
                       workspace, workspace_bytes, stream);
}

mla_status mla_decode_set_splits(int splits) {
  if (splits < 0 || splits > mla::decode_split_cap())
    return fail(MLA_ERR_INVALID_ARGUMENT, "splits must be in [0, %d] (got %d)", mla::decode_split_cap(), splits);
  mla::set_decode_splits(splits);
  return ok();
}

mla_status mla_set_lds_limit_override(size_t bytes) {
  g_lds_limit_override.store(bytes, std::memory_order_relaxed);
  return ok();
}

mla_status mla_kv_append(void* kv_cache, int32_t* seq_lens, const void* new_latent, int B, int Tmax, int r,
                         mla_dtype dt, void* stream) {
  if (!kv_cache || !seq_lens || !new_latent) return fail(MLA_ERR_INVALID_ARGUMENT, "null pointer");
  if (B < 1 || Tmax < 1 || r < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d Tmax=%d r=%d)", B, Tmax, r);
  if (dt != MLA_DTYPE_F32 && dt != MLA_DTYPE_BF16) return fail(MLA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  if (!aligned16(kv_cache) || !aligned16(new_latent) || ((uintptr_t)seq_lens & 3u))
    return fail(MLA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned (seq_lens 4-byte)");
  if ((double)B * Tmax >= 2147483647.0 || (double)B * Tmax * r >= 9.0e15)
    return fail(MLA_ERR_UNSUPPORTED, "problem too large");
  return launched(mla::kv_append(dt == MLA_DTYPE_BF16, kv_cache, seq_lens, new_latent, B, Tmax, r,
                                 (hipStream_t)stream),
                  "kv append launch");
}

}  // extern "C"

namespace mla {
bool mfma_supported(int d, int r) {
  return (r == 128 || r == 256 || r == 512) && (d == 32 || d == 64 || d == 128 || d == 256);
}
}  // namespace mla
