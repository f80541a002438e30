/* mla.h -- C ABI of the MI355X (gfx950) latent causal attention library.
 *
 * The operation (POPCORNBENCH page FW-GLM-5-1 l2_p31, the latent attention
 * problem and its algorithm restatement): for batch b, head h, query t and
 * every key s <= t,
 *     k_s = kv_latent[b,s,:] @ w_up_k[:,h,:],   v_s = kv_latent[b,s,:] @ w_up_v[:,h,:],
 *     logit_s = scale * <q[b,t,h,:], k_s>,      out[b,t,h,:] = sum_s softmax(logit)_s * v_s.
 * The optional producer of kv_latent is the KV down-projection of
 * POPCORNBENCH page FW-GLM-5-1 l2_p1 (its list of operations):
 *     kv_latent = hidden @ w_down.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never frees, retains or allocates it, and allocates no device memory of
 *     its own: scratch space is the caller's `workspace`, sized by the
 *     matching *_workspace_size query.
 *   - Tensors are dense and row-major with the shapes given below; all float
 *     tensors of one call share the dtype `dt` (float32 or bf16); seq_lens is
 *     int32.  Float pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued on it; no call synchronises the host.  Calls enqueue kernel
 *     launches only (no memset, copy or allocation), so a stream capture
 *     may record them into a HIP graph for replay; the first call of each
 *     kernel shape sets its LDS attribute and should precede the capture.
 *   - Arguments are checked before anything is enqueued.  A null pointer,
 *     a non-positive size or misalignment returns MLA_ERR_INVALID_ARGUMENT;
 *     a shape the kernels do not cover returns MLA_ERR_UNSUPPORTED; a
 *     workspace smaller than required returns MLA_ERR_WORKSPACE; a failed
 *     launch returns MLA_ERR_HIP.  mla_last_error() then describes the
 *     failure (per calling thread).  Nothing is written on error.
 *   - Arithmetic: float32 inputs are computed in float32; bf16 inputs use
 *     bf16 matrix-core operands with float32 accumulation and a float32
 *     softmax.  Results are deterministic run to run.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE = 3,
  MLA_ERR_HIP = 4
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* Largest latent rank r and head dim d any path accepts. */
#define MLA_MAX_RANK 1024
#define MLA_MAX_HEAD_DIM 256

/* KV down-projection (page FW-GLM-5-1 l2_p1, operations list):
 *   kv_latent[b,t,:] = hidden[b,t,:] @ w_down.
 * hidden [B,T,D], w_down [D,r] (row-major, used without transpose),
 * kv_latent [B,T,r] (output, same dtype).  1 <= r <= MLA_MAX_RANK. */
mla_status mla_down_proj(const void* hidden, const void* w_down, void* kv_latent,
                         int B, int T, int D, int r, mla_dtype dt, void* stream);

/* Bytes of workspace mla_latent_attn_fwd needs for this shape (0 on bad sizes). */
size_t mla_latent_attn_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt);

/* Causal latent attention, prefill (page FW-GLM-5-1 l2_p31, algorithm
 * restatement; keys s = 0..t inclusive):
 *   q [B,T,H,d], kv_latent [B,T,r], w_up_k / w_up_v [r,H,d]  (inputs),
 *   out [B,T,H,d] (output, dtype of q).
 * `scale` multiplies every logit (1/sqrt(d) is the usual choice).
 * Computed in absorbed form (q_lat = w_up_k[:,h,:] q, attention over the
 * latents, then the w_up_v up-projection), which equals the definition up to
 * rounding.  workspace must hold mla_latent_attn_workspace_size() bytes. */
mla_status mla_latent_attn_fwd(const void* q, const void* kv_latent, const void* w_up_k,
                               const void* w_up_v, void* out, int B, int T, int H, int d,
                               int r, float scale, mla_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_latent_attn_fwd_full needs for this shape (0 on bad sizes). */
size_t mla_latent_attn_full_workspace_size(int B, int T, int D, int H, int d, int r, mla_dtype dt);

/* The full path in one call: the KV down-projection (page FW-GLM-5-1 l2_p1,
 * operations list) writes the latent cache, then the causal prefill of
 * mla_latent_attn_fwd runs over it (page FW-GLM-5-1 l2_p31):
 *   kv_latent[b,t,:] = hidden[b,t,:] @ w_down,   out = attention(q, kv_latent).
 *   hidden [B,T,D], w_down [D,r] (inputs), kv_latent [B,T,r] (OUTPUT: the
 *   latent cache, stored in dt and then read back by the attention, so a
 *   later decode can use it as its cache); the rest as mla_latent_attn_fwd.
 * bf16 with D % 64 == 0 and r % 128 == 0 runs the down-projection on the
 * matrix cores (bf16 operands, float32 accumulation); other shapes and
 * float32 use the float32 vector path of mla_down_proj.  workspace must hold
 * mla_latent_attn_full_workspace_size() bytes.  Equal, bit for bit, to
 * mla_down_proj followed by mla_latent_attn_fwd when both take the vector
 * down-projection path. */
mla_status mla_latent_attn_fwd_full(const void* hidden, const void* w_down, const void* q, const void* w_up_k,
                                    const void* w_up_v, void* kv_latent, void* out, int B, int T, int D, int H,
                                    int d, int r, float scale, mla_dtype dt, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Bytes of workspace mla_latent_attn_fwd_masked needs for this shape (0 on bad sizes). */
size_t mla_latent_attn_masked_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt);

/* Causal prefill with a key mask: mla_latent_attn_fwd where query t of batch
 * b attends only the keys s <= t with key_mask[b,s] != 0.  A masked key's
 * logit is -infinity before the softmax (the masked-score fill of
 * POPCORNBENCH page Kimi-K2.6 l2_p29, its attention walk-through), so it
 * gets weight 0; a query row with no visible key has an all -infinity row,
 * whose softmax is undefined, and its output is NaN (what that page's
 * analysis of fully masked rows finds such a softmax returns).
 *   key_mask [B,T] uint8 in DEVICE memory (nonzero = visible), any alignment;
 *   every other argument as mla_latent_attn_fwd.  workspace must hold
 *   mla_latent_attn_masked_workspace_size() bytes.  With an all-nonzero mask
 *   the result equals mla_latent_attn_fwd's bit for bit. */
mla_status mla_latent_attn_fwd_masked(const void* q, const void* kv_latent, const uint8_t* key_mask,
                                      const void* w_up_k, const void* w_up_v, void* out, int B, int T, int H,
                                      int d, int r, float scale, mla_dtype dt, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_latent_attn_fwd_unabsorbed needs for this shape
 * (0 on bad sizes or a shape it does not cover). */
size_t mla_latent_attn_unabsorbed_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt);

/* The same causal prefill as mla_latent_attn_fwd, same arguments and result
 * up to rounding, computed in unabsorbed form: k and v of every head are
 * materialised from kv_latent (page FW-GLM-5-1 l2_p1, operations list: the
 * up-projections of the latent to keys and values), then causal attention
 * runs over them with d-wide products.  At r > d this takes r/d times fewer
 * matrix operations than the absorbed form, at the price of a workspace of
 * 2*B*T*H*d elements (k and v).  Covers bf16 with d = 128 and
 * r in {128, 256, 512}; other shapes and float32 return MLA_ERR_UNSUPPORTED.
 * The logit scale is folded into the stored k (rounded once to bf16). */
mla_status mla_latent_attn_fwd_unabsorbed(const void* q, const void* kv_latent, const void* w_up_k,
                                          const void* w_up_v, void* out, int B, int T, int H, int d,
                                          int r, float scale, mla_dtype dt, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* The form mla_latent_attn_fwd_auto takes for this shape: 1 for the
 * unabsorbed form (bf16, a shape mla_latent_attn_fwd_unabsorbed covers, and
 * r > d, where materialising k and v takes r/d times fewer matrix
 * operations), 0 for the absorbed form otherwise. */
int mla_latent_attn_auto_form(int B, int T, int H, int d, int r, mla_dtype dt);

/* Bytes of workspace mla_latent_attn_fwd_auto needs (that of the form it takes). */
size_t mla_latent_attn_auto_workspace_size(int B, int T, int H, int d, int r, mla_dtype dt);

/* The causal prefill of mla_latent_attn_fwd (same arguments, same result up
 * to rounding) in the form mla_latent_attn_auto_form picks for the shape:
 * the absorbed form of mla_latent_attn_fwd or the unabsorbed form of
 * mla_latent_attn_fwd_unabsorbed, whose result it returns bit for bit. */
mla_status mla_latent_attn_fwd_auto(const void* q, const void* kv_latent, const void* w_up_k, const void* w_up_v,
                                    void* out, int B, int T, int H, int d, int r, float scale, mla_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mla_decode_fwd needs for this shape (0 on bad sizes). */
size_t mla_decode_workspace_size(int B, int Tmax, int H, int d, int r, mla_dtype dt);

/* Decode: one query per sequence (the same definition for the last position
 * of a sequence of length L_b = seq_lens[b]: it attends cached latents
 * 0..L_b-1).
 *   q [B,1,H,d], kv_latent [B,Tmax,r] (rows >= L_b are never read),
 *   seq_lens [B] int32 in DEVICE memory with 1 <= L_b <= Tmax,
 *   w_up_k / w_up_v [r,H,d], out [B,1,H,d].
 * Long caches are split over workgroups and the partial softmax states are
 * merged by log-sum-exp.  A length outside [1, Tmax] is clamped to it (the
 * device-resident lengths are not inspected by the host). */
mla_status mla_decode_fwd(const void* q, const void* kv_latent, const int32_t* seq_lens,
                          const void* w_up_k, const void* w_up_v, void* out, int B, int Tmax,
                          int H, int d, int r, float scale, mla_dtype dt, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch behind mla_decode_fwd_noalloc (64 MiB). */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* mla_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (but workspace), same
 * kernels and the same result, bit for bit, as mla_decode_fwd.  Its scratch
 * (absorbed queries, W_uv^T, the split's partial states and the length
 * prefix) lives in a fixed MLA_NOALLOC_SCRATCH_BYTES device array the
 * library holds on each device until the process ends; the call allocates
 * nothing and needs no cleared memory.  A shape whose scratch would exceed
 * it returns MLA_ERR_UNSUPPORTED (bf16_decode's 64 sequences x 32 heads at
 * r = 512 take about 17 MiB at the default chunk count).  Every call on a
 * device shares that device's scratch: calls that overlap on one device
 * (other streams, other threads) race and give wrong results; calls on one
 * stream are ordered and safe.  The first call on each device looks up the
 * scratch's device address (a HIP query), so make one before a capture. */
mla_status mla_decode_fwd_noalloc(const void* q, const void* kv_latent, const int32_t* seq_lens,
                                  const void* w_up_k, const void* w_up_v, void* out, int B, int Tmax,
                                  int H, int d, int r, float scale, mla_dtype dt, void* stream);

/* Bytes of workspace mla_decode_varlen_fwd needs for this shape (0 on bad sizes). */
size_t mla_decode_varlen_workspace_size(int B, int total, int H, int d, int r, mla_dtype dt);

/* Decode over a packed (variable-length) latent cache: the same computation
 * as mla_decode_fwd, with sequence b's cached latents in rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of kv_latent [total, r] instead of a
 * padded [B, Tmax, r].
 *   cu_seqlens [B+1] int32 in DEVICE memory, 0 <= cu_seqlens[b] < cu_seqlens[b+1] <= total
 *   (every sequence non-empty); B * total must stay below 2^31
 *   (MLA_ERR_UNSUPPORTED otherwise), as B * Tmax for the padded layout.  The host does not inspect it; out of that
 *   contract each sequence is clamped into the cache (first row into [0, total),
 *   length into [1, total - first row]), so no read leaves kv_latent, but the
 *   result is unspecified.
 * Everything else as mla_decode_fwd; results are bit-identical to
 * mla_decode_fwd on the same latents laid out padded. */
mla_status mla_decode_varlen_fwd(const void* q, const void* kv_latent, const int32_t* cu_seqlens,
                                 const void* w_up_k, const void* w_up_v, void* out, int B, int total,
                                 int H, int d, int r, float scale, mla_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Append one latent per sequence to a padded decode cache, on the device:
 *   kv_cache [B, Tmax, r] (in/out), seq_lens [B] int32 DEVICE (in/out),
 *   new_latent [B, r] (e.g. from mla_down_proj of the new token).
 * For each b with 0 <= seq_lens[b] < Tmax: kv_cache[b, seq_lens[b], :] =
 * new_latent[b, :], then seq_lens[b] += 1.  A sequence whose cache is full
 * (or whose length is outside [0, Tmax)) is left unchanged; nothing else of
 * the cache is written.  The lengths stay on the device, so a decode step
 * (append, then mla_decode_fwd) needs no host round trip.  The position the
 * token is written to is the cache length before the call; it becomes part
 * of the attended keys of the following decode. */
mla_status mla_kv_append(void* kv_cache, int32_t* seq_lens, const void* new_latent, int B, int Tmax,
                         int r, mla_dtype dt, void* stream);

/* The number of chunks the decode split cuts the concatenated caches of one
 * call into, per group of 32 heads, for later mla_decode_fwd and
 * mla_decode_varlen_fwd calls of this process: 0 (the default) takes one
 * chunk per compute unit; 1 .. 1024 fixes the count.  The result is the same
 * up to rounding for every count (the partial softmax states are merged by
 * log-sum-exp, an associative combination: POPCORNBENCH page Kimi-K2.6
 * l2_p29, its online-softmax derivation); it exists for tuning and for
 * testing that invariance.  Returns MLA_ERR_INVALID_ARGUMENT outside
 * [0, 1024].  Process-wide; safe to call from any thread, but calls that
 * overlap a decode on another thread may see either count. */
mla_status mla_decode_set_splits(int splits);

/* Replace the device's per-block LDS limit that the argument checks compare
 * each kernel's LDS need against (0, the default, queries the device).  A
 * limit below a kernel's need makes the call fail with MLA_ERR_UNSUPPORTED
 * before anything is enqueued -- the check that keeps a launch from failing
 * on shared memory, as the KV-compression page's kernel did (POPCORNBENCH
 * page FW-GLM-5-1 l2_p1, its launch-failure passage).  For testing that
 * error path, including on a host without a device; process-wide. */
mla_status mla_set_lds_limit_override(size_t bytes);

/* Per-kernel timing, for benchmarking (not part of the computation).
 * mla_profile_enable(1) makes every later kernel launch of the library record
 * a pair of HIP events on its stream; mla_profile_enable(0) stops it.
 * mla_profile_collect() waits for the recorded events, and returns, for each
 * kernel name seen (up to `max`), the summed elapsed milliseconds and launch
 * count since the previous collect; *n receives the number of entries.
 * names[i] point to library-owned strings valid until the next collect.
 * Not meant for concurrent use from several threads. */
mla_status mla_profile_enable(int on);
mla_status mla_profile_collect(const char** names, double* total_ms, int* counts, int max, int* n);

/* Static description of a status code. */
const char* mla_status_string(mla_status s);

/* Detail of the last failed call on this thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
