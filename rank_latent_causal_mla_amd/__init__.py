"""Python binding of libmla.so, the gfx950 latent causal attention library.

Argument marshalling only: each function below calls the C entry point of
the same name in include/mla.h; every step of the computation runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.
A missing library is an error -- there is no other implementation behind
these names.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARGUMENT, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = range(5)
MLA_DTYPE_F32, MLA_DTYPE_BF16 = 0, 1

EXPORTED = ("mla_down_proj", "mla_latent_attn_workspace_size", "mla_latent_attn_fwd",
            "mla_latent_attn_masked_workspace_size", "mla_latent_attn_fwd_masked",
            "mla_latent_attn_full_workspace_size", "mla_latent_attn_fwd_full",
            "mla_latent_attn_auto_form", "mla_latent_attn_auto_workspace_size", "mla_latent_attn_fwd_auto",
            "mla_latent_attn_unabsorbed_workspace_size", "mla_latent_attn_fwd_unabsorbed",
            "mla_decode_workspace_size", "mla_decode_fwd", "mla_decode_varlen_workspace_size",
            "mla_decode_fwd_noalloc", "mla_decode_varlen_fwd", "mla_kv_append", "mla_decode_set_splits",
            "mla_set_lds_limit_override",
            "mla_profile_enable", "mla_profile_collect", "mla_status_string", "mla_last_error")

_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def load():
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with rank_latent_causal_mla_amd.build.build()")
    # Let torch bring up the GPU runtime before the library's kernels are
    # registered: loading the library first has left its own HIP calls
    # without a visible device once torch initialised afterwards.
    try:
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mla_down_proj.restype = i32
    lib.mla_down_proj.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.mla_latent_attn_workspace_size.restype = sz
    lib.mla_latent_attn_workspace_size.argtypes = [i32] * 6
    lib.mla_latent_attn_fwd.restype = i32
    lib.mla_latent_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mla_latent_attn_auto_form.restype = i32
    lib.mla_latent_attn_auto_form.argtypes = [i32] * 6
    lib.mla_latent_attn_auto_workspace_size.restype = sz
    lib.mla_latent_attn_auto_workspace_size.argtypes = [i32] * 6
    lib.mla_latent_attn_fwd_auto.restype = i32
    lib.mla_latent_attn_fwd_auto.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mla_latent_attn_full_workspace_size.restype = sz
    lib.mla_latent_attn_full_workspace_size.argtypes = [i32] * 7
    lib.mla_latent_attn_fwd_full.restype = i32
    lib.mla_latent_attn_fwd_full.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                                             sz, vp]
    lib.mla_latent_attn_masked_workspace_size.restype = sz
    lib.mla_latent_attn_masked_workspace_size.argtypes = [i32] * 6
    lib.mla_latent_attn_fwd_masked.restype = i32
    lib.mla_latent_attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz,
                                               vp]
    lib.mla_latent_attn_unabsorbed_workspace_size.restype = sz
    lib.mla_latent_attn_unabsorbed_workspace_size.argtypes = [i32] * 6
    lib.mla_latent_attn_fwd_unabsorbed.restype = i32
    lib.mla_latent_attn_fwd_unabsorbed.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode_workspace_size.argtypes = [i32] * 6
    lib.mla_decode_fwd.restype = i32
    lib.mla_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mla_decode_fwd_noalloc.restype = i32
    lib.mla_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.mla_decode_varlen_workspace_size.restype = sz
    lib.mla_decode_varlen_workspace_size.argtypes = [i32] * 6
    lib.mla_decode_varlen_fwd.restype = i32
    lib.mla_decode_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.mla_kv_append.restype = i32
    lib.mla_kv_append.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    lib.mla_decode_set_splits.restype = i32
    lib.mla_decode_set_splits.argtypes = [i32]
    lib.mla_set_lds_limit_override.restype = i32
    lib.mla_set_lds_limit_override.argtypes = [sz]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [i32]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_profile_enable.restype = i32
    lib.mla_profile_enable.argtypes = [i32]
    lib.mla_profile_collect.restype = i32
    lib.mla_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int), i32, ctypes.POINTER(ctypes.c_int)]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def last_error() -> str:
    return load().mla_last_error().decode()


def _check(status: int):
    if status != MLA_OK:
        raise MLAError(status, last_error())


# ---- raw C ABI (plain integers / pointers)

def mla_down_proj_raw(hidden, w_down, kv_latent, B, T, D, r, dt, stream=0):
    return load().mla_down_proj(hidden, w_down, kv_latent, B, T, D, r, dt, stream)


def mla_latent_attn_workspace_size(B, T, H, d, r, dt):
    return int(load().mla_latent_attn_workspace_size(B, T, H, d, r, dt))


def mla_latent_attn_auto_form(B, T, H, d, r, dt):
    """1 when mla_latent_attn_fwd_auto takes the unabsorbed form for this shape, else 0."""
    return int(load().mla_latent_attn_auto_form(B, T, H, d, r, dt))


def mla_latent_attn_auto_workspace_size(B, T, H, d, r, dt):
    return int(load().mla_latent_attn_auto_workspace_size(B, T, H, d, r, dt))


def mla_latent_attn_fwd_auto_raw(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws, ws_bytes, stream=0):
    return load().mla_latent_attn_fwd_auto(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws, ws_bytes,
                                           stream)


def mla_latent_attn_full_workspace_size(B, T, D, H, d, r, dt):
    return int(load().mla_latent_attn_full_workspace_size(B, T, D, H, d, r, dt))


def mla_latent_attn_fwd_full_raw(hidden, w_down, q, w_up_k, w_up_v, kv_latent, out, B, T, D, H, d, r, scale, dt, ws,
                                 ws_bytes, stream=0):
    return load().mla_latent_attn_fwd_full(hidden, w_down, q, w_up_k, w_up_v, kv_latent, out, B, T, D, H, d, r,
                                           scale, dt, ws, ws_bytes, stream)


def mla_latent_attn_masked_workspace_size(B, T, H, d, r, dt):
    return int(load().mla_latent_attn_masked_workspace_size(B, T, H, d, r, dt))


def mla_latent_attn_unabsorbed_workspace_size(B, T, H, d, r, dt):
    return int(load().mla_latent_attn_unabsorbed_workspace_size(B, T, H, d, r, dt))


def mla_decode_workspace_size(B, Tmax, H, d, r, dt):
    return int(load().mla_decode_workspace_size(B, Tmax, H, d, r, dt))


def mla_latent_attn_fwd_raw(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws, ws_bytes, stream=0):
    return load().mla_latent_attn_fwd(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws,
                                      ws_bytes, stream)


def mla_latent_attn_fwd_masked_raw(q, kv_latent, key_mask, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws,
                                   ws_bytes, stream=0):
    return load().mla_latent_attn_fwd_masked(q, kv_latent, key_mask, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt,
                                             ws, ws_bytes, stream)


def mla_latent_attn_fwd_unabsorbed_raw(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws, ws_bytes,
                                       stream=0):
    return load().mla_latent_attn_fwd_unabsorbed(q, kv_latent, w_up_k, w_up_v, out, B, T, H, d, r, scale, dt, ws,
                                                 ws_bytes, stream)


def mla_decode_fwd_raw(q, kv_latent, seq_lens, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt, ws,
                       ws_bytes, stream=0):
    return load().mla_decode_fwd(q, kv_latent, seq_lens, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt, ws,
                                 ws_bytes, stream)


def mla_decode_fwd_noalloc_raw(q, kv_latent, seq_lens, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt, stream=0):
    return load().mla_decode_fwd_noalloc(q, kv_latent, seq_lens, w_up_k, w_up_v, out, B, Tmax, H, d, r, scale, dt,
                                         stream)


def mla_decode_varlen_workspace_size(B, total, H, d, r, dt):
    return int(load().mla_decode_varlen_workspace_size(B, total, H, d, r, dt))


def mla_decode_varlen_fwd_raw(q, kv_latent, cu_seqlens, w_up_k, w_up_v, out, B, total, H, d, r, scale, dt, ws,
                              ws_bytes, stream=0):
    return load().mla_decode_varlen_fwd(q, kv_latent, cu_seqlens, w_up_k, w_up_v, out, B, total, H, d, r, scale,
                                        dt, ws, ws_bytes, stream)


def mla_kv_append_raw(kv_cache, seq_lens, new_latent, B, Tmax, r, dt, stream=0):
    return load().mla_kv_append(kv_cache, seq_lens, new_latent, B, Tmax, r, dt, stream)


def mla_decode_set_splits(splits: int = 0):
    """Chunks per 32-head group of the decode split for later decode calls (0 = one per compute unit)."""
    _check(load().mla_decode_set_splits(int(splits)))


def mla_set_lds_limit_override(nbytes: int = 0):
    """Per-block LDS limit the argument checks use instead of the device's (0 = query the device)."""
    _check(load().mla_set_lds_limit_override(int(nbytes)))


def mla_profile_enable(on: bool = True):
    _check(load().mla_profile_enable(1 if on else 0))


def mla_profile_collect(max_entries: int = 64) -> dict:
    """{kernel name: (total ms, launches)} since the previous collect."""
    names = (ctypes.c_char_p * max_entries)()
    tot = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_int * max_entries)()
    n = ctypes.c_int(0)
    _check(load().mla_profile_collect(names, tot, cnt, max_entries, ctypes.byref(n)))
    return {names[i].decode(): (tot[i], cnt[i]) for i in range(n.value) if cnt[i]}


# ---- torch-tensor marshalling (same names as the C entry points)

def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _shaped(t, shape, dtype, name):
    """A caller-supplied output must have exactly the shape and dtype the call writes."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {list(shape)} {dtype}, got {list(t.shape)} {t.dtype}")


# The C ABI takes plain pointers and sizes and cannot see the tensors' shapes,
# so the wrappers check here, before anything is enqueued, that every input
# has the shape and dtype the sizes it passes imply: a mismatch would make the
# kernels read or write outside a tensor.

def _want(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _same_float(*named):
    """All tensors share one float dtype (float32 or bfloat16)."""
    (n0, t0), rest = named[0], named[1:]
    _dt(t0)
    for n, t in rest:
        if t.dtype != t0.dtype:
            raise ValueError(f"{n} must be {t0.dtype} like {n0}, got {t.dtype}")


def _int32_vec(t, n, name):
    import torch
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name} must be int32 [{n}], got {t.dtype} {list(t.shape)}")


def _prefill_dims(q, kv_latent, w_up_k, w_up_v):
    """q [B,T,H,d], kv_latent [B,T,r], w_up_k / w_up_v [r,H,d] -> (B, T, H, d, r)."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, T, H, d], got {list(q.shape)}")
    B, T, H, d = q.shape
    if kv_latent.dim() != 3:
        raise ValueError(f"kv_latent must be [B, T, r], got {list(kv_latent.shape)}")
    r = kv_latent.shape[-1]
    _want(kv_latent, (B, T, r), "kv_latent")
    _want(w_up_k, (r, H, d), "w_up_k")
    _want(w_up_v, (r, H, d), "w_up_v")
    _same_float(("q", q), ("kv_latent", kv_latent), ("w_up_k", w_up_k), ("w_up_v", w_up_v))
    return B, T, H, d, r


def _decode_dims(q, w_up_k, w_up_v, r):
    """q [B,1,H,d], w_up_k / w_up_v [r,H,d] -> (B, H, d)."""
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError(f"q must be [B, 1, H, d], got {list(q.shape)}")
    B, _, H, d = q.shape
    _want(w_up_k, (r, H, d), "w_up_k")
    _want(w_up_v, (r, H, d), "w_up_v")
    return B, H, d


def mla_down_proj(hidden, w_down, kv_latent=None, stream=None):
    """kv_latent[B,T,r] = hidden[B,T,D] @ w_down[D,r]."""
    import torch
    if hidden.dim() != 3 or w_down.dim() != 2:
        raise ValueError(f"hidden must be [B, T, D] and w_down [D, r], got {list(hidden.shape)}, "
                         f"{list(w_down.shape)}")
    B, T, D = hidden.shape
    r = w_down.shape[1]
    _want(w_down, (D, r), "w_down")
    _same_float(("hidden", hidden), ("w_down", w_down))
    _dev(hidden, w_down)
    if kv_latent is None:
        kv_latent = torch.empty((B, T, r), dtype=hidden.dtype, device=hidden.device)
    _shaped(kv_latent, (B, T, r), hidden.dtype, "kv_latent")
    _dev(kv_latent)
    _check(mla_down_proj_raw(hidden.data_ptr(), w_down.data_ptr(), kv_latent.data_ptr(), B, T, D, r,
                             _dt(hidden), _stream(stream)))
    return kv_latent


def mla_latent_attn_fwd(q, kv_latent, w_up_k, w_up_v, out=None, scale=None, workspace=None, stream=None):
    """Causal latent attention, prefill: q[B,T,H,d], kv_latent[B,T,r], w_up_k/w_up_v[r,H,d] -> out[B,T,H,d]."""
    import torch
    B, T, H, d, r = _prefill_dims(q, kv_latent, w_up_k, w_up_v)
    _dev(q, kv_latent, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_latent_attn_workspace_size(B, T, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_latent_attn_fwd_raw(q.data_ptr(), kv_latent.data_ptr(), w_up_k.data_ptr(), w_up_v.data_ptr(),
                                   out.data_ptr(), B, T, H, d, r, float(scale), dt, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def mla_latent_attn_fwd_masked(q, kv_latent, key_mask, w_up_k, w_up_v, out=None, scale=None, workspace=None,
                               stream=None):
    """Causal prefill with a key mask: key_mask[B,T] (uint8 or bool, device; nonzero = visible).
    A query row with no visible key s <= t comes out NaN."""
    import torch
    B, T, H, d, r = _prefill_dims(q, kv_latent, w_up_k, w_up_v)
    if tuple(key_mask.shape) != (B, T):
        raise ValueError(f"key_mask must be [B, T] = [{B}, {T}], got {list(key_mask.shape)}")
    if key_mask.dtype == torch.bool:
        key_mask = key_mask.view(torch.uint8)
    if key_mask.dtype != torch.uint8:
        raise TypeError("key_mask must be uint8 or bool")
    _dev(q, kv_latent, key_mask, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_latent_attn_masked_workspace_size(B, T, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_latent_attn_fwd_masked_raw(q.data_ptr(), kv_latent.data_ptr(), key_mask.data_ptr(), w_up_k.data_ptr(),
                                          w_up_v.data_ptr(), out.data_ptr(), B, T, H, d, r, float(scale), dt,
                                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
    return out


def mla_latent_attn_fwd_auto(q, kv_latent, w_up_k, w_up_v, out=None, scale=None, workspace=None, stream=None):
    """The causal prefill in the form the library picks for the shape (mla_latent_attn_auto_form)."""
    import torch
    B, T, H, d, r = _prefill_dims(q, kv_latent, w_up_k, w_up_v)
    _dev(q, kv_latent, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_latent_attn_auto_workspace_size(B, T, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_latent_attn_fwd_auto_raw(q.data_ptr(), kv_latent.data_ptr(), w_up_k.data_ptr(), w_up_v.data_ptr(),
                                        out.data_ptr(), B, T, H, d, r, float(scale), dt, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def mla_latent_attn_fwd_unabsorbed(q, kv_latent, w_up_k, w_up_v, out=None, scale=None, workspace=None,
                                   stream=None):
    """The same prefill in unabsorbed form (k, v materialised; bf16, d = 128, r in {128, 256, 512})."""
    import torch
    B, T, H, d, r = _prefill_dims(q, kv_latent, w_up_k, w_up_v)
    _dev(q, kv_latent, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_latent_attn_unabsorbed_workspace_size(B, T, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_latent_attn_fwd_unabsorbed_raw(q.data_ptr(), kv_latent.data_ptr(), w_up_k.data_ptr(),
                                              w_up_v.data_ptr(), out.data_ptr(), B, T, H, d, r, float(scale), dt,
                                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                              _stream(stream)))
    return out


def mla_decode_fwd(q, kv_latent, seq_lens, w_up_k, w_up_v, out=None, scale=None, workspace=None, stream=None):
    """Decode: q[B,1,H,d], kv_latent[B,Tmax,r], seq_lens[B] int32 (device) -> out[B,1,H,d]."""
    import torch
    if kv_latent.dim() != 3:
        raise ValueError(f"kv_latent must be [B, Tmax, r], got {list(kv_latent.shape)}")
    B, Tmax, r = kv_latent.shape
    Bq, H, d = _decode_dims(q, w_up_k, w_up_v, r)
    if Bq != B:
        raise ValueError(f"q must be [B={B}, 1, H, d] like kv_latent, got {list(q.shape)}")
    _int32_vec(seq_lens, B, "seq_lens")
    _same_float(("q", q), ("kv_latent", kv_latent), ("w_up_k", w_up_k), ("w_up_v", w_up_v))
    _dev(q, kv_latent, seq_lens, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_decode_workspace_size(B, Tmax, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_decode_fwd_raw(q.data_ptr(), kv_latent.data_ptr(), seq_lens.data_ptr(), w_up_k.data_ptr(),
                              w_up_v.data_ptr(), out.data_ptr(), B, Tmax, H, d, r, float(scale), dt,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    return out


def mla_decode_fwd_noalloc(q, kv_latent, seq_lens, w_up_k, w_up_v, out, scale=None, stream=None):
    """mla_decode_fwd on the library's fixed device scratch: no workspace and no
    allocation (the caller passes `out`, [B,1,H,d] in q's dtype)."""
    if kv_latent.dim() != 3:
        raise ValueError(f"kv_latent must be [B, Tmax, r], got {list(kv_latent.shape)}")
    B, Tmax, r = kv_latent.shape
    Bq, H, d = _decode_dims(q, w_up_k, w_up_v, r)
    if Bq != B:
        raise ValueError(f"q must be [B={B}, 1, H, d] like kv_latent, got {list(q.shape)}")
    _int32_vec(seq_lens, B, "seq_lens")
    _same_float(("q", q), ("kv_latent", kv_latent), ("w_up_k", w_up_k), ("w_up_v", w_up_v))
    _shaped(out, q.shape, q.dtype, "out")
    _dev(q, kv_latent, seq_lens, w_up_k, w_up_v, out)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(mla_decode_fwd_noalloc_raw(q.data_ptr(), kv_latent.data_ptr(), seq_lens.data_ptr(), w_up_k.data_ptr(),
                                      w_up_v.data_ptr(), out.data_ptr(), B, Tmax, H, d, r, float(scale), _dt(q),
                                      _stream(stream)))
    return out


def mla_decode_varlen_fwd(q, kv_latent, cu_seqlens, w_up_k, w_up_v, out=None, scale=None, workspace=None,
                          stream=None):
    """Decode over a packed cache: q[B,1,H,d], kv_latent[total,r], cu_seqlens[B+1] int32 (device) -> out[B,1,H,d]."""
    import torch
    if kv_latent.dim() != 2:
        raise ValueError(f"kv_latent must be [total, r], got {list(kv_latent.shape)}")
    total, r = kv_latent.shape
    B, H, d = _decode_dims(q, w_up_k, w_up_v, r)
    _int32_vec(cu_seqlens, B + 1, "cu_seqlens")
    _same_float(("q", q), ("kv_latent", kv_latent), ("w_up_k", w_up_k), ("w_up_v", w_up_v))
    _dev(q, kv_latent, cu_seqlens, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_decode_varlen_workspace_size(B, total, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(out, workspace)
    _check(mla_decode_varlen_fwd_raw(q.data_ptr(), kv_latent.data_ptr(), cu_seqlens.data_ptr(), w_up_k.data_ptr(),
                                     w_up_v.data_ptr(), out.data_ptr(), B, total, H, d, r, float(scale), dt,
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return out


def mla_kv_append(kv_cache, seq_lens, new_latent, stream=None):
    """kv_cache[B,Tmax,r] and seq_lens[B] int32 (device) updated in place with new_latent[B,r]."""
    if kv_cache.dim() != 3:
        raise ValueError(f"kv_cache must be [B, Tmax, r], got {list(kv_cache.shape)}")
    B, Tmax, r = kv_cache.shape
    _int32_vec(seq_lens, B, "seq_lens")
    _want(new_latent, (B, r), "new_latent")
    _same_float(("kv_cache", kv_cache), ("new_latent", new_latent))
    _dev(kv_cache, seq_lens, new_latent)
    _check(mla_kv_append_raw(kv_cache.data_ptr(), seq_lens.data_ptr(), new_latent.data_ptr(), B, Tmax, r,
                             _dt(kv_cache), _stream(stream)))
    return kv_cache


def mla_latent_attn_fwd_full(hidden, w_down, q, w_up_k, w_up_v, kv_latent=None, out=None, scale=None,
                             workspace=None, stream=None):
    """Full path in one call: kv_latent[B,T,r] = hidden[B,T,D] @ w_down[D,r] (written: the latent
    cache), then causal latent attention -> out[B,T,H,d].  Returns (out, kv_latent)."""
    import torch
    if q.dim() != 4 or w_down.dim() != 2:
        raise ValueError(f"q must be [B, T, H, d] and w_down [D, r], got {list(q.shape)}, {list(w_down.shape)}")
    B, T, H, d = q.shape
    D, r = w_down.shape
    _want(hidden, (B, T, D), "hidden")
    _want(w_up_k, (r, H, d), "w_up_k")
    _want(w_up_v, (r, H, d), "w_up_v")
    _same_float(("q", q), ("hidden", hidden), ("w_down", w_down), ("w_up_k", w_up_k), ("w_up_v", w_up_v))
    _dev(hidden, w_down, q, w_up_k, w_up_v)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if kv_latent is None:
        kv_latent = torch.empty((B, T, r), dtype=q.dtype, device=q.device)
    _shaped(kv_latent, (B, T, r), q.dtype, "kv_latent")
    if out is None:
        out = torch.empty_like(q)
    _shaped(out, q.shape, q.dtype, "out")
    nbytes = mla_latent_attn_full_workspace_size(B, T, D, H, d, r, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _dev(kv_latent, out, workspace)
    _check(mla_latent_attn_fwd_full_raw(hidden.data_ptr(), w_down.data_ptr(), q.data_ptr(), w_up_k.data_ptr(),
                                        w_up_v.data_ptr(), kv_latent.data_ptr(), out.data_ptr(), B, T, D, H, d, r,
                                        float(scale), dt, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, kv_latent


def full_path(hidden, w_down, q, w_up_k, w_up_v, scale=None, stream=None):
    """hidden -> kv_latent -> causal latent attention, as one mla_latent_attn_fwd_full call."""
    out, _ = mla_latent_attn_fwd_full(hidden, w_down, q, w_up_k, w_up_v, scale=scale, stream=stream)
    return out
