"""ORACLE -- test infrastructure only.

A plain fp64 CPU statement of latent causal multi-head attention (k and v
materialised per head, two-pass max-subtracted softmax) and of the KV
down-projection, in `mla_oracle.cpp`.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product library
never does, and this package imports nothing from it.

Arrays are passed as stored: float32, bf16 bit patterns (uint16) or float64;
the C code widens every element exactly to double.  Results are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmla_oracle.so")
_SRC = os.path.join(_HERE, "mla_oracle.cpp")
_lib = None

_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def build(force: bool = True, src: str = _SRC, out: str = _SO) -> str:
    """Compile the oracle (g++ -O2, no fast-math: sums keep their written order)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, src])
        os.replace(tmp, out)
    return out


def _bind(lib):
    vp, L, i32, dbl = ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_double
    lib.oracle_threads.restype = i32
    lib.oracle_threads.argtypes = [i32]
    lib.oracle_down_proj.restype = i32
    lib.oracle_down_proj.argtypes = [vp, i32, vp, i32, L, L, L, vp]
    lib.oracle_attend_rows.restype = i32
    lib.oracle_attend_rows.argtypes = [vp, i32, L, vp, vp, vp, vp, i32, L, L, vp, vp, i32,
                                       L, L, L, dbl, vp, vp, L, i32]
    lib.oracle_attend_rows_masked.restype = i32
    lib.oracle_attend_rows_masked.argtypes = [vp, i32, L, vp, vp, vp, vp, i32, L, L, vp, vp, i32,
                                              L, L, L, dbl, vp, vp, vp, L, i32]
    lib.oracle_latent_attn_masked.restype = i32
    lib.oracle_latent_attn_masked.argtypes = [vp, i32, vp, i32, vp, vp, i32, L, L, L, L, L, dbl, vp, vp, i32]
    lib.oracle_latent_attn.restype = i32
    lib.oracle_latent_attn.argtypes = [vp, i32, vp, i32, vp, vp, i32, L, L, L, L, L, dbl, vp, i32]
    lib.oracle_decode.restype = i32
    lib.oracle_decode.argtypes = [vp, i32, vp, i32, vp, vp, vp, i32, L, L, L, L, L, dbl, vp, i32]
    return lib


def load(path: str | None = None):
    """The oracle library (built on first use if absent); `path` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_SO))
    return _lib


def _arr(x):
    x = np.ascontiguousarray(x)
    if x.dtype not in _DT:
        raise TypeError(f"oracle takes float32, bf16 bits (uint16) or float64, got {x.dtype}")
    return x, _DT[x.dtype]


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def threads(nthreads: int = 0, lib=None) -> int:
    return int((lib or load()).oracle_threads(nthreads))


def down_proj(hidden, w_down, lib=None):
    """latent = hidden @ w_down; hidden [..., D], w_down [D, r] -> float64 [..., r]."""
    lib = lib or load()
    h, dh = _arr(hidden)
    w, dw = _arr(w_down)
    D, r = w.shape
    M = h.size // D
    out = np.empty(h.shape[:-1] + (r,), dtype=np.float64)
    _check(lib.oracle_down_proj(h.ctypes.data, dh, w.ctypes.data, dw, M, D, r, out.ctypes.data), "down_proj")
    return out


def _mask(key_mask, shape):
    if key_mask is None:
        return None
    m = np.ascontiguousarray(key_mask, dtype=np.uint8)
    assert m.shape == shape, (m.shape, shape)
    return m


def latent_attn(q, kv_latent, w_up_k, w_up_v, scale, key_mask=None, nthreads=0, lib=None):
    """Causal prefill: q [B,T,H,d], kv_latent [B,T,r], w [r,H,d] -> float64 [B,T,H,d].
    key_mask [B,T] (optional, 0 = masked): masked keys get logit -inf; a row
    with no unmasked key is NaN."""
    lib = lib or load()
    q, dq = _arr(q)
    lat, dl = _arr(kv_latent)
    wk, dw = _arr(w_up_k)
    wv, dw2 = _arr(w_up_v)
    assert dw == dw2
    B, T, H, d = q.shape
    r = lat.shape[-1]
    assert lat.shape == (B, T, r) and wk.shape == (r, H, d) and wv.shape == (r, H, d)
    out = np.empty((B, T, H, d), dtype=np.float64)
    m = _mask(key_mask, (B, T))
    if m is None:
        _check(lib.oracle_latent_attn(q.ctypes.data, dq, lat.ctypes.data, dl, wk.ctypes.data, wv.ctypes.data, dw,
                                      B, T, H, d, r, float(scale), out.ctypes.data, nthreads), "latent_attn")
    else:
        _check(lib.oracle_latent_attn_masked(q.ctypes.data, dq, lat.ctypes.data, dl, wk.ctypes.data,
                                             wv.ctypes.data, dw, B, T, H, d, r, float(scale), m.ctypes.data,
                                             out.ctypes.data, nthreads), "latent_attn_masked")
    return out


def attend_rows(q_rows, row_b, row_h, row_nkeys, kv_latent, w_up_k, w_up_v, scale,
                want_probs=False, key_mask=None, nthreads=0, lib=None):
    """Rows i of q_rows [n, d] (batch row_b[i], head row_h[i]) attending key
    positions 0 .. row_nkeys[i]-1 of kv_latent [B, Tlat, r].  Returns float64
    out [n, d] (and probs [n, max nkeys], zero beyond each row's keys)."""
    lib = lib or load()
    q, dq = _arr(q_rows)
    lat, dl = _arr(kv_latent)
    wk, dw = _arr(w_up_k)
    wv, _ = _arr(w_up_v)
    n, d = q.shape
    B, Tlat, r = lat.shape
    H = wk.shape[1]
    rb = np.ascontiguousarray(row_b, dtype=np.int64)
    rh = np.ascontiguousarray(row_h, dtype=np.int64)
    rk = np.ascontiguousarray(row_nkeys, dtype=np.int64)
    out = np.empty((n, d), dtype=np.float64)
    pstride = int(rk.max()) if (want_probs and n) else 0
    probs = np.zeros((n, max(pstride, 1)), dtype=np.float64) if want_probs else None
    m = _mask(key_mask, (B, Tlat))
    _check(lib.oracle_attend_rows_masked(q.ctypes.data, dq, n, rb.ctypes.data, rh.ctypes.data, rk.ctypes.data,
                                         lat.ctypes.data, dl, B, Tlat, wk.ctypes.data, wv.ctypes.data, dw,
                                         H, d, r, float(scale), None if m is None else m.ctypes.data,
                                         out.ctypes.data, probs.ctypes.data if want_probs else None, pstride,
                                         nthreads), "attend_rows")
    return (out, probs) if want_probs else out


def decode(q, kv_latent, seq_lens, w_up_k, w_up_v, scale, nthreads=0, lib=None):
    """Decode: q [B,1,H,d] or [B,H,d], kv_latent [B,Tmax,r], seq_lens [B] -> float64 [B,1,H,d]."""
    lib = lib or load()
    q, dq = _arr(q)
    lat, dl = _arr(kv_latent)
    wk, dw = _arr(w_up_k)
    wv, _ = _arr(w_up_v)
    B, Tmax, r = lat.shape
    H, d = wk.shape[1], wk.shape[2]
    assert q.size == B * H * d
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((B, 1, H, d), dtype=np.float64)
    _check(lib.oracle_decode(q.ctypes.data, dq, lat.ctypes.data, dl, sl.ctypes.data, wk.ctypes.data,
                             wv.ctypes.data, dw, B, Tmax, H, d, r, float(scale), out.ctypes.data, nthreads),
           "decode")
    return out


def full_path(hidden, w_down, q, w_up_k, w_up_v, scale, nthreads=0, lib=None):
    """latent = hidden @ w_down (kept in float64), then causal prefill on it."""
    lat = down_proj(hidden, w_down, lib=lib)
    return latent_attn(q, lat, w_up_k, w_up_v, scale, nthreads=nthreads, lib=lib)
