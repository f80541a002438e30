"""Seeded synthetic inputs for the latent causal attention workloads.

This module is input plumbing only: it draws the random tensors that both the
CPU oracle and the HIP library consume, and holds none of the attention
arithmetic.  Every tensor comes from a counter-based stream, so any slice of
any tensor can be regenerated on its own (the oracle side uses that to build
only the rows it checks at full size).

Generator (published definitions, written out here):
  * SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014): value i of a stream with
    key K is mix(K + (i + 1) * 0x9E3779B97F4A7C15), where
    mix(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
             z *= 0x94D049BB133111EB; z ^= z >> 31   (all mod 2^64).
  * The key of tensor `tid` under `seed` is mix(seed * 0x9E3779B97F4A7C15 + tid).
  * Uniform on (0, 1): ((x >> 11) + 0.5) * 2^-53.
  * Normal: Box-Muller (Box & Muller 1958) on the pair (u[2p], u[2p+1]):
    element 2p = R cos(2 pi u2), element 2p+1 = R sin(2 pi u2),
    R = sqrt(-2 ln u1).  Then scaled by the requested standard deviation,
    rounded to float32 (and, for bf16 tensors, to bf16 by round-to-nearest-even).
  * Integer uniform on [lo, hi]: lo + floor(u * (hi - lo + 1)).

The streams are computed by gen.c (built into libsynth.so); a slow NumPy
statement of the same definition is kept for the tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import (CONFIGS, TENSOR_IDS, WORKLOADS, Config, make_inputs, make_key_mask, make_rows,  # noqa: F401
                      seq_lens)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so (gcc, -O2, pthreads)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp,
                               os.path.join(_HERE, "gen.c"), "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64]
        for fn in (lib.synth_normal_f32, lib.synth_normal_bf16):
            fn.restype = None
            fn.argtypes = [u64, u64, u64, u64, dbl, vp, i32]
        lib.synth_uniform.restype = None
        lib.synth_uniform.argtypes = [u64, u64, u64, u64, vp, i32]
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def stream_key(seed: int, tid: int) -> int:
    return int(_load().synth_stream_key(seed & (2**64 - 1), tid))


def uniform(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    if count:
        _load().synth_uniform(seed & (2**64 - 1), tid, start, count, out.ctypes.data, _threads())
    return out


def normal_tensor(seed: int, tid: int, shape, std: float, dtype: str, start: int = 0) -> np.ndarray:
    """A stored tensor: float32 array for dtype 'f32', uint16 bf16 bits for 'bf16'.

    Values are elements start .. start+prod(shape)-1 of the stream, scaled by
    std, rounded to float32 and (for bf16) then to bf16, nearest-even.  A row
    range of a larger tensor is therefore reproduced exactly by passing its
    flat offset.
    """
    n = int(np.prod(shape))
    lib = _load()
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        fn = lib.synth_normal_f32
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        fn = lib.synth_normal_bf16
    else:
        raise ValueError(f"unknown dtype {dtype}")
    if n:
        fn(seed & (2**64 - 1), tid, start, n, float(std), out.ctypes.data, _threads())
    return out.reshape(shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def randint(seed: int, tid: int, count: int, lo: int, hi: int) -> np.ndarray:
    """count integers uniform on [lo, hi] (both ends included), int32."""
    u = uniform(seed, tid, 0, count)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int32)


# ---- slow NumPy statement of the same generator, used by the tests to check the C code
_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def _mix_np(z):
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(0xBF58476D1CE4E5B9)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def reference_normal(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        key = _mix_np(np.array([seed], dtype=np.uint64) * _GAMMA + np.uint64(tid))[0]
        idx = np.arange(start, start + count, dtype=np.uint64)
        p = idx >> np.uint64(1)

        def u(i):
            return ((_mix_np(key + (i + np.uint64(1)) * _GAMMA) >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
        u1, u2 = u(np.uint64(2) * p), u(np.uint64(2) * p + np.uint64(1))
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    return np.where(idx & np.uint64(1), rad * np.sin(ang), rad * np.cos(ang))
