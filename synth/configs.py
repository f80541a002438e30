"""The workloads, as seeded synthetic input recipes.

Each config states shapes, storage dtype and the distribution of every input
tensor; `make_inputs` draws them from the counter-based streams defined in
`synth/__init__.py`.  Shapes follow the latent causal attention definition:
q[B,T,H,d], kv_latent[B,T,r], w_up_k / w_up_v[r,H,d], optional hidden[B,T,D]
with w_down[D,r]; decode adds seq_lens[B] and a padded cache [B,Tmax,r].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# stream ids: one independent stream per tensor role
TENSOR_IDS = {"q": 1, "kv_latent": 2, "w_up_k": 3, "w_up_v": 4, "hidden": 5, "w_down": 6, "seq_lens": 7,
              "key_mask": 8, "key_valid_len": 9}
SEED_BASE = 0x4D4C41


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str               # "f32" or "bf16": storage dtype of every float tensor
    B: int
    T: int                   # prefill length, or the padded cache length Tmax for decode
    H: int
    d: int
    r: int
    D: int = 0               # model dim of the optional down-projection (0: none)
    decode: bool = False
    len_lo: int = 0          # decode: cache lengths uniform on [len_lo, len_hi]
    len_hi: int = 0
    seed: int = SEED_BASE

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(d), held as a float32 value by both sides
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def w_std(self) -> float:
        return 1.0 / math.sqrt(self.r)

    @property
    def w_down_std(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.D else 0.0


def _cfg(idx, **kw):
    return Config(seed=SEED_BASE + idx, **kw)


CONFIGS = {
    # the five workloads
    "fp32_small": _cfg(0, name="fp32_small", dtype="f32", B=2, T=64, H=4, d=32, r=32),
    "fp32_full_path": _cfg(1, name="fp32_full_path", dtype="f32", B=4, T=512, H=8, d=64, r=128, D=1024),
    "bf16_prefill": _cfg(2, name="bf16_prefill", dtype="bf16", B=8, T=2048, H=16, d=128, r=512),
    "bf16_decode": _cfg(3, name="bf16_decode", dtype="bf16", B=64, T=8192, H=32, d=128, r=512,
                        decode=True, len_lo=1024, len_hi=8192),
    "bf16_long_prefill": _cfg(4, name="bf16_long_prefill", dtype="bf16", B=2, T=16384, H=64, d=128, r=512),
    # the pages' own problem sizes (latent attention page: B=2,T=32,H=4,d=16,r=24;
    # KV-compression page: hidden (4,96,256), w_down (256,48), H*d = 128)
    "page_attn_size": _cfg(5, name="page_attn_size", dtype="f32", B=2, T=32, H=4, d=16, r=24),
    "page_kv_size_h8": _cfg(6, name="page_kv_size_h8", dtype="f32", B=4, T=96, H=8, d=16, r=48, D=256),
    "page_kv_size_h1": _cfg(7, name="page_kv_size_h1", dtype="f32", B=4, T=96, H=1, d=128, r=48, D=256),
}

WORKLOADS = ["fp32_small", "fp32_full_path", "bf16_prefill", "bf16_decode", "bf16_long_prefill"]


def seq_lens(cfg: Config) -> np.ndarray:
    from . import randint
    return randint(cfg.seed, TENSOR_IDS["seq_lens"], cfg.B, cfg.len_lo, cfg.len_hi)


def make_inputs(cfg: Config, with_q: bool = True) -> dict:
    """All inputs of a config as stored arrays (float32, or uint16 bf16 bits)."""
    from . import normal_tensor
    dt, s = cfg.dtype, cfg.seed
    out = {}
    qT = 1 if cfg.decode else cfg.T
    if with_q:
        out["q"] = normal_tensor(s, TENSOR_IDS["q"], (cfg.B, qT, cfg.H, cfg.d), 1.0, dt)
    out["w_up_k"] = normal_tensor(s, TENSOR_IDS["w_up_k"], (cfg.r, cfg.H, cfg.d), cfg.w_std, dt)
    out["w_up_v"] = normal_tensor(s, TENSOR_IDS["w_up_v"], (cfg.r, cfg.H, cfg.d), cfg.w_std, dt)
    if cfg.D:
        out["hidden"] = normal_tensor(s, TENSOR_IDS["hidden"], (cfg.B, cfg.T, cfg.D), 1.0, dt)
        out["w_down"] = normal_tensor(s, TENSOR_IDS["w_down"], (cfg.D, cfg.r), cfg.w_down_std, dt)
    else:
        out["kv_latent"] = normal_tensor(s, TENSOR_IDS["kv_latent"], (cfg.B, cfg.T, cfg.r), 1.0, dt)
    if cfg.decode:
        out["seq_lens"] = seq_lens(cfg)
    return out


def make_rows(cfg: Config, name: str, b: int, t0: int, nrows: int) -> np.ndarray:
    """Rows [b, t0:t0+nrows] of a [B, T, ...] input, drawn without the rest of it."""
    from . import normal_tensor
    qT = 1 if cfg.decode else cfg.T
    if name == "q":
        row, T, std = cfg.H * cfg.d, qT, 1.0
    elif name == "kv_latent":
        row, T, std = cfg.r, cfg.T, 1.0
    elif name == "hidden":
        row, T, std = cfg.D, cfg.T, 1.0
    else:
        raise ValueError(name)
    start = (b * T + t0) * row
    return normal_tensor(cfg.seed, TENSOR_IDS[name], (nrows, row), std, cfg.dtype, start=start)


def make_key_mask(cfg: Config, p_hole: float = 0.1, pad: bool = True, lead: int = 0) -> np.ndarray:
    """A key mask [B, T] uint8 (1 = visible) in the shape of padded batches:
    with `pad`, batch b keeps keys below a valid length uniform on [T/2, T]
    (both ends included) and masks the rest; every key is also masked with
    probability p_hole (independent uniforms); the first `lead` keys of odd
    batches are masked, so their first rows see no key at all."""
    from . import randint, uniform
    B, T = cfg.B, cfg.T
    u = uniform(cfg.seed, TENSOR_IDS["key_mask"], 0, B * T).reshape(B, T)
    mask = (u >= p_hole).astype(np.uint8)
    if pad:
        valid = randint(cfg.seed, TENSOR_IDS["key_valid_len"], B, (T + 1) // 2, T)
        mask[np.arange(T)[None, :] >= valid[:, None]] = 0
    mask[1::2, :lead] = 0
    return mask
