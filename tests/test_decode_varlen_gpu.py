"""GPU tests of the packed (variable-length) decode cache and of the device-side
cache append, against the fp64 oracle and against the padded decode path."""
import numpy as np
import pytest

import oracle
import rank_latent_causal_mla_amd as mla
import synth
from tests.helpers import compare, to_device, to_f64
from tests.test_parity_gpu import DECODE_SMALL, cfg_like, run_decode, tight

pytestmark = pytest.mark.gpu


def pack(inp, lens):
    """Packed cache [sum L, r] (the first L_b latents of each sequence, in order) and cu_seqlens."""
    lat = inp["kv_latent"]
    packed = np.concatenate([lat[b, :int(L)] for b, L in enumerate(lens)], axis=0)
    cu = np.concatenate([[0], np.cumsum(np.asarray(lens, np.int64))]).astype(np.int32)
    return packed, cu


def run_varlen(cfg, inp, lens):
    import torch
    dev = {k: to_device(v) for k, v in inp.items() if k not in ("seq_lens", "kv_latent")}
    packed, cu = pack(inp, lens)
    out = mla.mla_decode_varlen_fwd(dev["q"], to_device(packed), torch.from_numpy(cu).cuda(), dev["w_up_k"],
                                    dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,kw,lens", DECODE_SMALL, ids=[f"varlen-{n}-{i}" for i, (n, _, _) in enumerate(DECODE_SMALL)])
def test_varlen_decode_matches_oracle(name, kw, lens):
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    print(f"varlen decode parity {cfg} lens={lens}", flush=True)
    out = run_varlen(cfg, inp, lens)
    ref = oracle.decode(inp["q"], inp["kv_latent"], lens, inp["w_up_k"], inp["w_up_v"], cfg.scale)
    err = compare(to_f64(out), ref, cfg.dtype, "varlen decode")
    print(f"max abs err {err:.3e}")


@pytest.mark.parametrize("name,kw,lens", [DECODE_SMALL[0], DECODE_SMALL[1], DECODE_SMALL[4]],
                         ids=["bf16-a", "bf16-b", "fp32"])
def test_varlen_equals_padded_bitwise(name, kw, lens):
    import torch
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    assert torch.equal(run_varlen(cfg, inp, lens), run_decode(cfg, inp, lens))


def test_varlen_full_size_equals_padded():
    import torch
    cfg = synth.CONFIGS["bf16_decode"]
    inp = synth.make_inputs(cfg)
    lens = inp["seq_lens"]
    print(f"full-size varlen decode, sum L = {int(lens.sum())}", flush=True)
    a = run_varlen(cfg, inp, lens)
    b = run_decode(cfg, inp, lens)
    assert torch.isfinite(a.float()).all().item()
    assert torch.equal(a, b)


def test_varlen_out_of_contract_stays_in_bounds():
    """Empty and overlong sequences are clamped into the cache (results unspecified, no fault, finite)."""
    import torch
    cfg = cfg_like("bf16_decode", B=4, T=96, H=32)
    inp = synth.make_inputs(cfg)
    dev = {k: to_device(v) for k, v in inp.items() if k not in ("seq_lens", "kv_latent")}
    packed, _ = pack(inp, [96, 96, 96, 96])
    cu = torch.tensor([0, 40, 40, 300, 999], dtype=torch.int32, device="cuda")  # empty, past the end
    out = mla.mla_decode_varlen_fwd(dev["q"], to_device(packed[:200]), cu, dev["w_up_k"], dev["w_up_v"],
                                    scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item()


# ---------------------------------------------------------------- cache append
@pytest.mark.parametrize("dtype,r", [("bf16", 512), ("f32", 48)])
def test_kv_append_semantics(dtype, r):
    import torch
    B, Tmax = 5, 8
    cache0 = synth.normal_tensor(7, 1, (B, Tmax, r), 1.0, dtype)
    new = synth.normal_tensor(7, 2, (B, r), 1.0, dtype)
    lens0 = np.array([0, 3, 7, 8, -1], np.int32)   # 8: full, -1: invalid -> both unchanged
    cache = to_device(cache0)
    lens = torch.from_numpy(lens0.copy()).cuda()
    mla.mla_kv_append(cache, lens, to_device(new))
    torch.cuda.synchronize()
    expect = cache0.copy()
    for b, L in enumerate(lens0):
        if 0 <= L < Tmax:
            expect[b, L] = new[b]
    got = cache.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
    assert np.array_equal(got.view(expect.dtype), expect)
    assert lens.cpu().numpy().tolist() == [1, 4, 8, 8, -1]


def test_append_then_decode_matches_oracle():
    """One decode step: the new token's latent is appended, then attended with the cache."""
    import torch
    cfg = cfg_like("bf16_decode", B=3, T=130, H=32)
    inp = synth.make_inputs(cfg)
    lens0 = [129, 1, 64]
    new = synth.normal_tensor(11, 2, (cfg.B, cfg.r), 1.0, "bf16")
    dev = {k: to_device(v) for k, v in inp.items() if k != "seq_lens"}
    cache = dev["kv_latent"].clone()
    dlens = torch.tensor(lens0, dtype=torch.int32, device="cuda")
    mla.mla_kv_append(cache, dlens, to_device(new))
    out = mla.mla_decode_fwd(dev["q"], cache, dlens, dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    lat = inp["kv_latent"].copy()
    for b, L in enumerate(lens0):
        lat[b, L] = new[b]
    lens1 = [L + 1 for L in lens0]
    assert dlens.cpu().numpy().tolist() == lens1
    ref = oracle.decode(inp["q"], lat, lens1, inp["w_up_k"], inp["w_up_v"], cfg.scale)
    compare(to_f64(out), ref, "bf16", "append then decode")
    tight(to_f64(out), ref)
