"""GPU parity of the full path in one call (mla_latent_attn_fwd_full): the
KV down-projection writes the latent cache, then the causal prefill runs
over it.  Both outputs are checked against the fp64 oracle, which keeps its
own latent in fp64 (the GPU stores it in the call's dtype):
|gpu - oracle| <= atol + rtol |oracle|, 1e-4 for float32, 2e-2 for bf16."""
import dataclasses

import numpy as np
import pytest

import oracle
import rank_latent_causal_mla_amd as mla
import synth
from tests.helpers import compare, to_device, to_f64

pytestmark = pytest.mark.gpu


def cfg_like(name, **kw):
    return dataclasses.replace(synth.CONFIGS[name], **kw)


def run_full(cfg, inp):
    import torch
    dev = {k: to_device(v) for k, v in inp.items()}
    out, lat = mla.mla_latent_attn_fwd_full(dev["hidden"], dev["w_down"], dev["q"], dev["w_up_k"], dev["w_up_v"],
                                            scale=cfg.scale)
    torch.cuda.synchronize()
    return out, lat, dev


def rel_rms(got, ref):
    return float(np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2)))


CASES = [
    ("fp32_full_path", {}),                                                    # the full-path workload
    ("page_kv_size_h8", {}),                                                   # the KV page's shapes, r = 48
    ("page_kv_size_h1", {}),
    ("bf16_prefill", dict(B=2, T=100, H=16, D=1024)),                          # matrix-core down-projection
    ("bf16_prefill", dict(B=1, T=300, H=2, d=64, r=128, D=256)),               # ragged 128-token blocks
    ("bf16_prefill", dict(B=2, T=70, H=4, r=256, D=192)),
    ("bf16_prefill", dict(B=2, T=50, H=4, r=128, D=96)),                       # D % 64 != 0: vector path
    ("bf16_prefill", dict(B=3, T=1, H=2, d=32, r=128, D=64)),                  # 3 tokens: one ragged block
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_full_path_matches_oracle(name, kw):
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    print(f"full path parity {cfg}", flush=True)
    out, lat, _ = run_full(cfg, inp)
    lat_ref = oracle.down_proj(inp["hidden"], inp["w_down"])
    lerr = compare(to_f64(lat), lat_ref, cfg.dtype, f"{cfg.name} latent")
    ref = oracle.full_path(inp["hidden"], inp["w_down"], inp["q"], inp["w_up_k"], inp["w_up_v"], cfg.scale)
    got = to_f64(out)
    err = compare(got, ref, cfg.dtype, f"{cfg.name} output")
    print(f"latent max abs err {lerr:.3e}, output max abs err {err:.3e}, rel rms {rel_rms(got, ref):.3e}")
    if cfg.dtype == "bf16":
        assert rel_rms(to_f64(lat), lat_ref) < 3e-3     # one bf16 rounding of the latent
        assert rel_rms(got, ref) < 5e-3


@pytest.mark.parametrize("name,kw", [("fp32_full_path", {}), ("bf16_prefill", dict(B=2, T=50, H=4, r=128, D=96))])
def test_vector_path_equals_two_calls_bitwise(name, kw):
    """Where the down-projection takes the vector path, one call equals
    mla_down_proj followed by mla_latent_attn_fwd bit for bit."""
    import torch
    cfg = cfg_like(name, **kw)
    out, lat, dev = run_full(cfg, synth.make_inputs(cfg))
    lat2 = mla.mla_down_proj(dev["hidden"], dev["w_down"])
    out2 = mla.mla_latent_attn_fwd(dev["q"], lat2, dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(lat.view(torch.int16) if lat.dtype == torch.bfloat16 else lat,
                       lat2.view(torch.int16) if lat2.dtype == torch.bfloat16 else lat2)
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2)


def test_bf16_full_path_full_size_sampled():
    """bf16_prefill's shape with a D = 1024 down-projection at full size: the
    latent cache on sampled rows and the output on sampled query rows, each
    against the oracle (which computes its own fp64 latent from hidden)."""
    import torch
    cfg = cfg_like("bf16_prefill", D=1024)
    inp = synth.make_inputs(cfg)
    print(f"full-size full path {cfg}", flush=True)
    out, lat, _ = run_full(cfg, inp)
    lat_ref = oracle.down_proj(inp["hidden"], inp["w_down"])          # [B, T, r] fp64, every row
    compare(to_f64(lat), lat_ref, "bf16", "latent")
    assert rel_rms(to_f64(lat), lat_ref) < 3e-3
    rng = np.random.default_rng(11)
    T = cfg.T
    rb, rh, rt = [], [], []
    for (b, h) in [(0, 0), (5, 9), (7, 15)]:
        for t in sorted(set([0, 1, 31, 32, 127, 128, T // 2, T - 1] + list(rng.integers(0, T, 16)))):
            rb.append(b); rh.append(h); rt.append(t)
    rb, rh, rt = map(np.array, (rb, rh, rt))
    ref = oracle.attend_rows(inp["q"][rb, rt, rh], rb, rh, rt + 1, lat_ref, inp["w_up_k"], inp["w_up_v"], cfg.scale)
    got = to_f64(out[torch.from_numpy(rb).cuda(), torch.from_numpy(rt).cuda(), torch.from_numpy(rh).cuda()])
    err = compare(got, ref, "bf16", "output")
    print(f"{len(rb)} sampled rows, max abs err {err:.3e}, rel rms {rel_rms(got, ref):.3e}")
    assert rel_rms(got, ref) < 5e-3
