"""GPU parity of the key-masked causal prefill (mla_latent_attn_fwd_masked)
against the fp64 oracle with the same mask: a masked key's logit is -inf
before the softmax, and a query row with no visible key is NaN on both
sides.  Bar as for the unmasked prefill: |gpu - oracle| <= atol + rtol |oracle|
(1e-4 float32, 2e-2 bf16) on every row that has a visible key, and NaN on
exactly the rows that have none."""
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


def run_masked(cfg, inp, mask):
    import torch
    dev = {k: to_device(v) for k, v in inp.items()}
    out = mla.mla_latent_attn_fwd_masked(dev["q"], dev["kv_latent"], torch.from_numpy(mask).cuda(), dev["w_up_k"],
                                         dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    return out, dev


def compare_nan(got, ref, dtype, what):
    """NaN exactly where the oracle is NaN (rows with no visible key); the rest within the bar."""
    got = np.asarray(got, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), (
        f"{what}: NaN pattern differs ({int(np.isnan(got).sum())} NaN on the GPU, {int(nan_ref.sum())} in the oracle)")
    if nan_ref.all():
        return 0.0
    return compare(got[~nan_ref], ref[~nan_ref], dtype, what)


CASES = [
    ("fp32_small", {}, dict(p_hole=0.3, lead=3)),
    ("page_attn_size", {}, dict(p_hole=0.2, lead=1)),                          # r = 24
    ("bf16_prefill", dict(B=2, T=100, H=16), dict(p_hole=0.2, lead=5)),        # ragged tail, several tiles
    ("bf16_prefill", dict(B=3, T=130, H=3), dict(p_hole=0.5, lead=40)),        # a whole tile masked
    ("bf16_prefill", dict(B=2, T=65, H=8, r=256), dict(p_hole=0.1, lead=0)),   # r = 256 kernel
    ("bf16_prefill", dict(B=2, T=70, H=2, r=128, d=64), dict(p_hole=0.3, lead=33)),
    ("bf16_prefill", dict(B=1, T=40, H=4, r=48, d=16), dict(p_hole=0.3, lead=0)),  # bf16 outside the tiles
    ("fp32_small", dict(T=129, r=512, d=128, H=2), dict(p_hole=0.2, lead=2)),
    ("bf16_prefill", dict(B=4, T=1, H=16), dict(p_hole=0.5, lead=1)),          # single key: v_0 or NaN
]


@pytest.mark.parametrize("name,kw,mkw", CASES, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(CASES)])
def test_masked_matches_oracle(name, kw, mkw):
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    mask = synth.make_key_mask(cfg, **mkw)
    print(f"masked prefill parity {cfg} {mkw}", flush=True)
    out, _ = run_masked(cfg, inp, mask)
    ref = oracle.latent_attn(inp["q"], inp["kv_latent"], inp["w_up_k"], inp["w_up_v"], cfg.scale, key_mask=mask)
    err = compare_nan(to_f64(out), ref, cfg.dtype, cfg.name)
    print(f"max abs err {err:.3e}, NaN rows {int(np.isnan(ref[..., 0]).sum())}")


@pytest.mark.parametrize("name,kw", [("bf16_prefill", dict(B=2, T=100, H=16)), ("fp32_small", {})])
def test_all_visible_mask_equals_unmasked_bitwise(name, kw):
    import torch
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    out, dev = run_masked(cfg, inp, np.ones((cfg.B, cfg.T), np.uint8))
    ref = mla.mla_latent_attn_fwd(dev["q"], dev["kv_latent"], dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)


@pytest.mark.parametrize("name,kw", [("bf16_prefill", dict(B=2, T=70, H=4)), ("fp32_small", {})])
def test_no_visible_key_is_nan(name, kw):
    import torch
    cfg = cfg_like(name, **kw)
    inp = synth.make_inputs(cfg)
    mask = np.zeros((cfg.B, cfg.T), np.uint8)
    mask[1, 50:] = 1   # batch 1: rows 50.. see keys; rows below 50 see none
    out, _ = run_masked(cfg, inp, mask)
    got = to_f64(out)
    assert np.isnan(got[0]).all()
    assert np.isnan(got[1, :50]).all()
    assert np.isfinite(got[1, 50:]).all()
    # bool masks are accepted as bytes
    dev = {k: to_device(v) for k, v in inp.items()}
    out2 = mla.mla_latent_attn_fwd_masked(dev["q"], dev["kv_latent"], torch.from_numpy(mask.astype(bool)).cuda(),
                                          dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    assert np.array_equal(np.isnan(to_f64(out2)), np.isnan(got))
    assert np.array_equal(np.nan_to_num(to_f64(out2)), np.nan_to_num(got))


def test_bf16_prefill_full_size_masked_sampled():
    """bf16_prefill at full size with a padding-plus-holes mask: sampled rows
    against the oracle, and every row below a batch's first masked key equal
    bit for bit to the unmasked call (those rows see no masked key)."""
    import torch
    cfg = synth.CONFIGS["bf16_prefill"]
    inp = synth.make_inputs(cfg)
    mask = synth.make_key_mask(cfg, p_hole=0.05, lead=0)
    mask[0, :200] = 1                     # batch 0: 200 leading rows with every key visible
    print(f"full-size masked prefill {cfg.name}", flush=True)
    out, dev = run_masked(cfg, inp, mask)
    rng = np.random.default_rng(5)
    T = cfg.T
    fixed = [0, 1, 31, 32, 33, 127, 128, 255, 256, T // 2, T - 2, T - 1]
    rb, rh, rt = [], [], []
    for (b, h) in [(0, 0), (3, 7), (6, 15)]:
        for t in sorted(set(fixed + list(rng.integers(0, T, 24)))):
            rb.append(b); rh.append(h); rt.append(t)
    rb, rh, rt = map(np.array, (rb, rh, rt))
    ref = oracle.attend_rows(inp["q"][rb, rt, rh], rb, rh, rt + 1, inp["kv_latent"], inp["w_up_k"], inp["w_up_v"],
                             cfg.scale, key_mask=mask)
    got = to_f64(out[torch.from_numpy(rb).cuda(), torch.from_numpy(rt).cuda(), torch.from_numpy(rh).cuda()])
    err = compare_nan(got, ref, cfg.dtype, cfg.name)
    print(f"{len(rb)} sampled rows, max abs err {err:.3e}")
    unmasked = mla.mla_latent_attn_fwd(dev["q"], dev["kv_latent"], dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    torch.cuda.synchronize()
    for b in range(cfg.B):
        first = int(np.argmin(mask[b])) if not mask[b].all() else T
        assert torch.equal(out[b, :first].view(torch.int16), unmasked[b, :first].view(torch.int16)), b


def test_bf16_long_prefill_masked_sampled():
    """bf16_long_prefill (the benchmarked workload) with the benchmark's mask:
    sampled rows of both batches against the oracle, including rows past a
    batch's valid length (they attend its visible keys only)."""
    import torch
    cfg = synth.CONFIGS["bf16_long_prefill"]
    inp = synth.make_inputs(cfg)
    mask = synth.make_key_mask(cfg, p_hole=0.05)
    print(f"full-size masked prefill {cfg.name}", flush=True)
    out, _ = run_masked(cfg, inp, mask)
    rng = np.random.default_rng(9)
    T = cfg.T
    rb, rh, rt = [], [], []
    for (b, h) in [(0, 0), (1, 63), (1, 17)]:
        last = int(np.nonzero(mask[b])[0].max())
        for t in sorted(set([0, 31, 32, 4095, last - 1, last, min(last + 1, T - 1), T - 1] +
                            list(rng.integers(0, T, 10)))):
            rb.append(b); rh.append(h); rt.append(t)
    rb, rh, rt = map(np.array, (rb, rh, rt))
    ref = oracle.attend_rows(inp["q"][rb, rt, rh], rb, rh, rt + 1, inp["kv_latent"], inp["w_up_k"], inp["w_up_v"],
                             cfg.scale, key_mask=mask)
    got = to_f64(out[torch.from_numpy(rb).cuda(), torch.from_numpy(rt).cuda(), torch.from_numpy(rh).cuda()])
    err = compare_nan(got, ref, cfg.dtype, cfg.name)
    rel = float(np.sqrt(np.nanmean((got - ref) ** 2) / np.nanmean(ref ** 2)))
    print(f"{len(rb)} sampled rows, max abs err {err:.3e}, rel rms {rel:.3e}")
    assert rel < 4e-3


def test_masked_beyond_int32_offsets_sampled():
    """B=4, T=16400, H=64, r=512 with a padding-plus-holes mask: q_lat and
    o_lat hold more than 2^31 elements, so the rows of batch 3 from
    t = 16336 on sit past every 32-bit element offset.  Sampled rows either
    side of that line, in the last batch and another, against the oracle."""
    import torch
    cfg = cfg_like("bf16_long_prefill", B=4, T=16400)
    assert cfg.B * cfg.T * cfg.H * cfg.r > 2 ** 31
    inp = synth.make_inputs(cfg)
    mask = synth.make_key_mask(cfg, p_hole=0.05)
    mask[3, :] = 1
    mask[3, 100:140] = 0                      # batch 3: every row past 140 sees all but 40 keys
    print(f"masked prefill past 32-bit offsets {cfg}", flush=True)
    out, _ = run_masked(cfg, inp, mask)
    first_past = 2 ** 31 // (cfg.H * cfg.r) - 3 * cfg.T
    rb, rh, rt = [], [], []
    for (b, h) in [(3, 0), (3, 63), (1, 9)]:
        for t in sorted({0, 99, 100, 139, 140, first_past - 1, first_past, first_past + 1, cfg.T - 1}):
            rb.append(b); rh.append(h); rt.append(t)
    rb, rh, rt = map(np.array, (rb, rh, rt))
    ref = oracle.attend_rows(inp["q"][rb, rt, rh], rb, rh, rt + 1, inp["kv_latent"], inp["w_up_k"], inp["w_up_v"],
                             cfg.scale, key_mask=mask)
    got = to_f64(out[torch.from_numpy(rb).cuda(), torch.from_numpy(rt).cuda(), torch.from_numpy(rh).cuda()])
    err = compare_nan(got, ref, cfg.dtype, cfg.name)
    print(f"{len(rb)} sampled rows, max abs err {err:.3e}")
