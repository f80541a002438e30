"""mla_decode_fwd_noalloc, the decode entry point that allocates nothing (its
scratch is the library's fixed device array), against mla_decode_fwd: two
calls in a row through the C ABI, the second with a smaller input, each equal
bit for bit to mla_decode_fwd on the same inputs (same kernels, same chunk
count), and the smaller one also within the bf16 bar of the oracle.  The
scratch is never cleared, so the second call runs over the first one's
leftovers."""
import dataclasses

import numpy as np
import pytest

import oracle
import rank_latent_causal_mla_amd as mla
import synth
from tests.helpers import compare, to_device, to_f64

pytestmark = pytest.mark.gpu


def decode_both(cfg, lens):
    import torch
    inp = synth.make_inputs(cfg)
    dev = {k: to_device(v) for k, v in inp.items() if k != "seq_lens"}
    dlens = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    ref = mla.mla_decode_fwd(dev["q"], dev["kv_latent"], dlens, dev["w_up_k"], dev["w_up_v"], scale=cfg.scale)
    out = torch.full_like(dev["q"], float("nan"))
    B, Tmax, r = dev["kv_latent"].shape
    H, d = cfg.H, cfg.d
    status = mla.mla_decode_fwd_noalloc_raw(dev["q"].data_ptr(), dev["kv_latent"].data_ptr(), dlens.data_ptr(),
                                            dev["w_up_k"].data_ptr(), dev["w_up_v"].data_ptr(), out.data_ptr(), B,
                                            Tmax, H, d, r, cfg.scale, mla.MLA_DTYPE_BF16,
                                            torch.cuda.current_stream().cuda_stream)
    assert status == mla.MLA_OK, mla.last_error()
    torch.cuda.synchronize()
    return inp, out, ref


def test_noalloc_decode_equals_decode_on_two_calls():
    import torch
    # 1: the bf16_decode workload (64 ragged sequences of 1024..8192 latents, 32 heads)
    cfg = synth.CONFIGS["bf16_decode"]
    lens = synth.make_inputs(cfg)["seq_lens"]
    print(f"no-alloc decode, call 1: {cfg}", flush=True)
    _, out, ref = decode_both(cfg, lens)
    assert torch.equal(out, ref), "call 1 differs from mla_decode_fwd"
    # 2: a smaller input over the scratch the first call left behind
    cfg2 = dataclasses.replace(synth.CONFIGS["bf16_decode"], B=5, T=700)
    lens2 = np.array([700, 1, 333, 64, 699], np.int32)
    print(f"no-alloc decode, call 2: {cfg2}", flush=True)
    inp2, out2, ref2 = decode_both(cfg2, lens2)
    assert torch.equal(out2, ref2), "call 2 differs from mla_decode_fwd"
    want = oracle.decode(inp2["q"], inp2["kv_latent"], lens2, inp2["w_up_k"], inp2["w_up_v"], cfg2.scale)
    compare(to_f64(out2), want, "bf16", "no-alloc decode")


def test_noalloc_decode_rejects_a_shape_beyond_the_scratch():
    import torch
    q = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda")
    # 4096 sequences x 128 heads at r = 512: the absorbed queries alone take 512 MiB
    status = mla.mla_decode_fwd_noalloc_raw(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                            q.data_ptr(), 4096, 8, 128, 128, 512, 0.1, mla.MLA_DTYPE_BF16, 0)
    assert status == mla.MLA_ERR_UNSUPPORTED
    assert "scratch" in mla.last_error()
