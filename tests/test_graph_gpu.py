"""The calls can be captured into a HIP graph: they allocate nothing, never
synchronise and record no memset, so a serving loop may capture them once and
replay them.  Prefill (absorbed and unabsorbed), key-masked prefill and decode are captured once, then
replayed several times with new values written into the captured input
buffers and eager work plus synchronisation between the replays; every replay
equals the eager call on the same inputs bit for bit."""
import dataclasses

import numpy as np
import pytest

import rank_latent_causal_mla_amd as mla
import synth
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


def _setup(what):
    import torch
    cfg = dataclasses.replace(synth.CONFIGS["bf16_prefill"], B=2, T=300, H=8)
    inp = synth.make_inputs(cfg)
    dev = {k: to_device(v) for k, v in inp.items()}
    wk, wv = dev["w_up_k"], dev["w_up_v"]
    if what == "decode":
        q = dev["q"][:, -1:].contiguous()
        lens = torch.tensor([300, 123], dtype=torch.int32, device="cuda")
        return q, lambda: mla.mla_decode_fwd(q, dev["kv_latent"], lens, wk, wv, scale=cfg.scale)
    q = dev["q"]
    if what == "masked":
        mask = torch.from_numpy(synth.make_key_mask(cfg, p_hole=0.2, lead=3)).cuda()
        return q, lambda: mla.mla_latent_attn_fwd_masked(q, dev["kv_latent"], mask, wk, wv, scale=cfg.scale)
    if what == "unabsorbed":
        return q, lambda: mla.mla_latent_attn_fwd_unabsorbed(q, dev["kv_latent"], wk, wv, scale=cfg.scale)
    return q, lambda: mla.mla_latent_attn_fwd(q, dev["kv_latent"], wk, wv, scale=cfg.scale)


@pytest.mark.parametrize("what", ["prefill", "unabsorbed", "masked", "decode"])
def test_graph_replays_equal_eager(what):
    import torch
    q, fn = _setup(what)
    q0 = q.clone()
    print(f"graph capture of {what}", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # first call outside the capture (kernel attributes)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    x = torch.randn(1024, 1024, device="cuda")
    for i in range(4):
        q.copy_(q0 * (1.0 + 0.25 * i))             # new values in the captured buffer
        ref = fn()                                   # eager, on the same inputs
        x = torch.tanh(torch.mm(x, x))               # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        assert np.isfinite(ref.float().cpu().numpy()).all() or what == "masked"
