"""The seeded input generator: C streams match their NumPy statement, slices
are consistent, and the configs draw what they state."""
import numpy as np

import synth


def test_c_matches_numpy_statement():
    for seed, tid, start, n in [(1, 1, 0, 1000), (0x4D4C41, 2, 12345, 777), (7, 3, 1, 64)]:
        c = synth.normal_tensor(seed, tid, (n,), 1.0, "f32", start=start)
        ref = synth.reference_normal(seed, tid, start, n).astype(np.float32)
        assert np.array_equal(c, ref)


def test_slices_are_consistent():
    full = synth.normal_tensor(3, 1, (100, 37), 0.5, "bf16")
    part = synth.normal_tensor(3, 1, (10, 37), 0.5, "bf16", start=41 * 37)
    assert np.array_equal(full[41:51], part)


def test_thread_split_independent():
    big = synth.normal_tensor(9, 4, (300000,), 1.0, "f32")
    assert np.array_equal(big[:70000], synth.normal_tensor(9, 4, (70000,), 1.0, "f32"))


def test_bf16_rounding_nearest_even():
    x = synth.normal_tensor(5, 5, (4096,), 1.0, "f32")
    b = synth.normal_tensor(5, 5, (4096,), 1.0, "bf16")
    w = synth.bf16_bits_to_f32(b).astype(np.float64)
    err = np.abs(w - x.astype(np.float64))
    # round-to-nearest: error at most half a bf16 ulp (2^-8 relative)
    assert (err <= np.abs(x) * 2.0 ** -8 + 1e-30).all()


def test_distribution_moments():
    x = synth.normal_tensor(11, 1, (1 << 20,), 0.25, "f32").astype(np.float64)
    assert abs(x.mean()) < 3 * 0.25 / 1024
    assert abs(x.std() - 0.25) < 0.25 * 0.005


def test_decode_lengths():
    cfg = synth.CONFIGS["bf16_decode"]
    lens = synth.seq_lens(cfg)
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 8192
    u = synth.randint(1, 7, 200000, 1, 4)
    assert set(np.unique(u)) == {1, 2, 3, 4}


def test_make_rows_matches_make_inputs():
    cfg = synth.CONFIGS["page_attn_size"]
    full = synth.make_inputs(cfg)
    assert np.array_equal(synth.make_rows(cfg, "q", 1, 5, 3), full["q"][1, 5:8].reshape(3, -1))
    assert np.array_equal(synth.make_rows(cfg, "kv_latent", 0, 2, 4), full["kv_latent"][0, 2:6])


def test_key_mask_recipe():
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["bf16_prefill"], B=4, T=200)
    m = synth.make_key_mask(cfg, p_hole=0.1, lead=7)
    assert m.shape == (4, 200) and m.dtype == np.uint8 and set(np.unique(m)) <= {0, 1}
    assert np.array_equal(m, synth.make_key_mask(cfg, p_hole=0.1, lead=7))      # seeded
    assert not m[1::2, :7].any()                                                   # leading keys of odd batches
    for b in range(4):   # padding: nothing visible past the last visible key's run, valid length >= T/2
        vis = np.nonzero(m[b])[0]
        assert vis.size and vis.max() < 200
    nopad = synth.make_key_mask(cfg, p_hole=0.0, pad=False)
    assert nopad.all()
