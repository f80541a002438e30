"""Pins of the CPU oracle to facts outside itself.

Each pin takes the oracle library handle (so the same pins can be run against
deliberately broken builds of the oracle) and raises AssertionError when the
oracle disagrees with what the definition of latent causal attention and
plain mathematics fix:

  * brute force on tiny inputs, written directly from the definition;
  * a library routine (torch's scaled_dot_product_attention, fp64, CPU) on
    k and v up-projected by a library matmul;
  * the textbook special case H = 1, r = d, W = I (plain causal attention
    with K = V = latent);
  * the weight-absorbed form (q_lat = W_uk q, o_lat = sum p latent,
    out = o_lat W_uv), which equals the definition by bilinearity;
  * invariants: row t = 0 equals v_0; softmax rows sum to 1; rows <= t are
    unchanged when latents at s > t change; closed forms for W_uk = 0
    (causal prefix mean of v) and for equal latents (c W_uv);
  * max subtraction: huge logits give the v of the arg-max key;
  * decode(L) equals prefill row L-1, and never reads cache rows >= L;
  * down-projection equals a library fp64 matmul;
  * bf16 inputs are read exactly (same result as the widened float32 values);
  * key mask: brute force over the unmasked keys s <= t, NaN for rows with
    none (the -inf fill then softmax of the MSA page), and the closed form
    that a row whose only visible key is s outputs v_s;
  * an all-ones mask changes nothing.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def _rand(rng, shape, std=1.0):
    return rng.standard_normal(shape) * std


def _problem(seed, B, T, H, d, r):
    rng = np.random.default_rng(seed)
    q = _rand(rng, (B, T, H, d))
    lat = _rand(rng, (B, T, r))
    wk = _rand(rng, (r, H, d), 1 / math.sqrt(r))
    wv = _rand(rng, (r, H, d), 1 / math.sqrt(r))
    return q, lat, wk, wv, 1 / math.sqrt(d)


def _close(a, b, rtol, atol, what):
    a, b = np.asarray(a), np.asarray(b)
    bad = ~(np.abs(a - b) <= atol + rtol * np.abs(b))
    if bad.any():
        err = np.abs(a - b)
        worst = np.max(err[np.isfinite(err)]) if np.isfinite(err).any() else float("nan")
        raise AssertionError(f"{what}: {bad.sum()} mismatches, max finite abs err {worst}")


def pin_brute_force_scalar(lib):
    # B=1, T=3, H=1, d=1, r=1: everything is a scalar
    q = np.array([0.7, -1.3, 2.1]).reshape(1, 3, 1, 1)
    lat = np.array([1.5, -0.4, 0.9]).reshape(1, 3, 1)
    wk = np.array([0.8]).reshape(1, 1, 1)
    wv = np.array([-1.7]).reshape(1, 1, 1)
    scale = 0.6
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    for t in range(3):
        ls = [scale * q[0, t, 0, 0] * lat[0, s, 0] * wk[0, 0, 0] for s in range(t + 1)]
        ws = [math.exp(x) for x in ls]
        want = sum(w * lat[0, s, 0] * wv[0, 0, 0] for s, w in enumerate(ws)) / sum(ws)
        assert abs(got[0, t, 0, 0] - want) <= 1e-14 * (1 + abs(want)), (t, got[0, t, 0, 0], want)


def pin_brute_force_small(lib):
    # B=1, T=4, H=2, d=2, r=3, written as explicit loops over the definition
    q, lat, wk, wv, scale = _problem(11, 1, 4, 2, 2, 3)
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    for h in range(2):
        for t in range(4):
            logits, vs = [], []
            for s in range(t + 1):
                k = [sum(lat[0, s, j] * wk[j, h, e] for j in range(3)) for e in range(2)]
                v = [sum(lat[0, s, j] * wv[j, h, e] for j in range(3)) for e in range(2)]
                logits.append(scale * sum(q[0, t, h, e] * k[e] for e in range(2)))
                vs.append(v)
            w = [math.exp(x) for x in logits]
            want = [sum(w[s] * vs[s][e] for s in range(t + 1)) / sum(w) for e in range(2)]
            _close(got[0, t, h], want, 1e-13, 1e-14, f"brute force h={h} t={t}")


def pin_library_sdpa(lib):
    import torch
    q, lat, wk, wv, scale = _problem(12, 2, 9, 3, 5, 7)
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    L = torch.from_numpy(lat)
    K = torch.einsum("btr,rhe->bhte", L, torch.from_numpy(wk))
    V = torch.einsum("btr,rhe->bhte", L, torch.from_numpy(wv))
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    _close(got, ref.permute(0, 2, 1, 3).numpy(), 1e-12, 1e-13, "vs torch sdpa")


def pin_textbook_identity(lib):
    import torch
    rng = np.random.default_rng(13)
    B, T, d = 2, 11, 6
    q = rng.standard_normal((B, T, 1, d))
    lat = rng.standard_normal((B, T, d))
    eye = np.eye(d).reshape(d, 1, d)
    scale = 0.37
    got = oracle.latent_attn(q, lat, eye, eye, scale, lib=lib)
    L = torch.from_numpy(lat)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q).permute(0, 2, 1, 3), L, L,
                                                           is_causal=True, scale=scale)
    _close(got, ref.permute(0, 2, 1, 3).numpy(), 1e-12, 1e-13, "H=1, W=I")


def pin_absorbed_identity(lib):
    q, lat, wk, wv, scale = _problem(14, 2, 13, 3, 4, 6)
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    B, T, H, d = q.shape
    want = np.empty_like(got)
    for b in range(B):
        for h in range(H):
            q_lat = q[b, :, h, :] @ wk[:, h, :].T            # [T, r]
            S = scale * (q_lat @ lat[b].T)                   # [T, T]
            S[np.triu_indices(T, 1)] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            o_lat = P @ lat[b]                               # [T, r]
            want[b, :, h, :] = o_lat @ wv[:, h, :]
    _close(got, want, 1e-12, 1e-13, "absorbed form")


def pin_first_row_is_v0(lib):
    q, lat, wk, wv, scale = _problem(15, 3, 5, 4, 8, 6)
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    v0 = np.einsum("br,rhe->bhe", lat[:, 0, :], wv)
    _close(got[:, 0], v0, 1e-13, 1e-15, "row t=0 equals v_0")


def pin_probs_normalised(lib):
    q, lat, wk, wv, scale = _problem(16, 2, 7, 2, 3, 5)
    B, T, H, d = q.shape
    rb, rh, rk, rows = [], [], [], []
    for b in range(B):
        for t in range(T):
            for h in range(H):
                rb.append(b); rh.append(h); rk.append(t + 1); rows.append(q[b, t, h])
    out, P = oracle.attend_rows(np.array(rows), rb, rh, rk, lat, wk, wv, scale, want_probs=True, lib=lib)
    assert (P >= 0).all()
    for i, n in enumerate(rk):
        assert abs(P[i, :n].sum() - 1.0) <= 1e-14, P[i, :n].sum()
        assert (P[i, n:] == 0).all()
    # the output is the p-weighted sum of v
    v = np.einsum("bsr,rhe->bshe", lat, wv)
    for i in range(len(rb)):
        want = P[i, :rk[i]] @ v[rb[i], :rk[i], rh[i]]
        _close(out[i], want, 1e-13, 1e-15, "out = sum p v")


def pin_causality(lib):
    q, lat, wk, wv, scale = _problem(17, 2, 12, 3, 4, 5)
    base = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    for t0 in (0, 5, 10):
        lat2 = lat.copy()
        lat2[:, t0 + 1:, :] = np.random.default_rng(t0).standard_normal(lat2[:, t0 + 1:, :].shape) * 50
        pert = oracle.latent_attn(q, lat2, wk, wv, scale, lib=lib)
        assert np.array_equal(base[:, :t0 + 1], pert[:, :t0 + 1]), f"rows <= {t0} changed"
        assert not np.array_equal(base[:, t0 + 1:], pert[:, t0 + 1:]), "later rows did not change"


def pin_uniform_weights(lib):
    q, lat, wk, wv, scale = _problem(18, 2, 10, 3, 4, 5)
    got = oracle.latent_attn(q, lat, np.zeros_like(wk), wv, scale, lib=lib)
    v = np.einsum("bsr,rhe->bshe", lat, wv)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, v.shape[1] + 1)[None, :, None, None]
    _close(got, prefix_mean, 1e-13, 1e-14, "W_uk = 0 gives the causal prefix mean")


def pin_equal_latents(lib):
    q, lat, wk, wv, scale = _problem(19, 2, 9, 3, 4, 5)
    c = np.random.default_rng(1).standard_normal(5)
    lat[:] = c
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    want = np.einsum("r,rhe->he", c, wv)
    _close(got, np.broadcast_to(want, got.shape), 1e-13, 1e-14, "equal latents give c W_uv")


def pin_large_logits(lib):
    q, lat, wk, wv, _ = _problem(20, 1, 8, 2, 4, 5)
    scale = 1e4  # exp of unshifted logits overflows; the max-shifted softmax is one-hot
    got = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    assert np.isfinite(got).all()
    k = np.einsum("bsr,rhe->bshe", lat, wk)
    v = np.einsum("bsr,rhe->bshe", lat, wv)
    for h in range(2):
        for t in range(8):
            s_star = int(np.argmax(k[0, :t + 1, h] @ q[0, t, h]))
            _close(got[0, t, h], v[0, s_star, h], 1e-12, 1e-12, f"one-hot t={t}")


def pin_decode_is_last_prefill_row(lib):
    rng = np.random.default_rng(21)
    B, Tmax, H, d, r = 3, 17, 2, 4, 6
    lat = rng.standard_normal((B, Tmax, r))
    wk = rng.standard_normal((r, H, d)) / math.sqrt(r)
    wv = rng.standard_normal((r, H, d)) / math.sqrt(r)
    lens = np.array([1, 9, 17], dtype=np.int32)
    qd = rng.standard_normal((B, 1, H, d))
    lat_pad = lat.copy()
    for b in range(B):
        lat_pad[b, lens[b]:] = np.nan       # rows past the length are never read
    got = oracle.decode(qd, lat_pad, lens, wk, wv, 0.5, lib=lib)
    assert np.isfinite(got).all()
    for b in range(B):
        L = int(lens[b])
        qp = np.zeros((1, L, H, d))
        qp[0, L - 1] = qd[b, 0]
        pre = oracle.latent_attn(qp, lat[b:b + 1, :L], wk, wv, 0.5, lib=lib)
        _close(got[b, 0], pre[0, L - 1], 1e-13, 1e-15, f"decode b={b}")


def pin_down_proj(lib):
    rng = np.random.default_rng(22)
    for dt in ("f64", "f32"):
        h = rng.standard_normal((2, 7, 13))
        w = rng.standard_normal((13, 5)) / math.sqrt(13)
        if dt == "f32":
            h, w = h.astype(np.float32), w.astype(np.float32)
        got = oracle.down_proj(h, w, lib=lib)
        want = h.astype(np.float64).reshape(-1, 13) @ w.astype(np.float64)
        _close(got.reshape(-1, 5), want, 1e-13, 1e-14, "down_proj vs matmul")


def pin_bf16_inputs_exact(lib):
    q, lat, wk, wv, scale = _problem(23, 1, 6, 2, 4, 8)

    def bf16_bits(x):   # truncation toward zero is enough to make bf16-representable values
        return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)

    def widen(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32)
    qb, lb, kb, vb = (bf16_bits(x) for x in (q, lat, wk, wv))
    got = oracle.latent_attn(qb, lb, kb, vb, scale, lib=lib)
    want = oracle.latent_attn(widen(qb), widen(lb), widen(kb), widen(vb), scale, lib=lib)
    assert np.array_equal(got, want)
    want64 = oracle.latent_attn(*(widen(x).astype(np.float64) for x in (qb, lb, kb, vb)), scale, lib=lib)
    assert np.array_equal(got, want64)


def pin_mask_brute_force(lib):
    q, lat, wk, wv, scale = _problem(11, 2, 6, 2, 3, 4)
    rng = np.random.default_rng(5)
    mask = (rng.random((2, 6)) < 0.6).astype(np.uint8)
    mask[0, :] = 1
    mask[0, 2] = 0
    mask[1, :3] = 0       # rows t < 3 of batch 1 see no key
    mask[1, 4] = 1
    got = oracle.latent_attn(q, lat, wk, wv, scale, key_mask=mask, lib=lib)
    for b in range(2):
        for h in range(2):
            k = lat[b] @ wk[:, h, :]
            v = lat[b] @ wv[:, h, :]
            for t in range(6):
                keys = [s for s in range(t + 1) if mask[b, s]]
                if not keys:
                    assert np.isnan(got[b, t, h]).all(), (b, t, h)
                    continue
                lg = np.array([scale * q[b, t, h] @ k[s] for s in keys])
                w = np.exp(lg - lg.max())
                p = w / w.sum()
                ref = sum(p[i] * v[s] for i, s in enumerate(keys))
                _close(got[b, t, h], ref, 1e-12, 1e-14, f"masked brute force b={b} t={t} h={h}")


def pin_mask_single_visible_key(lib):
    # keys 0..2 masked: rows 0..2 have no key (NaN); row 3 sees only key 3, so it is v_3 exactly
    q, lat, wk, wv, scale = _problem(12, 1, 5, 3, 4, 6)
    mask = np.array([[0, 0, 0, 1, 1]], dtype=np.uint8)
    got = oracle.latent_attn(q, lat, wk, wv, scale, key_mask=mask, lib=lib)
    assert np.isnan(got[0, :3]).all()
    assert np.isfinite(got[0, 3:]).all()
    for h in range(3):
        _close(got[0, 3, h], lat[0, 3] @ wv[:, h, :], 1e-13, 1e-15, f"single visible key h={h}")


def pin_mask_all_ones_changes_nothing(lib):
    q, lat, wk, wv, scale = _problem(13, 2, 7, 2, 3, 5)
    a = oracle.latent_attn(q, lat, wk, wv, scale, lib=lib)
    b = oracle.latent_attn(q, lat, wk, wv, scale, key_mask=np.ones((2, 7), np.uint8), lib=lib)
    assert np.array_equal(a, b)


PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}
