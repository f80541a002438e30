"""The C ABI on a host without a GPU: the library loads, exports what
include/mla.h declares, and rejects bad arguments before touching a device."""
import os
import re

import pytest

import rank_latent_causal_mla_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F32, BF16 = mla.MLA_DTYPE_F32, mla.MLA_DTYPE_BF16
P = 1 << 20   # a 16-byte aligned fake address: never dereferenced on these paths


def declared_symbols():
    with open(os.path.join(ROOT, "include", "mla.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:mla_status|size_t|int|const char\*)\s+(mla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_symbols() == sorted(mla.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = mla.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings():
    assert mla.status_string(mla.MLA_OK) == "ok"
    for s in range(1, 5):
        assert mla.status_string(s) not in ("", "ok", "unknown status")
    assert mla.status_string(99) == "unknown status"


def attn(**kw):
    a = dict(q=P, kv=P, wk=P, wv=P, out=P, B=2, T=64, H=4, d=32, r=32, scale=0.17, dt=F32, ws=P, wsb=1 << 40)
    a.update(kw)
    return mla.mla_latent_attn_fwd_raw(a["q"], a["kv"], a["wk"], a["wv"], a["out"], a["B"], a["T"], a["H"], a["d"],
                                       a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


def dec(**kw):
    a = dict(q=P, kv=P, lens=P, wk=P, wv=P, out=P, B=2, T=64, H=4, d=32, r=32, scale=0.17, dt=F32, ws=P,
             wsb=1 << 40)
    a.update(kw)
    return mla.mla_decode_fwd_raw(a["q"], a["kv"], a["lens"], a["wk"], a["wv"], a["out"], a["B"], a["T"], a["H"],
                                  a["d"], a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("fn", [attn, dec])
@pytest.mark.parametrize("kw,status", [
    ({"q": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"out": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"ws": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"B": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"T": -1}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"H": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"d": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"r": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"dt": 7}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"scale": float("nan")}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"q": P + 2}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"r": 2048}, mla.MLA_ERR_UNSUPPORTED),
    ({"d": 512}, mla.MLA_ERR_UNSUPPORTED),
    ({"wsb": 7}, mla.MLA_ERR_WORKSPACE),
])
def test_argument_errors(fn, kw, status):
    assert fn(**kw) == status
    assert mla.last_error() != ""


def unabs(**kw):
    a = dict(q=P, kv=P, wk=P, wv=P, out=P, B=2, T=64, H=4, d=128, r=512, scale=0.09, dt=BF16, ws=P, wsb=1 << 40)
    a.update(kw)
    return mla.mla_latent_attn_fwd_unabsorbed_raw(a["q"], a["kv"], a["wk"], a["wv"], a["out"], a["B"], a["T"],
                                                  a["H"], a["d"], a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    ({"q": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"ws": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"T": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"dt": 7}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"scale": float("inf")}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"out": P + 8}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"dt": F32}, mla.MLA_ERR_UNSUPPORTED),
    ({"d": 64}, mla.MLA_ERR_UNSUPPORTED),
    ({"r": 48}, mla.MLA_ERR_UNSUPPORTED),
    ({"r": 2048}, mla.MLA_ERR_UNSUPPORTED),
    ({"wsb": 1 << 20}, mla.MLA_ERR_WORKSPACE),
])
def test_unabsorbed_argument_errors(kw, status):
    assert unabs(**kw) == status
    assert mla.last_error() != ""


def test_unabsorbed_workspace_size():
    # k and v [B*T][H][d] plus W_uk^T and W_uv^T [H][d][r], bf16
    assert mla.mla_latent_attn_unabsorbed_workspace_size(2, 64, 4, 128, 512, BF16) == \
        (2 * 2 * 64 * 4 * 128 + 2 * 4 * 128 * 512) * 2
    assert mla.mla_latent_attn_unabsorbed_workspace_size(2, 64, 4, 128, 512, F32) == 0
    assert mla.mla_latent_attn_unabsorbed_workspace_size(2, 64, 4, 64, 512, BF16) == 0


def varlen(**kw):
    a = dict(q=P, kv=P, cu=P, wk=P, wv=P, out=P, B=2, total=100, H=4, d=32, r=32, scale=0.17, dt=F32, ws=P,
             wsb=1 << 40)
    a.update(kw)
    return mla.mla_decode_varlen_fwd_raw(a["q"], a["kv"], a["cu"], a["wk"], a["wv"], a["out"], a["B"], a["total"],
                                         a["H"], a["d"], a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    ({"cu": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"cu": P + 2}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"q": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"total": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"B": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"dt": 5}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"r": 2048}, mla.MLA_ERR_UNSUPPORTED),
    ({"B": 4096, "total": 1 << 20}, mla.MLA_ERR_UNSUPPORTED),   # B * total >= 2^31: the length prefix is int32
    ({"wsb": 3}, mla.MLA_ERR_WORKSPACE),
])
def test_varlen_argument_errors(kw, status):
    assert varlen(**kw) == status
    assert mla.last_error() != ""


def test_varlen_workspace_matches_padded():
    for dt in (F32, BF16):
        assert mla.mla_decode_varlen_workspace_size(64, 300000, 32, 128, 512, dt) == \
            mla.mla_decode_workspace_size(64, 300000, 32, 128, 512, dt) > 0


@pytest.mark.parametrize("args,status", [
    ((0, P, P, 2, 8, 32, F32), mla.MLA_ERR_INVALID_ARGUMENT),     # null cache
    ((P, 0, P, 2, 8, 32, F32), mla.MLA_ERR_INVALID_ARGUMENT),     # null lengths
    ((P, P + 2, P, 2, 8, 32, F32), mla.MLA_ERR_INVALID_ARGUMENT), # misaligned lengths
    ((P, P, P, 0, 8, 32, F32), mla.MLA_ERR_INVALID_ARGUMENT),
    ((P, P, P, 2, 8, 0, BF16), mla.MLA_ERR_INVALID_ARGUMENT),
    ((P, P, P, 2, 8, 32, 9), mla.MLA_ERR_INVALID_ARGUMENT),
])
def test_kv_append_argument_errors(args, status):
    assert mla.mla_kv_append_raw(*args) == status
    assert mla.last_error() != ""


def test_decode_null_lengths():
    assert dec(lens=0) == mla.MLA_ERR_INVALID_ARGUMENT
    assert dec(lens=P + 2) == mla.MLA_ERR_INVALID_ARGUMENT


def test_down_proj_errors():
    assert mla.mla_down_proj_raw(0, P, P, 1, 1, 1, 1, F32) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_down_proj_raw(P, P, P, 1, 0, 1, 1, F32) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_down_proj_raw(P, P, P, 1, 1, 1, 1, 3) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_down_proj_raw(P, P + 4, P, 1, 1, 1, 1, F32) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_down_proj_raw(P, P, P, 1, 1, 1, 4096, F32) == mla.MLA_ERR_UNSUPPORTED


def test_workspace_sizes():
    # float32 path: q_lat and o_lat in float32
    assert mla.mla_latent_attn_workspace_size(2, 64, 4, 32, 32, F32) == 2 * 2 * 64 * 4 * 32 * 4
    # bf16 matrix-core path: q_lat, o_lat in bf16 and W_uv^T
    rows = 8 * 2048 * 16
    assert mla.mla_latent_attn_workspace_size(8, 2048, 16, 128, 512, BF16) == \
        (2 * rows * 512 + 16 * 128 * 512) * 2
    assert mla.mla_latent_attn_workspace_size(0, 1, 1, 1, 1, F32) == 0
    assert mla.mla_decode_workspace_size(64, 8192, 32, 128, 512, BF16) > 64 * 32 * 512 * 4
    assert mla.mla_decode_workspace_size(1, 1, 1, 1, 1, 9) == 0


def masked(**kw):
    a = dict(q=P, kv=P, mask=P + 1, wk=P, wv=P, out=P, B=2, T=64, H=4, d=32, r=32, scale=0.17, dt=F32, ws=P,
             wsb=1 << 40)
    a.update(kw)
    return mla.mla_latent_attn_fwd_masked_raw(a["q"], a["kv"], a["mask"], a["wk"], a["wv"], a["out"], a["B"], a["T"],
                                              a["H"], a["d"], a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,status", [
    ({"mask": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"q": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"T": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"dt": 4}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"scale": float("nan")}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"kv": P + 4}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"r": 2048}, mla.MLA_ERR_UNSUPPORTED),
    ({"wsb": 1000}, mla.MLA_ERR_WORKSPACE),
])
def test_masked_argument_errors(kw, status):
    assert masked(**kw) == status
    assert mla.last_error() != ""


def test_masked_needs_room_for_the_mask_bits():
    # bf16 matrix-core shape: the unmasked workspace is too small (the mask bits follow it)
    wsb = mla.mla_latent_attn_workspace_size(2, 100, 4, 128, 512, BF16)
    assert masked(dt=BF16, d=128, r=512, T=100, wsb=wsb) == mla.MLA_ERR_WORKSPACE


def test_masked_workspace_size():
    # bf16 matrix-core path: the unmasked workspace, then the packed visible latents [B][T][r] bf16 and
    # two int32 tables [B][T] (visible keys up to t, position of the j-th visible key)
    for T in (1, 32, 33, 100, 16384):
        assert mla.mla_latent_attn_masked_workspace_size(2, T, 4, 128, 512, BF16) == \
            mla.mla_latent_attn_workspace_size(2, T, 4, 128, 512, BF16) + 2 * T * (512 * 2 + 8)
    # float32 path reads the byte mask directly
    assert mla.mla_latent_attn_masked_workspace_size(2, 64, 4, 32, 32, F32) == \
        mla.mla_latent_attn_workspace_size(2, 64, 4, 32, 32, F32)
    assert mla.mla_latent_attn_masked_workspace_size(0, 64, 4, 32, 32, F32) == 0


def full(**kw):
    a = dict(hid=P, wd=P, q=P, wk=P, wv=P, kv=P, out=P, B=2, T=64, D=256, H=4, d=32, r=32, scale=0.17, dt=F32, ws=P,
             wsb=1 << 40)
    a.update(kw)
    return mla.mla_latent_attn_fwd_full_raw(a["hid"], a["wd"], a["q"], a["wk"], a["wv"], a["kv"], a["out"], a["B"],
                                            a["T"], a["D"], a["H"], a["d"], a["r"], a["scale"], a["dt"], a["ws"],
                                            a["wsb"])


@pytest.mark.parametrize("kw,status", [
    ({"hid": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"wd": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"kv": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"D": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"hid": P + 4}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"wd": P + 8}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"T": 0}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"scale": float("inf")}, mla.MLA_ERR_INVALID_ARGUMENT),
    ({"r": 2048}, mla.MLA_ERR_UNSUPPORTED),
    ({"wsb": 100}, mla.MLA_ERR_WORKSPACE),
])
def test_full_argument_errors(kw, status):
    assert full(**kw) == status
    assert mla.last_error() != ""


def test_full_workspace_size():
    # bf16 matrix-core down-projection: the attention workspace, then w_down^T [r][D] bf16
    base = mla.mla_latent_attn_workspace_size(8, 2048, 16, 128, 512, BF16)
    assert mla.mla_latent_attn_full_workspace_size(8, 2048, 1024, 16, 128, 512, BF16) == base + 1024 * 512 * 2
    # float32 and D % 64 != 0: the vector down-projection needs no scratch
    assert mla.mla_latent_attn_full_workspace_size(4, 512, 1024, 8, 64, 128, F32) == \
        mla.mla_latent_attn_workspace_size(4, 512, 8, 64, 128, F32)
    assert mla.mla_latent_attn_full_workspace_size(2, 50, 96, 4, 128, 128, BF16) == \
        mla.mla_latent_attn_workspace_size(2, 50, 4, 128, 128, BF16)
    assert mla.mla_latent_attn_full_workspace_size(2, 50, 0, 4, 128, 128, BF16) == 0
    # the workspace test above must pass with the full requirement, not the attention one
    need = mla.mla_latent_attn_full_workspace_size(2, 64, 1024, 4, 128, 512, BF16)
    assert full(dt=BF16, d=128, r=512, D=1024, wsb=need - 1) == mla.MLA_ERR_WORKSPACE


def test_auto_form_choice():
    # unabsorbed where it is covered and r > d; absorbed otherwise
    assert mla.mla_latent_attn_auto_form(2, 16384, 64, 128, 512, BF16) == 1
    assert mla.mla_latent_attn_auto_form(8, 2048, 16, 128, 256, BF16) == 1
    assert mla.mla_latent_attn_auto_form(8, 2048, 16, 128, 128, BF16) == 0     # r = d
    assert mla.mla_latent_attn_auto_form(8, 2048, 16, 64, 512, BF16) == 0      # d not covered by the unabsorbed form
    assert mla.mla_latent_attn_auto_form(4, 512, 8, 64, 128, F32) == 0         # float32
    assert mla.mla_latent_attn_auto_workspace_size(2, 64, 4, 128, 512, BF16) == \
        mla.mla_latent_attn_unabsorbed_workspace_size(2, 64, 4, 128, 512, BF16)
    assert mla.mla_latent_attn_auto_workspace_size(2, 64, 4, 32, 32, F32) == \
        mla.mla_latent_attn_workspace_size(2, 64, 4, 32, 32, F32)


# ---- the LDS-limit check: a device that allows less LDS per block than a
# kernel needs makes the call fail with MLA_ERR_UNSUPPORTED before anything is
# enqueued (here on a host without a device: the override replaces the query)
@pytest.fixture
def lds_limit():
    yield mla.mla_set_lds_limit_override
    mla.mla_set_lds_limit_override(0)


def unabs(**kw):
    a = dict(q=P, kv=P, wk=P, wv=P, out=P, B=2, T=64, H=4, d=128, r=512, scale=0.17, dt=BF16, ws=P, wsb=1 << 40)
    a.update(kw)
    return mla.mla_latent_attn_fwd_unabsorbed_raw(a["q"], a["kv"], a["wk"], a["wv"], a["out"], a["B"], a["T"],
                                                  a["H"], a["d"], a["r"], a["scale"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("fn", [attn, dec, unabs])
def test_lds_limit_below_the_kernels_need(fn, lds_limit):
    lds_limit(64 * 1024)   # well below the 140 KB the r = 512 kernels take
    assert fn(dt=BF16, d=128, r=512) == mla.MLA_ERR_UNSUPPORTED
    assert "LDS" in mla.last_error()


def test_lds_limit_is_only_checked_for_the_matrix_core_paths(lds_limit):
    lds_limit(1024)
    # float32 runs the vector kernels, which need no large LDS tile: the call
    # gets past the check and fails only at the (absent) device
    assert attn() == mla.MLA_ERR_HIP


def test_decode_split_count_control():
    try:
        for bad in (-1, 1025):
            assert mla.load().mla_decode_set_splits(bad) == mla.MLA_ERR_INVALID_ARGUMENT
            assert "splits" in mla.last_error()
        for good in (1, 7, 1024, 0):
            mla.mla_decode_set_splits(good)
    finally:
        mla.mla_decode_set_splits(0)
