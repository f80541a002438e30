"""The Python binding checks, before anything is enqueued, that the tensors
it is given agree with each other in shape and dtype: the C ABI sees only
pointers and sizes, and a mismatch would make the kernels read or write
outside a tensor.  These run on the CPU with host tensors: the shape checks
come before the device check, so a mismatch raises ValueError naming the
tensor, and matching host tensors then fail only for not being on the GPU."""
import pytest
import torch

import rank_latent_causal_mla_amd as mla

BF = torch.bfloat16


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def prefill_args(B=2, T=8, H=4, d=32, r=64):
    return dict(q=t(B, T, H, d), kv_latent=t(B, T, r), w_up_k=t(r, H, d), w_up_v=t(r, H, d))


PREFILL = [mla.mla_latent_attn_fwd, mla.mla_latent_attn_fwd_auto, mla.mla_latent_attn_fwd_unabsorbed]


@pytest.mark.parametrize("fwd", PREFILL)
@pytest.mark.parametrize("name,bad", [
    ("q", t(2, 8, 4)),                  # not 4-d
    ("kv_latent", t(3, 8, 64)),         # wrong batch
    ("kv_latent", t(2, 9, 64)),         # wrong length
    ("w_up_k", t(64, 4, 16)),           # wrong head dim
    ("w_up_v", t(32, 4, 32)),           # wrong rank
    ("w_up_v", t(64, 5, 32)),           # wrong head count
    ("w_up_k", t(64, 4, 32, dtype=torch.float32)),   # dtype differs from q
])
def test_prefill_rejects_mismatched_inputs(fwd, name, bad):
    a = prefill_args()
    a[name] = bad
    with pytest.raises(ValueError, match=name):
        fwd(**a)


@pytest.mark.parametrize("fwd", PREFILL)
def test_prefill_with_matching_host_tensors_fails_only_on_the_device(fwd):
    with pytest.raises(ValueError, match="GPU"):
        fwd(**prefill_args())


def test_masked_rejects_a_mask_of_the_wrong_shape():
    a = prefill_args()
    with pytest.raises(ValueError, match="key_mask"):
        mla.mla_latent_attn_fwd_masked(a["q"], a["kv_latent"], torch.ones(2, 7, dtype=torch.uint8), a["w_up_k"],
                                       a["w_up_v"])
    with pytest.raises(ValueError, match="kv_latent"):
        mla.mla_latent_attn_fwd_masked(a["q"], t(2, 9, 64), torch.ones(2, 8, dtype=torch.uint8), a["w_up_k"],
                                       a["w_up_v"])


def decode_args(B=3, Tmax=16, H=4, d=32, r=64):
    return dict(q=t(B, 1, H, d), kv_latent=t(B, Tmax, r), seq_lens=torch.ones(B, dtype=torch.int32),
                w_up_k=t(r, H, d), w_up_v=t(r, H, d))


@pytest.mark.parametrize("name,bad", [
    ("q", t(2, 1, 4, 32)),                           # fewer sequences than the cache
    ("q", t(3, 2, 4, 32)),                           # more than one query per sequence
    ("seq_lens", torch.ones(2, dtype=torch.int32)),  # too few lengths
    ("seq_lens", torch.ones(3, dtype=torch.int64)),  # not int32
    ("w_up_k", t(64, 5, 32)),                        # head count differs from q
    ("kv_latent", t(3, 16, 64, dtype=torch.float32)),  # dtype differs from q
])
def test_decode_rejects_mismatched_inputs(name, bad):
    a = decode_args()
    a[name] = bad
    with pytest.raises(ValueError, match=name):
        mla.mla_decode_fwd(**a)


def test_decode_with_matching_host_tensors_fails_only_on_the_device():
    with pytest.raises(ValueError, match="GPU"):
        mla.mla_decode_fwd(**decode_args())


@pytest.mark.parametrize("name,bad", [
    ("cu_seqlens", torch.zeros(3, dtype=torch.int32)),   # B + 1 = 4 entries needed
    ("cu_seqlens", torch.zeros(4, dtype=torch.int64)),
    ("kv_latent", t(3, 16, 64)),                         # packed cache is 2-d
    ("w_up_v", t(32, 4, 32)),
])
def test_varlen_rejects_mismatched_inputs(name, bad):
    a = dict(q=t(3, 1, 4, 32), kv_latent=t(40, 64), cu_seqlens=torch.zeros(4, dtype=torch.int32),
             w_up_k=t(64, 4, 32), w_up_v=t(64, 4, 32))
    a[name] = bad
    with pytest.raises(ValueError, match=name):
        mla.mla_decode_varlen_fwd(**a)


def test_kv_append_rejects_mismatched_inputs():
    cache, lens = t(3, 16, 64), torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="new_latent"):
        mla.mla_kv_append(cache, lens, t(3, 32))
    with pytest.raises(ValueError, match="new_latent"):
        mla.mla_kv_append(cache, lens, t(3, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="seq_lens"):
        mla.mla_kv_append(cache, torch.zeros(2, dtype=torch.int32), t(3, 64))


def test_down_proj_and_full_path_reject_mismatched_inputs():
    with pytest.raises(ValueError, match="w_down"):
        mla.mla_down_proj(t(2, 8, 128), t(64, 32))
    a = prefill_args()
    with pytest.raises(ValueError, match="hidden"):
        mla.mla_latent_attn_fwd_full(t(2, 7, 128), t(128, 64), a["q"], a["w_up_k"], a["w_up_v"])
    with pytest.raises(ValueError, match="w_up_k"):
        mla.mla_latent_attn_fwd_full(t(2, 8, 128), t(128, 64), a["q"], t(32, 4, 32), a["w_up_v"])
