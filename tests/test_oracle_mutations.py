"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle source, plants one plausible mistake (a dropped
term, a wrong index, a transposed operand, an off-by-one mask), builds it on
the CPU into a temporary library, and checks that at least one pin fails.
"""
import os

import pytest

import oracle
from tests.oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.cpp")

MUTANTS = {
    "diagonal_key_dropped": ("const long n = P.row_nkeys[i];",
                             "const long n = P.row_nkeys[i] > 1 ? P.row_nkeys[i] - 1 : 1;"),
    "v_uses_w_up_k": ("vs += lat * load(P.wv, P.dt_w, w);", "vs += lat * load(P.wk, P.dt_w, w);"),
    "no_max_shift": ("z += std::exp(logit[s] - m);", "z += std::exp(logit[s]);"),
    "no_scale": ("logit[s] = dot * P.scale;", "logit[s] = dot;"),
    "head_ignored": ("const size_t w = (size_t)(rho * H + h) * d + e;",
                     "const size_t w = (size_t)(rho * H + 0) * d + e;"),
    "weights_transposed": ("const size_t w = (size_t)(rho * H + h) * d + e;",
                           "const size_t w = (size_t)(h * r + rho) * d + e;"),
    "no_normalisation": ("p[s] = std::exp(logit[s] - m) / z;", "p[s] = std::exp(logit[s] - m);"),
    "latent_row_halved": ("(size_t)(b * P.Tlat + s) * r + rho", "(size_t)(b * P.Tlat + s / 2) * r + rho"),
    "query_reversed": ("load(P.q, P.dt_q, (size_t)i * d + e)", "load(P.q, P.dt_q, (size_t)i * d + (d - 1 - e))"),
    "down_proj_transposed": ("load(w_down, dt_w, (size_t)i * r + j)", "load(w_down, dt_w, (size_t)j * D + i)"),
    "bf16_widened_wrong": ("<< 16;  // bf16", "<< 15;  // bf16"),
    "decode_length_short": ("rk[b * H + h] = seq_lens[b];", "rk[b * H + h] = seq_lens[b] > 1 ? seq_lens[b] - 1 : 1;"),
    "mask_ignored": ("if (P.key_mask && !P.key_mask[(size_t)b * P.Tlat + s]) logit[s] = -INFINITY;", ""),
    "mask_inverted": ("if (P.key_mask && !P.key_mask[(size_t)b * P.Tlat + s])",
                      "if (P.key_mask && P.key_mask[(size_t)b * P.Tlat + s])"),
    "mask_wrong_batch": ("P.key_mask[(size_t)b * P.Tlat + s]", "P.key_mask[(size_t)0 * P.Tlat + s]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as fh:
        src = fh.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mutant.cpp"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(src=str(mutated), out=str(tmp_path / "mutant.so")))
    failed = []
    for pin_name, pin in PINS.items():
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin_name)
    assert failed, f"no pin catches the planted mistake {name}"
