"""Plausible mistakes planted in copies of the CPU oracle must each fail a pin.

Every mutant is a text substitution in a temporary copy of oracle/attn_oracle.c,
compiled with gcc into a temporary directory and loaded next to the real one.
The pins of tests/oracle_pins.py are run against it; at least one must fail.
All mutants stay in bounds (they change arithmetic or indices within the same
arrays), so a mutant can give wrong numbers but not crash.
"""
import os
import re
import subprocess

import pytest

import oracle_pins
from oracle.oracle import Oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")


def _strict_mask(src):
    """Exclude the diagonal key in the probability rows (mask t_k >= t_q)."""
    start = src.index("static void head_probabilities")
    end = src.index("int oracle_causal_fwd")
    body = src[start:end].replace("j <= i", "j < i").replace("j = i + 1; j < T", "j = i; j < T")
    return src[:start] + body + src[end:]


MUTANTS = {
    "drop_scale": ("s *= scale;", ""),
    "lse_without_max": ("if (lse) lse[i] = m + log(z);", "if (lse) lse[i] = log(z);"),
    "strict_mask": _strict_mask,
    "output_uses_P_transposed": ("acc += P[i * T + j] * vg[j * D + c];",
                                 "acc += P[j * T + i] * vg[j * D + c];"),
    "gqa_modulo_heads_fwd": ("h = bh % Hq, g = h / G;", "h = bh % Hq, g = h % Hkv;"),
    "delta_without_P": ("delta += P[i * T + j] * dp;", "delta += dp;"),
    "dS_sign": ("P[i * T + j] * (dS[i * T + j] - delta)", "P[i * T + j] * (delta - dS[i * T + j])"),
    "dQ_no_scale": ("dqh[i * D + c] = scale * acc;", "dqh[i * D + c] = acc;"),
    "dK_transposed_dS": ("const double dsij = dS[i * T + j], pij = P[i * T + j];",
                         "const double dsij = dS[j * T + i], pij = P[i * T + j];"),
    "dV_transposed_P": ("const double dsij = dS[i * T + j], pij = P[i * T + j];",
                        "const double dsij = dS[i * T + j], pij = P[j * T + i];"),
    "dV_not_group_summed": ("dvg[e] += dvh[e];", "dvg[e] = dvh[e];"),
    "dK_not_group_summed": ("dkg[e] += dkh[e];", "dkg[e] = dkh[e];"),
    "dK_no_scale": ("for (int64_t e = 0; e < T * D; ++e) dkh[e] = scale * dkh[e];", ""),
    "gqa_modulo_heads_bwd": ("h = bh % Hq, kvh = h / G;", "h = bh % Hq, kvh = h % Hkv;"),
    "bwd_strided_groups": ("for (int64_t h = g * G; h < (g + 1) * G; ++h)",
                           "for (int64_t h = g; h < Hq; h += Hkv)"),
    "decode_no_scale": ("p[t] = scale * s;", "p[t] = s;"),
    "decode_lse_without_max": ("if (lse) lse[h] = m + log(z);", "if (lse) lse[h] = log(z);"),
    "decode_gqa_modulo": ("const int64_t g = h / G;\n        double m", "const int64_t g = h % Hkv;\n        double m"),
    "decode_pool_axes_swapped": ("((phys * Hkv + g) * page_size + t % page_size) * D",
                                 "((phys * page_size + t % page_size) * Hkv + g) * D"),
    "decode_drops_newest": ("vseq, n, Hq, Hkv, D, scale,", "vseq, n - 1, Hq, Hkv, D, scale,"),
    "prefill_sees_whole_sequence": ("kseq, vseq, pos + 1, Hq, Hkv, D, scale,", "kseq, vseq, n, Hq, Hkv, D, scale,"),
    "prefill_rows_reversed": ("const int64_t row = token_start[s] + j;",
                              "const int64_t row = token_start[s + 1] - 1 - j;"),
    "prefill_positions_from_start": ("const int64_t pos = n - n_new + j;", "const int64_t pos = j;"),
}


def _mutate(name):
    src = open(SRC).read()
    m = MUTANTS[name]
    if callable(m):
        out = m(src)
    else:
        old, new = m
        assert src.count(old) == 1, f"mutation anchor for {name} is not unique"
        out = src.replace(old, new)
    assert out != src
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    csrc = tmp_path / "mutant.c"
    csrc.write_text(_mutate(name))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-w", "-o",
                    str(lib), str(csrc), "-lm"], check=True)
    mutant = Oracle(str(lib))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError) as e:
            caught.append((pin.__name__, repr(e)[:120]))
            break
    assert caught, f"mutant {name} passed every pin"


def test_anchor_regex_sanity():
    # the strict-mask mutant must actually change the probability loops
    src = open(SRC).read()
    assert re.search(r"j <= i", src)
    assert _strict_mask(src) != src
