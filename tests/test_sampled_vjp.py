"""Pins of oracle/sampled_vjp.py (CPU): every sampled row of dQ and every sampled
key of dK, dV must equal the full oracle VJP (independent C code, itself pinned by
brute force and finite differences) on small grouped-query shapes; a dropped
scale or a missing group sum must be caught."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import sampled_vjp as sv


@pytest.mark.parametrize("Hq,Hkv,T,D", [(4, 2, 40, 8), (6, 3, 33, 16), (2, 2, 17, 32)])
def test_sampled_vjp_matches_full_oracle(orc, Hq, Hkv, T, D):
    x = si.causal_inputs(1, Hq, Hkv, T, D, seed=90 + T)
    scale = 1.0 / np.sqrt(D)
    dq, dk, dv = orc.causal_bwd(x["q"], x["k"], x["v"], x["dout"], scale)
    rows = [0, 1, T // 2, T - 1]
    cols = [0, 3, T // 3, T - 2, T - 1]
    q, k, v, do = x["q"][0], x["k"][0], x["v"][0], x["dout"][0]
    sdq = sv.dq_rows(q, k, v, do, rows, scale)
    sdk, sdv = sv.dkv_cols(q, k, v, do, cols, scale)
    np.testing.assert_allclose(sdq, dq[0][:, rows], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(sdk, dk[0][:, cols], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(sdv, dv[0][:, cols], rtol=1e-11, atol=1e-13)


def test_mistakes_are_caught(orc):
    x = si.causal_inputs(1, 4, 2, 24, 8, seed=7)
    scale = 1.0 / np.sqrt(8)
    dq, dk, dv = orc.causal_bwd(x["q"], x["k"], x["v"], x["dout"], scale)
    q, k, v, do = x["q"][0], x["k"][0], x["v"][0], x["dout"][0]
    # a dQ without its scale factor
    assert not np.allclose(sv.dq_rows(q, k, v, do, [5, 20], 1.0) * 1.0, dq[0][:, [5, 20]], rtol=1e-6)
    # dK, dV from only the first query head of each group (group sum missing)
    sdk, sdv = sv.dkv_cols(q[::2], k, v, do[::2], [3, 10], scale)
    assert not np.allclose(sdv, dv[0][:, [3, 10]], rtol=1e-6)
