"""Pins of oracle/materialized.py (CPU).

  * its P and O equal the C oracle's materialized forward (independent code);
  * with no cotangent on P its VJP equals the C oracle's VJP;
  * with a cotangent on P its VJP equals central finite differences of
    L = sum(dO * O) + sum(dPx * P) evaluated through the C oracle's forward;
  * dropping the dPx term is caught by the same differences.
"""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import materialized as mat


@pytest.mark.parametrize("Hq,Hkv,T,D", [(4, 2, 23, 8), (3, 1, 16, 16)])
def test_forward_and_vjp_match_c_oracle(orc, Hq, Hkv, T, D):
    x = si.causal_inputs(2, Hq, Hkv, T, D, seed=60 + T)
    scale = 1.0 / np.sqrt(D)
    ro, _, rp = orc.causal_fwd(x["q"], x["k"], x["v"], scale, return_p=True)
    o, p = mat.forward(x["q"], x["k"], x["v"], scale)
    np.testing.assert_allclose(p, rp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
    dq, dk, dv = mat.backward(x["q"], x["k"], x["v"], x["dout"], None, scale)
    rdq, rdk, rdv = orc.causal_bwd(x["q"], x["k"], x["v"], x["dout"], scale)
    for a, b in ((dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def _loss(orc, q, k, v, dout, dpx, scale):
    o, _, p = orc.causal_fwd(q, k, v, scale, return_p=True)
    return float((o * dout).sum() + (p * dpx).sum())


def test_vjp_with_probability_cotangent_matches_finite_differences(orc):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, T, D = 1, 2, 1, 5, 3
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    dout = rng.standard_normal((B, Hq, T, D))
    dpx = rng.standard_normal((B, Hq, T, T))
    scale = 0.7
    dq, dk, dv = mat.backward(q, k, v, dout, dpx, scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = _loss(orc, q, k, v, dout, dpx, scale)
            x[idx] = keep - eps
            lm = _loss(orc, q, k, v, dout, dpx, scale)
            x[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)
    # plausible mistakes are caught by the same differences
    wrong, _, _ = mat.backward(q, k, v, dout, None, scale)  # dPx term dropped
    assert not np.allclose(wrong, dq, rtol=1e-3)
