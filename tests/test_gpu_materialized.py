"""GPU parity of the materialized path (attn_materialized_fwd / _bwd) against
the oracle: P, O and LSE within 1e-4, gradients within 1e-3 (max-abs error
relative to the reference's largest magnitude), with and without a cotangent on
P; P's zeros above the diagonal are exact."""
import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_GRAD, TOL_LSE, TOL_O, announce, rel_err, require_gpu
from oracle import materialized as mat

pytestmark = pytest.mark.gpu

TOL_P = 1e-4  # a reading: P lies in [0, 1] like the softmax weights inside O


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


CASES = [(1, 2, 2, 16, 8), (8, 4, 4, 256, 32), (2, 8, 2, 300, 64), (1, 4, 1, 129, 128), (2, 3, 3, 1, 16),
         (1, 2, 2, 65, 16), (1, 6, 2, 97, 64), (4, 8, 8, 1024, 64)]


@pytest.mark.parametrize("B,Hq,Hkv,T,D", CASES)
def test_materialized_forward_backward(dev, orc, B, Hq, Hkv, T, D):
    announce(f"materialized B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    x = si.causal_inputs(B, Hq, Hkv, T, D, seed=700 + T + D)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse, p = attn.attn_materialized_fwd(q, k, v)
    torch.cuda.synchronize()
    ro, rlse, rp = orc.causal_fwd(x["q"], x["k"], x["v"], scale, return_p=True)
    assert rel_err(p, rp) <= TOL_P, ("P", rel_err(p, rp))
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE
    upper = torch.triu(torch.ones(T, T, dtype=torch.bool, device=dev), 1)
    assert bool((p[..., upper] == 0).all()), "nonzero probability above the diagonal"
    dq, dk, dv = attn.attn_materialized_bwd(q, k, v, o, p, do)
    torch.cuda.synchronize()
    rdq, rdk, rdv = orc.causal_bwd(x["q"], x["k"], x["v"], x["dout"], scale)
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))
    if B * Hq * T * T <= 4_000_000:  # with a cotangent on P (numpy oracle)
        g = torch.Generator("cpu").manual_seed(T)
        dpx = torch.randn((B, Hq, T, T), generator=g)
        dq, dk, dv = attn.attn_materialized_bwd(q, k, v, o, p, do, dp=dpx.to(dev))
        torch.cuda.synchronize()
        rdq, rdk, rdv = mat.backward(x["q"], x["k"], x["v"], x["dout"], dpx, scale)
        for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            assert rel_err(a, b) <= TOL_GRAD, (nm + " with dP", rel_err(a, b))


def test_materialized_rows_sum_to_one(dev):
    x = si.causal_inputs(2, 4, 2, 333, 64, seed=3)
    _, _, p = attn.attn_materialized_fwd(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev))
    s = p.double().sum(-1)
    assert float((s - 1).abs().max()) <= 1e-5
