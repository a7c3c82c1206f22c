"""GPU tests of the autograd binding and of the grouped-query backward at long T.

  * causal_attention's gradients are the C-ABI backward's outputs, bit for bit,
    and match the oracle's VJP;
  * composed with ordinary torch ops (projections of one input), the input's
    gradient matches the chain rule evaluated in float64 on the CPU from the
    oracle's VJP;
  * at the 8192-token grouped-query size (Hq=16, Hkv=4, d=64) the forward and
    backward are checked on sampled rows of dQ and sampled key positions of dK,
    dV (oracle/sampled_vjp.py computes each from its definition) and on
    identities that hold at any size: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    over each key/value head's query heads.
"""
import math

import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_GRAD, TOL_O, announce, rel_err, require_gpu
from oracle import sampled_vjp as sv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("B,Hq,Hkv,T,D", [(2, 8, 2, 300, 64), (1, 4, 4, 129, 32), (3, 6, 1, 64, 16)])
def test_autograd_matches_direct_calls_and_oracle(dev, orc, B, Hq, Hkv, T, D):
    announce(f"autograd B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=500 + T)
    q, k, v, do = (host[n].to(dev) for n in ("q", "k", "v", "dout"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attn.causal_attention(qa, ka, va)
    o.backward(do)
    torch.cuda.synchronize()
    o2, lse2 = attn.attn_causal_fwd(q, k, v)
    dq2, dk2, dv2 = attn.attn_causal_bwd(q, k, v, o2, lse2, do)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    assert torch.equal(ka.grad, dk2) and torch.equal(va.grad, dv2)
    assert rel_err(qa.grad, dq2) <= 1e-6  # dQ sums with float atomics
    ro, _ = orc.causal_fwd(host["q"], host["k"], host["v"])
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    assert rel_err(o.detach(), ro) <= TOL_O
    for nm, a, b in (("dQ", qa.grad, rdq), ("dK", ka.grad, rdk), ("dV", va.grad, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


def test_autograd_composes_with_projections(dev, orc):
    """x -> (Q, K, V) by three projections, heads split by a view and a transpose
    (non-contiguous inputs), loss = sum(O * R); dL/dx against the chain rule in
    float64 from the oracle's VJP with dO = R."""
    announce("autograd composition")
    B, T, C, Hq, Hkv, D = 2, 96, 48, 4, 2, 16
    g = torch.Generator("cpu").manual_seed(21)
    x = torch.randn((B, T, C), generator=g)
    wq = torch.randn((C, Hq * D), generator=g) / math.sqrt(C)
    wk = torch.randn((C, Hkv * D), generator=g) / math.sqrt(C)
    wv = torch.randn((C, Hkv * D), generator=g) / math.sqrt(C)
    r = torch.randn((B, Hq, T, D), generator=g)
    xg = x.to(dev).requires_grad_(True)

    def heads(t, H):
        return t.view(B, T, H, D).transpose(1, 2)

    q = heads(xg @ wq.to(dev), Hq)
    k = heads(xg @ wk.to(dev), Hkv)
    v = heads(xg @ wv.to(dev), Hkv)
    o = attn.causal_attention(q, k, v)
    (o * r.to(dev)).sum().backward()
    torch.cuda.synchronize()
    # expected, float64 on the CPU
    x64, wq64, wk64, wv64 = (t.double().numpy() for t in (x, wq, wk, wv))
    q64 = (x64 @ wq64).reshape(B, T, Hq, D).transpose(0, 2, 1, 3)
    k64 = (x64 @ wk64).reshape(B, T, Hkv, D).transpose(0, 2, 1, 3)
    v64 = (x64 @ wv64).reshape(B, T, Hkv, D).transpose(0, 2, 1, 3)
    dq, dk, dv = orc.causal_bwd(q64, k64, v64, r.double().numpy())
    def flat(t, H):
        return t.transpose(0, 2, 1, 3).reshape(B, T, H * D)
    dx = flat(dq, Hq) @ wq64.T + flat(dk, Hkv) @ wk64.T + flat(dv, Hkv) @ wv64.T
    assert rel_err(xg.grad, dx) <= TOL_GRAD, rel_err(xg.grad, dx)


DQ_ROWS = [0, 1, 15, 63, 64, 65, 1000, 4095, 4096, 8127, 8128, 8190, 8191]
DKV_COLS = [8191, 8190, 8176, 8160, 8128, 8100, 8064]


def test_gqa_t8192_forward_backward(dev, orc):
    """The 8192-token grouped-query shape through autograd: sampled outputs and
    whole-tensor identities."""
    c = si.CAUSAL_WORKLOADS["gqa_b1_hq16_hkv4_t8192_d64"]
    announce("gqa T=8192 fwd+bwd (autograd)")
    host = si.causal_inputs(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["seed"], with_do=True)
    q, k, v, do = (host[n].to(dev) for n in ("q", "k", "v", "dout"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attn.causal_attention(qa, ka, va)
    o.backward(do)
    torch.cuda.synchronize()
    dq, dk, dv = qa.grad[0].cpu(), ka.grad[0].cpu(), va.grad[0].cpu()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    scale = 1.0 / 8.0
    hq, hk, hv, hdo = host["q"][0], host["k"][0], host["v"][0], host["dout"][0]
    rdq = sv.dq_rows(hq, hk, hv, hdo, DQ_ROWS, scale)
    assert rel_err(dq[:, DQ_ROWS], rdq) <= TOL_GRAD, rel_err(dq[:, DQ_ROWS], rdq)
    rdk, rdv = sv.dkv_cols(hq, hk, hv, hdo, DKV_COLS, scale)
    assert rel_err(dk[:, DKV_COLS], rdk) <= TOL_GRAD, rel_err(dk[:, DKV_COLS], rdk)
    assert rel_err(dv[:, DKV_COLS], rdv) <= TOL_GRAD, rel_err(dv[:, DKV_COLS], rdv)
    # identities over whole tensors (each P row sums to 1, each dS row to 0)
    G = c["Hq"] // c["Hkv"]
    want_dv_sum = hdo.double().sum(1).reshape(c["Hkv"], G, c["D"]).sum(1)
    assert rel_err(dv.double().sum(1), want_dv_sum) <= 1e-4
    dk_sum = dk.double().sum(1)
    assert float(dk_sum.abs().max()) <= 1e-3 * float(dk.abs().max()) * math.sqrt(c["T"])
    # one sampled forward row through the dense decode definition
    i = 5000
    ro, _ = orc.decode_dense(hq[:, i, :], hk[:, :i + 1, :].transpose(0, 1), hv[:, :i + 1, :].transpose(0, 1),
                             scale)
    assert rel_err(o.detach()[0, :, i, :].cpu(), ro) <= TOL_O
