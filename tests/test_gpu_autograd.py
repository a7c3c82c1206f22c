"""GPU tests of the autograd binding and of the grouped-query backward at long T.

  * causal_attention's gradients are the C-ABI backward's outputs, bit for bit,
    and match the oracle's VJP;
  * composed with ordinary torch ops (projections of one input), the input's
    gradient matches the chain rule evaluated in float64 on the CPU from the
    oracle's VJP;
  * at the 8192-token grouped-query size (Hq=16, Hkv=4, d=64) the forward and
    backward are compared with the oracle on whole tensors (O, dQ, dK, dV: every
    key block, including those that two work-groups add atomically), sampled rows
    of dQ are compared with oracle/sampled_vjp.py (a second route through the
    definition), and identities that hold at any size are checked: sum_j dK_j = 0
    and sum_j dV_j = sum_i dO_i over each key/value head's query heads.
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


def test_gqa_t8192_forward_backward(dev, gqa_t8192_reference):
    """The 8192-token grouped-query shape through autograd: whole tensors against the
    oracle, sampled dQ rows against the sampled-VJP oracle, whole-tensor identities."""
    ref = gqa_t8192_reference
    host = ref["host"]
    c = si.CAUSAL_WORKLOADS["gqa_b1_hq16_hkv4_t8192_d64"]
    announce("gqa T=8192 fwd+bwd (autograd, whole tensors)")
    q, k, v, do = (host[n].to(dev) for n in ("q", "k", "v", "dout"))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = attn.causal_attention(qa, ka, va, scale=ref["scale"])
    o.backward(do)
    torch.cuda.synchronize()
    dq, dk, dv = qa.grad.cpu(), ka.grad.cpu(), va.grad.cpu()
    assert rel_err(o.detach(), ref["o"]) <= TOL_O, rel_err(o.detach(), ref["o"])
    for nm, a, b in (("dQ", dq, ref["dq"]), ("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))
    # the key blocks that two work-groups of the backward add onto zero (the first
    # key block of each pair) on their own, so a wrong sum there cannot hide behind
    # a larger error elsewhere
    for kb in (0, 1, 31, 63):
        sl = slice(64 * kb, 64 * kb + 64)
        for nm, a, b in (("dK", dk, ref["dk"]), ("dV", dv, ref["dv"])):
            assert rel_err(a[:, :, sl], b[:, :, sl]) <= TOL_GRAD, (nm, kb, rel_err(a[:, :, sl], b[:, :, sl]))
    scale = ref["scale"]
    hq, hk, hv, hdo = host["q"][0], host["k"][0], host["v"][0], host["dout"][0]
    rdq = sv.dq_rows(hq, hk, hv, hdo, DQ_ROWS, scale)
    assert rel_err(dq[0][:, DQ_ROWS], rdq) <= TOL_GRAD, rel_err(dq[0][:, DQ_ROWS], rdq)
    dq, dk, dv = dq[0], dk[0], dv[0]
    # identities over whole tensors (each P row sums to 1, each dS row to 0)
    G = c["Hq"] // c["Hkv"]
    want_dv_sum = hdo.double().sum(1).reshape(c["Hkv"], G, c["D"]).sum(1)
    assert rel_err(dv.double().sum(1), want_dv_sum) <= 1e-4
    dk_sum = dk.double().sum(1)
    assert float(dk_sum.abs().max()) <= 1e-3 * float(dk.abs().max()) * math.sqrt(c["T"])
