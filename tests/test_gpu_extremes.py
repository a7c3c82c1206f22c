"""Size and value extremes against the CPU oracle.

* 32768-token causal forward and backward, once with grouped-query heads (B=1, Hq=4,
  Hkv=2: every key block whole in one work-group) and once with one head (its 512 key
  blocks fill the chip once, so the backward takes half pairs and adds the first key
  block of each pair atomically).  The oracle cannot hold [T,T] there: O and LSE are
  checked on sampled rows against its single-query decode over the row's prefix, dQ on
  sampled rows and dK, dV on the last keys against the sampled-VJP oracle (tolerances
  as everywhere: O, LSE 1e-4; gradients 1e-3 of the sampled values' largest
  magnitude), and every key through identities that hold at any size: each dS row sums
  to zero, so sum_j dK_j = 0, and each P row sums to one, so sum_j dV_j = sum_i dO_i per
  KV head.
* A one-hot softmax by construction (each query a multiple of its own key): at scores
  of about 1e6 the forward's O must be V bit for bit; at about 200 (where float32 holds
  the scores that the backward's recompute subtracts) dV must be the group sums of dO
  and dQ, dK vanish to rounding.
* Paged decode over contexts of up to 131072 positions (64-position pages, 2048-entry
  block tables) and a prefill whose new tokens follow a cached prefix of up to 60000.
"""
import math

import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_DECODE, TOL_GRAD, TOL_LSE, TOL_O, announce, rel_err, require_gpu
from oracle import sampled_vjp as sv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (1, 1)])
def test_long_context_forward_backward(dev, orc, Hq, Hkv):
    B, T, D = 1, 32768, 64
    announce(f"long context fwd+bwd B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=32768 + Hq)
    x = {k: v.to(dev) for k, v in host.items()}
    scale = 1.0 / math.sqrt(D)
    o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], scale=scale)
    dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], scale=scale)
    torch.cuda.synchronize()
    q, k, v, do = (host[n][0] for n in ("q", "k", "v", "dout"))
    o_h, lse_h = o[0].cpu(), lse[0].cpu()
    for i in (0, 1, 63, 64, 4095, 16383, 16384, 30001, T - 65, T - 64, T - 1):
        ro, rlse = orc.decode_dense(q[:, i, :], k[:, : i + 1, :].transpose(0, 1), v[:, : i + 1, :].transpose(0, 1),
                                    scale)
        assert rel_err(o_h[:, i, :], ro) <= TOL_O, ("O row", i, rel_err(o_h[:, i, :], ro))
        assert rel_err(lse_h[:, i], rlse) <= TOL_LSE, ("LSE row", i)
    rows = [0, 5, 8191, 20000, T - 1]
    rdq = sv.dq_rows(q, k, v, do, rows, scale)
    assert rel_err(dq[0][:, rows, :], rdq) <= TOL_GRAD, ("dQ rows", rel_err(dq[0][:, rows, :], rdq))
    cols = [T - 160, T - 129, T - 128, T - 64, T - 2, T - 1]
    rdk, rdv = sv.dkv_cols(q, k, v, do, cols, scale)
    assert rel_err(dk[0][:, cols, :], rdk) <= TOL_GRAD, ("dK cols", rel_err(dk[0][:, cols, :], rdk))
    assert rel_err(dv[0][:, cols, :], rdv) <= TOL_GRAD, ("dV cols", rel_err(dv[0][:, cols, :], rdv))
    G = Hq // Hkv
    want_dv_sum = host["dout"][0].double().sum(1).reshape(Hkv, G, D).sum(1)
    assert rel_err(dv[0].double().sum(1), want_dv_sum) <= 1e-4
    dk_sum = dk[0].double().sum(1)
    assert float(dk_sum.abs().max()) <= 1e-3 * float(dk.abs().max()) * math.sqrt(T)
    assert bool(torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all())


def _one_hot_inputs(c, seed=300):
    """Q_hi = c K_gi: query i's own key dominates its scores (B=2, Hq=4, Hkv=2, T=333)."""
    B, Hq, Hkv, T, D = 2, 4, 2, 333, 64
    G = Hq // Hkv
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=seed)
    host["q"] = (host["k"].repeat_interleave(G, dim=1) * c).contiguous()
    scale = 1.0 / math.sqrt(D)
    qd, kd = host["q"].double(), host["k"].double().repeat_interleave(G, dim=1)
    s_all = scale * qd @ kd.transpose(-1, -2)
    diag = torch.diagonal(s_all, dim1=-2, dim2=-1)
    off = s_all.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool), -1), -math.inf).amax(-1)
    return host, scale, G, float(diag.abs().max()), float((diag - off)[..., 1:].min())


def test_one_hot_forward(dev, orc):
    """Scores about 1e6 with the diagonal at least 1e5 above every other one (Q = 1.25e5 K):
    P is one-hot and every other term underflows to exactly zero, so O is V row for row,
    bit for bit (the running max moves by far more than its 2^8 slack and the earlier
    keys' terms are scaled by exactly 0), and LSE is the diagonal score."""
    announce("one-hot forward, scores about 1e6")
    host, scale, G, smax, gap = _one_hot_inputs(1.25e5)
    assert smax > 5e5 and gap > 1e5
    x = {k: v.to(dev) for k, v in host.items()}
    o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), host["v"].repeat_interleave(G, dim=1)), "O must be V row for row"
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"], scale)
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))


def test_one_hot_backward(dev, orc):
    """The backward recomputes P = exp(s - LSE) from two float32 quantities, so it is
    taken at scores that float32 holds to about 1e-5 (Q = 25 K: diagonal about 200, at
    least 50 above every other score; off-diagonal P below e^-50).  dV_j is then the sum
    of dO_j over the query heads of its KV head, and dQ, dK vanish: each dS_ii is the
    difference of two float32 dot products of the same vectors, so they are bounded by
    1e-5 of their terms' size (scale max|K| max|Delta| for dQ, scale max|Q| max|Delta|
    for dK) instead of being compared with the oracle's values of order 1e-20."""
    announce("one-hot backward, scores about 200")
    host, scale, G, smax, gap = _one_hot_inputs(25.0)
    assert 100 < smax < 1000 and gap > 50
    B, Hq, T, D = host["q"].shape
    Hkv = Hq // G
    x = {k: v.to(dev) for k, v in host.items()}
    o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], scale=scale)
    dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], scale=scale)
    torch.cuda.synchronize()
    want_dv = host["dout"].double().reshape(B, Hkv, G, T, D).sum(2)
    assert rel_err(dv, want_dv) <= 1e-4, rel_err(dv, want_dv)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"], scale)
    assert rel_err(dv, rdv) <= TOL_GRAD
    delta = float((host["dout"].double() * host["v"].double().repeat_interleave(G, dim=1)).sum(-1).abs().max())
    for nm, g, big in (("dQ", dq, host["k"]), ("dK", dk, host["q"])):
        bound = 1e-5 * scale * float(big.abs().max()) * delta
        assert float(g.abs().max()) <= bound, (nm, float(g.abs().max()), bound)


def test_long_context_decode(dev, orc):
    S, Hq, Hkv, D, ps = 3, 8, 2, 128, 64
    announce("decode over contexts up to 131072 positions")
    d = si.paged_decode_inputs(S=S, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, ctx_lo=100000, ctx_hi=131072,
                               max_pages=2048, seed=131072)
    d["context_lens"][0] = 131072
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, lse = attn.attn_paged_decode(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"])
    torch.cuda.synchronize()
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE and rel_err(lse, rlse) <= TOL_DECODE, (rel_err(o, ro), rel_err(lse, rlse))


def test_long_cached_prefill(dev, orc):
    announce("prefill after cached prefixes of up to 60000 positions")
    d = si.paged_prefill_inputs(S=2, Hq=8, Hkv=2, D=64, page_size=32, cached_lo=40000, cached_hi=60000, new_lo=200,
                                new_hi=500, max_pages=1900, seed=60000)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, lse = attn.attn_paged_prefill(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"],
                                     x["token_start"])
    torch.cuda.synchronize()
    ro, rlse = orc.paged_prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                                 d["token_start"])
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))
