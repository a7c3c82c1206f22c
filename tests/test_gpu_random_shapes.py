"""Seeded random shapes against the CPU oracle, beyond the fixed cases.

Sizes, head groupings, head widths, page sizes and ragged lengths are drawn from one
generator (random.Random(2026)), so every run checks the same cases:
  * causal forward and backward: O and LSE within 1e-4, dQ/dK/dV within 1e-3 of each
    tensor's largest magnitude;
  * paged decode, both paths (more than 1024 sequences take the fused one): O and LSE
    within 1e-5 of the oracle's decode over the same pages; the no-allocation entry point
    gives the same bits whenever its scratch holds the batch;
  * batched prefill: O and LSE within 1e-4;
  * the materialized path: P, O and LSE within 1e-4 (P's zeros above the diagonal
    exact), its VJP within 1e-3, with a cotangent on P on the smaller cases.
"""
import math
import random

import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_DECODE, TOL_GRAD, TOL_LSE, TOL_O, announce, rel_err, require_gpu
from oracle import materialized as mat

pytestmark = pytest.mark.gpu

_R = random.Random(2026)
D_CHOICES = (8, 16, 32, 64, 128)
G_CHOICES = (1, 1, 2, 3, 4, 5, 8)


def _causal_cases(n):
    out = []
    while len(out) < n:
        B, Hkv, G = _R.randint(1, 3), _R.randint(1, 4), _R.choice(G_CHOICES)
        if B * Hkv * G > 16:
            continue
        T = max(1, int(round(math.exp(_R.uniform(0.0, math.log(640))))))
        out.append((B, Hkv * G, Hkv, T, _R.choice(D_CHOICES), _R.randrange(1 << 20)))
    return out


def _decode_cases(n):
    out = []
    for i in range(n):
        ps, D, G, Hkv = _R.choice((16, 32, 64)), _R.choice(D_CHOICES), _R.choice(G_CHOICES + (16,)), _R.choice((1, 2, 4, 8))
        if Hkv * G > 64:
            G = 64 // Hkv
        S = _R.choice((1, 2, 7, 33, 150, 700)) if i % 6 else _R.randint(1025, 1200)
        hi = _R.randint(1, 3000 if S <= 150 else 400)
        lo = _R.randint(1, hi)
        out.append((S, Hkv * G, Hkv, D, ps, lo, hi, _R.randrange(1 << 20)))
    return out


def _prefill_cases(n):
    out = []
    for _ in range(n):
        ps, D, G, Hkv = _R.choice((16, 32, 64)), _R.choice(D_CHOICES), _R.choice(G_CHOICES), _R.choice((1, 2, 4))
        S = _R.randint(1, 12)
        chi, nhi = _R.randint(0, 500), _R.randint(1, 200)
        out.append((S, Hkv * G, Hkv, D, ps, _R.randint(0, chi), chi, _R.randint(1, nhi), nhi, _R.randrange(1 << 20)))
    return out


def _materialized_cases(n):
    out = []
    while len(out) < n:
        B, Hkv, G = _R.randint(1, 2), _R.randint(1, 3), _R.choice(G_CHOICES)
        if B * Hkv * G > 8:
            continue
        out.append((B, Hkv * G, Hkv, _R.randint(1, 300), _R.choice(D_CHOICES), _R.randrange(1 << 20)))
    return out


CAUSAL = _causal_cases(120)
DECODE = _decode_cases(60)
PREFILL = _prefill_cases(48)
MATERIALIZED = _materialized_cases(20)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("B,Hq,Hkv,T,D,seed", CAUSAL)
def test_random_causal(dev, orc, B, Hq, Hkv, T, D, seed):
    announce(f"random causal B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} seed={seed}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed)
    x = {k: v.to(dev) for k, v in host.items()}
    scale = D ** -0.5
    o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], scale=scale)
    dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], scale=scale)
    torch.cuda.synchronize()
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"], scale)
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"], scale)
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


@pytest.mark.parametrize("S,Hq,Hkv,D,ps,lo,hi,seed", DECODE)
def test_random_decode(dev, orc, S, Hq, Hkv, D, ps, lo, hi, seed):
    announce(f"random decode S={S} Hq={Hq} Hkv={Hkv} D={D} page={ps} ctx={lo}..{hi} seed={seed}")
    d = si.paged_decode_inputs(S=S, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, ctx_lo=lo, ctx_hi=hi,
                               max_pages=math.ceil(hi / ps) + 1, seed=seed)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, lse = attn.attn_paged_decode(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"])
    torch.cuda.synchronize()
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE and rel_err(lse, rlse) <= TOL_DECODE, (rel_err(o, ro), rel_err(lse, rlse))
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    try:
        attn.attn_paged_decode_noalloc(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"], o2,
                                       lse2)
    except attn.AttnError as e:
        assert e.status == attn.ATTN_WORKSPACE_TOO_SMALL, e
        return
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("S,Hq,Hkv,D,ps,clo,chi,nlo,nhi,seed", PREFILL)
def test_random_prefill(dev, orc, S, Hq, Hkv, D, ps, clo, chi, nlo, nhi, seed):
    announce(f"random prefill S={S} Hq={Hq} Hkv={Hkv} D={D} page={ps} cached={clo}..{chi} new={nlo}..{nhi}")
    d = si.paged_prefill_inputs(S=S, Hq=Hq, Hkv=Hkv, D=D, page_size=ps, cached_lo=clo, cached_hi=chi, new_lo=nlo,
                                new_hi=nhi, max_pages=math.ceil((chi + nhi) / ps) + 1, seed=seed)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    o, lse = attn.attn_paged_prefill(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"],
                                     x["token_start"])
    torch.cuda.synchronize()
    ro, rlse = orc.paged_prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                                 d["token_start"])
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))


@pytest.mark.parametrize("B,Hq,Hkv,T,D,seed", MATERIALIZED)
def test_random_materialized(dev, orc, B, Hq, Hkv, T, D, seed):
    announce(f"random materialized B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} seed={seed}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed)
    x = {k: v.to(dev) for k, v in host.items()}
    scale = D ** -0.5
    o, lse, p = attn.attn_materialized_fwd(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    ro, rlse, rp = orc.causal_fwd(host["q"], host["k"], host["v"], scale, return_p=True)
    assert rel_err(p, rp) <= 1e-4 and rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE
    upper = torch.triu(torch.ones(T, T, dtype=torch.bool, device=dev), 1)
    assert bool((p[..., upper] == 0).all())
    g = torch.Generator("cpu").manual_seed(seed)
    dpx = torch.randn((B, Hq, T, T), generator=g) if B * Hq * T * T <= 2_000_000 else None
    dq, dk, dv = attn.attn_materialized_bwd(x["q"], x["k"], x["v"], o, p, x["dout"], scale=scale,
                                            dp=None if dpx is None else dpx.to(dev))
    torch.cuda.synchronize()
    if dpx is None:
        rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"], scale)
    else:
        rdq, rdk, rdv = mat.backward(host["q"], host["k"], host["v"], host["dout"], dpx, scale)
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))
