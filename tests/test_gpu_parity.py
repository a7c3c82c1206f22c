"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Tolerances (max-abs error relative to the reference's largest magnitude):
O and LSE 1e-4, dQ/dK/dV 1e-3, paged decode vs dense decode 1e-5.

Every named workload is compared element by element on whole tensors, the
8192-token grouped-query forward included (the oracle takes tens of seconds
there); its rows are also checked against the oracle's single-query decode over
the row's causal prefix, a second route through the definition.
"""
import math

import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_DECODE, TOL_GRAD, TOL_LSE, TOL_O, announce, rel_err, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _to(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _run_fwd(x, scale=None):
    o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _run_bwd(x, o, lse, scale=None):
    dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


# ---------------------------------------------------------------------------
# the named causal workloads
# ---------------------------------------------------------------------------
FULL_WORKLOADS = ["mha_b1_h2_t16_d8", "mha_b8_h4_t256_d32", "mha_b4_h8_t1024_d64"]


@pytest.mark.parametrize("name", FULL_WORKLOADS)
def test_workload_forward_backward(dev, orc, name):
    announce(f"fwd+bwd workload {name}")
    host = si.causal_workload(name)
    x = _to(host, dev)
    D = host["q"].shape[-1]
    scale = 1.0 / math.sqrt(D)
    o, lse = _run_fwd(x, scale)
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"], scale)
    assert rel_err(o, ro) <= TOL_O, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_LSE, ("LSE", rel_err(lse, rlse))
    dq, dk, dv = _run_bwd(x, o, lse, scale)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"], scale)
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


SAMPLE_ROWS = [0, 1, 15, 16, 63, 64, 65, 127, 128, 1000, 4095, 4096, 8127, 8128, 8190, 8191]


def test_gqa_t8192_forward_whole(dev, gqa_t8192_reference, orc):
    """Whole O [1,16,8192,64] and LSE [1,16,8192] against the oracle's causal forward,
    and sampled rows against its single-query decode over the row's prefix."""
    ref = gqa_t8192_reference
    host = ref["host"]
    announce("fwd workload gqa_b1_hq16_hkv4_t8192_d64 (whole tensors)")
    x = _to(host, dev)
    o, lse = _run_fwd(x, ref["scale"])
    o_h, lse_h = o.cpu(), lse.cpu()
    assert rel_err(o_h, ref["o"]) <= TOL_O, ("O", rel_err(o_h, ref["o"]))
    assert rel_err(lse_h, ref["lse"]) <= TOL_LSE, ("LSE", rel_err(lse_h, ref["lse"]))
    rng = np.random.default_rng(4)
    rows = sorted(set(SAMPLE_ROWS) | set(int(r) for r in rng.integers(0, 8192, 8)))
    q, k, v = host["q"][0], host["k"][0], host["v"][0]  # [H, T, D]
    for i in rows:
        ro, rlse = orc.decode_dense(q[:, i, :], k[:, : i + 1, :].transpose(0, 1), v[:, : i + 1, :].transpose(0, 1),
                                    ref["scale"])
        assert rel_err(o_h[0, :, i, :], ro) <= TOL_O, ("O row", i, rel_err(o_h[0, :, i, :], ro))
        assert rel_err(lse_h[0, :, i], rlse) <= TOL_LSE, ("LSE row", i)


# ---------------------------------------------------------------------------
# edge shapes: ragged tiles, every head width, grouped heads
# ---------------------------------------------------------------------------
EDGE_CASES = [(1, 2, 2, T, D) for D in (8, 16, 32, 64, 128) for T in (1, 17, 65, 129)]
EDGE_CASES += [(2, 3, 3, 2, 64), (1, 1, 1, 15, 32), (1, 2, 1, 63, 64), (2, 4, 2, 200, 64),
               (1, 4, 1, 100, 64), (1, 8, 1, 77, 32), (1, 8, 2, 130, 16), (1, 16, 2, 96, 128),
               (2, 4, 2, 777, 128)]  # d = 128: the forward's four key parts over 13 tiles


@pytest.mark.parametrize("B,Hq,Hkv,T,D", EDGE_CASES)
def test_edge_shapes(dev, orc, B, Hq, Hkv, T, D):
    announce(f"edge fwd+bwd B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=1000 + T * 7 + D + Hq)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"])
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))
    dq, dk, dv = _run_bwd(x, o, lse)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


def test_gqa_backward_long_context(dev, orc):
    """Grouped heads (G = 4) through the backward at T = 1024."""
    announce("gqa fwd+bwd B=1 Hq=16 Hkv=4 T=1024 D=64")
    host = si.causal_inputs(1, 16, 4, 1024, 64, seed=44)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    ro, _ = orc.causal_fwd(host["q"], host["k"], host["v"])
    assert rel_err(o, ro) <= TOL_O
    dq, dk, dv = _run_bwd(x, o, lse)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


def _check_fwd_bwd(dev, orc, B, Hq, Hkv, T, D, seed):
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=seed)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    ro, rlse = orc.causal_fwd(host["q"], host["k"], host["v"])
    assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, (rel_err(o, ro), rel_err(lse, rlse))
    dq, dk, dv = _run_bwd(x, o, lse)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 32), (8, 4, 64)])
def test_backward_whole_key_block_schedule(dev, orc, Hq, Hkv, D):
    """More key blocks than two per CU: one work-group per whole key block."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    T = 600  # 10 key blocks, the last one ragged
    B = (2 * cus + 10 * Hkv) // (10 * Hkv) + 1
    assert B * Hkv * 10 > 2 * cus
    announce(f"bwd whole-key-block schedule B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    _check_fwd_bwd(dev, orc, B, Hq, Hkv, T, D, seed=300 + D)


def _bwd_schedule(cus, B, Hq, Hkv, T, D):
    """Which cut of the backward's work the library takes for this shape on `cus` CUs:
    one whole key block per work-group, half pairs of key blocks, or finer runs (as
    many as the chip holds work-groups, at most 512, at least two steps each)."""
    nkb, nbkv = (T + 63) // 64, B * Hkv
    if nkb * nbkv > 2 * cus:
        return "whole"
    fine = min((1 if D >= 128 else 2) * cus // nbkv, 512 // nbkv, Hq // Hkv * nkb * (nkb + 1) // 2 // 2)
    return "fine" if fine > nkb else "half"


@pytest.mark.parametrize("nbkv,Hkv,G,D", [(32, 8, 1, 64), (39, 13, 1, 32), (16, 8, 1, 128), (22, 2, 3, 16)])
def test_backward_half_pair_schedule(dev, orc, nbkv, Hkv, G, D):
    """Key blocks that just fill the chip: half pairs of key blocks per work-group, odd and
    even counts of blocks, the last one ragged."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    B = nbkv // Hkv
    nkb = (1 if D >= 128 else 2) * cus // nbkv
    T = 64 * nkb - 23
    assert _bwd_schedule(cus, B, G * Hkv, Hkv, T, D) == "half"
    announce(f"bwd half-pair schedule B={B} Hq={G * Hkv} Hkv={Hkv} T={T} D={D}")
    _check_fwd_bwd(dev, orc, B, G * Hkv, Hkv, T, D, seed=400 + T)


@pytest.mark.parametrize("B,Hq,Hkv,T,D", [(1, 8, 2, 777, 32), (1, 1, 1, 1088, 64), (3, 6, 3, 960, 16),
                                          (1, 8, 1, 512, 64), (2, 8, 2, 1000, 128)])
def test_backward_fine_schedule(dev, orc, B, Hq, Hkv, T, D):
    """Few batch x KV heads: the step list cut into as many runs as the chip holds, so a key
    block is shared by many runs (up to 32 at B=1, Hkv=1, T=512), whose pieces are summed in
    run order: parity, and bitwise equal dK, dV on a second call."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert _bwd_schedule(cus, B, Hq, Hkv, T, D) == "fine"
    announce(f"bwd fine schedule B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=450 + T + D)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    dq, dk, dv = _run_bwd(x, o, lse)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))
    _, dk2, dv2 = _run_bwd(x, o, lse)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("B,Hq,Hkv,T,D,cut", [(3, 6, 6, 2025, 16, "whole"), (1, 2, 1, 2100, 64, "fine"),
                                              (2, 8, 4, 4073, 16, "half")])
def test_backward_descending_query_order(dev, orc, B, Hq, Hkv, T, D, cut):
    """From 32 key blocks per sequence on, the backward takes a key block's query tiles in
    descending order: parity under each of the three cuts of the work (the last tile
    ragged), and bitwise equal dK, dV on a second call."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert (T + 63) // 64 >= 32 and _bwd_schedule(cus, B, Hq, Hkv, T, D) == cut
    announce(f"bwd descending query order ({cut} cut) B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    host = si.causal_inputs(B, Hq, Hkv, T, D, seed=470 + T + D)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    dq, dk, dv = _run_bwd(x, o, lse)
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    for nm, a, b in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD, (nm, rel_err(a, b))
    _, dk2, dv2 = _run_bwd(x, o, lse)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


# ---------------------------------------------------------------------------
# invariants and closed forms on the GPU outputs
# ---------------------------------------------------------------------------
def test_single_position_is_exact(dev):
    announce("T=1 closed form")
    host = si.causal_inputs(2, 4, 2, 1, 64, seed=7)
    x = _to(host, dev)
    o, lse = _run_fwd(x, 0.3)
    assert torch.equal(o.cpu(), host["v"].repeat_interleave(2, dim=1)), "T=1: O must equal V exactly"
    want = 0.3 * (host["q"][:, :, 0].double() * host["k"].repeat_interleave(2, dim=1)[:, :, 0].double()).sum(-1)
    assert rel_err(lse[:, :, 0], want) <= TOL_LSE
    dq, dk, dv = _run_bwd(x, o, lse, 0.3)
    # P = 1, so dS = dP - Delta is rounding noise only
    assert float(dq.abs().max()) < 1e-4 and float(dk.abs().max()) < 1e-4
    want_dv = host["dout"].reshape(2, 2, 2, 1, 64).sum(2)
    assert rel_err(dv, want_dv) <= 1e-5


def test_zero_scale_is_prefix_mean(dev):
    announce("scale=0 prefix mean")
    host = si.causal_inputs(1, 2, 2, 150, 32, seed=8)
    x = _to(host, dev)
    o, lse = _run_fwd(x, 0.0)
    cnt = torch.arange(1, 151, dtype=torch.float64)
    want = torch.cumsum(host["v"].double(), dim=2) / cnt[None, None, :, None]
    assert rel_err(o, want) <= TOL_O
    assert rel_err(lse, torch.log(cnt).expand(1, 2, 150)) <= TOL_LSE
    dq, dk, dv = _run_bwd(x, o, lse, 0.0)
    assert float(dq.abs().max()) == 0.0 and float(dk.abs().max()) == 0.0


def test_causality_is_bitwise(dev):
    """Changing keys/values at positions >= s leaves rows < s unchanged, bit for bit."""
    announce("causality")
    host = si.causal_inputs(1, 4, 2, 300, 64, seed=9)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    for s in (5, 64, 100, 257):
        y = dict(x)
        k2, v2 = x["k"].clone(), x["v"].clone()
        k2[:, :, s:] += 2.5
        v2[:, :, s:] *= -3.0
        y["k"], y["v"] = k2, v2
        o2, lse2 = _run_fwd(y)
        assert torch.equal(o2[:, :, :s], o[:, :, :s]), ("O", s)
        assert torch.equal(lse2[:, :, :s], lse[:, :, :s]), ("LSE", s)
        # NaN keys in the future are masked by selection, not arithmetic
        k3 = x["k"].clone()
        k3[:, :, s:] = float("nan")
        y["k"], y["v"] = k3, x["v"]
        o3, lse3 = _run_fwd(y)
        assert torch.equal(o3[:, :, :s], o[:, :, :s]), ("NaN K", s)


def test_gradient_sums(dev):
    """Each dS row sums to zero, so sum_j dK_j = 0; sum_j dV_j = sum_i dO_i per group."""
    announce("gradient sums")
    host = si.causal_inputs(2, 4, 2, 190, 32, seed=10)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    dq, dk, dv = _run_bwd(x, o, lse)
    dk_sum = dk.double().sum(2)
    assert float(dk_sum.abs().max()) <= 1e-3 * float(dk.abs().max()) * math.sqrt(190)
    want = host["dout"].double().sum(2).reshape(2, 2, 2, 32).sum(2)
    assert rel_err(dv.double().sum(2), want) <= 1e-4


def test_forward_is_deterministic(dev):
    announce("forward determinism")
    host = si.causal_inputs(2, 8, 2, 333, 64, seed=11)
    x = _to(host, dev)
    o1, l1 = _run_fwd(x)
    o2, l2 = _run_fwd(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    dq1, dk1, dv1 = _run_bwd(x, o1, l1)
    dq2, dk2, dv2 = _run_bwd(x, o1, l1)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)  # dQ uses float atomics
    assert rel_err(dq1, dq2) <= 1e-6


def test_outputs_fully_overwritten(dev, orc):
    """Outputs (including dQ) do not depend on what the buffers held before."""
    announce("outputs overwritten")
    host = si.causal_inputs(1, 2, 2, 70, 16, seed=12)
    x = _to(host, dev)
    o = torch.full_like(x["q"], float("nan"))
    lse = torch.full((1, 2, 70), float("nan"), device=dev)
    attn.attn_causal_fwd(x["q"], x["k"], x["v"], o=o, lse=lse)
    dq = torch.full_like(x["q"], 7.0)
    dk = torch.full_like(x["k"], float("nan"))
    dv = torch.full_like(x["v"], float("nan"))
    ws = torch.full((attn.attn_causal_bwd_workspace_bytes(1, 2, 2, 70, 16) // 4,), float("nan"), device=dev)
    attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    ro, _ = orc.causal_fwd(host["q"], host["k"], host["v"])
    rdq, rdk, rdv = orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
    assert rel_err(o, ro) <= TOL_O
    for a, b in ((dq, rdq), (dk, rdk), (dv, rdv)):
        assert rel_err(a, b) <= TOL_GRAD


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------
def _decode(d, dev, scale=None, **kw):
    o, lse = attn.attn_paged_decode(d["q"].to(dev), d["k_pool"].to(dev), d["v_pool"].to(dev),
                                    d["block_table"].to(dev), d["context_lens"].to(dev), scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def _contiguous_layout(d):
    """Same sequences, pages laid out in logical order with identity-like tables."""
    bt, ctx, ps = d["block_table"], d["context_lens"], d["page_size"]
    S = bt.shape[0]
    pages, rows = [], torch.full_like(bt, 0)
    off = 0
    for s in range(S):
        n = math.ceil(int(ctx[s]) / ps)
        pages.append(bt[s, :n].long())
        rows[s, :n] = torch.arange(off, off + n, dtype=torch.int32)
        off += n
    idx = torch.cat(pages + [torch.tensor([d["poison_page"]])])
    for s in range(S):
        n = math.ceil(int(ctx[s]) / ps)
        rows[s, n:] = off  # padding -> the copied poison page
    out = dict(d)
    out["k_pool"] = d["k_pool"][idx].contiguous()
    out["v_pool"] = d["v_pool"][idx].contiguous()
    out["block_table"] = rows
    return out


def test_decode_workload(dev, orc):
    name = next(iter(si.DECODE_WORKLOADS))
    announce(f"decode workload {name}")
    d = si.decode_workload(name)
    o, lse = _decode(d, dev)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE, ("LSE", rel_err(lse, rlse))
    # the same kernel on a contiguous copy of the gathered sequences: identical bits
    c = _contiguous_layout(d)
    o2, lse2 = _decode(c, dev)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_decode_poisoned_tail_and_padding(dev):
    """NaN in pool slots past each context and in the padding page changes nothing."""
    announce("decode poison")
    d = si.paged_decode_inputs(S=9, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=700, max_pages=48, seed=21)
    o, lse = _decode(d, dev)
    kp, vp = d["k_pool"].clone(), d["v_pool"].clone()
    kp[d["poison_page"]] = float("nan")
    vp[d["poison_page"]] = float("nan")
    for s in range(9):
        n = int(d["context_lens"][s])
        last = int(d["block_table"][s, (n - 1) // 16])
        kp[last, :, (n - 1) % 16 + 1:] = float("nan")
        vp[last, :, (n - 1) % 16 + 1:] = float("nan")
    p = dict(d)
    p["k_pool"], p["v_pool"] = kp, vp
    o2, lse2 = _decode(p, dev)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_decode_pool_permutation(dev):
    announce("decode pool permutation")
    d = si.paged_decode_inputs(S=6, Hq=8, Hkv=2, D=32, page_size=16, ctx_lo=100, ctx_hi=900, max_pages=64, seed=22)
    o, lse = _decode(d, dev)
    perm = torch.randperm(d["num_pages"], generator=torch.Generator().manual_seed(23))
    p = dict(d)
    kp = torch.empty_like(d["k_pool"])
    vp = torch.empty_like(d["v_pool"])
    kp[perm] = d["k_pool"]
    vp[perm] = d["v_pool"]
    p["k_pool"], p["v_pool"] = kp, vp
    p["block_table"] = perm[d["block_table"].long()].to(torch.int32)
    o2, lse2 = _decode(p, dev)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


DECODE_CASES = [(D, G, ps) for D in (8, 16, 32, 64, 128) for G in (1, 4) for ps in (16, 64)]
DECODE_CASES += [(64, 8, 16), (32, 2, 32), (16, 8, 32)]
# more than 8 query heads per KV head: the MFMA split kernel (8 or fewer: the VALU one)
DECODE_CASES += [(64, 16, 16), (32, 12, 32), (128, 16, 64), (8, 16, 16), (16, 3, 16), (128, 6, 32)]


DECODE_SPLIT_MAX_S = 1024  # the split path's partition holds up to this many sequences


def _decode_batch(dev, path, Hkv):
    """Sequences per batch that select the split (at most 1024 sequences) or the
    fused (more) decode path."""
    return 5 if path == "split" else DECODE_SPLIT_MAX_S + 1


@pytest.mark.parametrize("path", ["split", "fused"])
@pytest.mark.parametrize("D,G,ps", DECODE_CASES)
def test_decode_shapes(dev, orc, D, G, ps, path):
    Hkv = 2
    S = _decode_batch(dev, path, Hkv)
    announce(f"decode {path} S={S} D={D} G={G} page={ps}")
    hi = 520 if path == "split" else 160  # the fused batch is 205 times larger
    d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1, ctx_hi=hi,
                               max_pages=math.ceil(520 / ps) + 1, seed=100 + D + G + ps)
    d["context_lens"][1] = 520  # several 64-group passes of the split path's waves
    d["context_lens"][0] = 1  # a single cached position
    o, lse = _decode(d, dev)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE
    # one position: the output is that position's value row
    g_of = torch.arange(Hkv * G) // G
    assert torch.equal(o[0].cpu(), d["v_pool"][int(d["block_table"][0, 0]), g_of, 0, :])
    # without lse
    o3, lse3 = _decode(d, dev, with_lse=False)
    assert lse3 is None and torch.equal(o3, o)


@pytest.mark.parametrize("path", ["split", "fused"])
def test_decode_long_context(dev, orc, path):
    """A context longer than one pass of the fused waves (8 waves x 64 groups x 16)."""
    Hkv, G, D, ps = 2, 4, 64, 64
    S = _decode_batch(dev, path, Hkv)
    announce(f"decode long context {path} S={S}")
    d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1,
                               ctx_hi=9000 if path == "split" else 200, max_pages=math.ceil(9000 / ps), seed=77)
    d["context_lens"][0] = 9000
    d["context_lens"][1] = 8193
    o, lse = _decode(d, dev)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE


def test_decode_split_many_sequences(dev, orc):
    """More sequences than one wave's lanes on the split path (the partition's prefix
    sums carry across 64-sequence chunks), with empty-looking short ones mixed in."""
    Hkv, G, D, ps = 1, 4, 64, 16
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    S = min(200, cus - 1)
    announce(f"decode split S={S}")
    d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1, ctx_hi=300,
                               max_pages=math.ceil(300 / ps), seed=91)
    d["context_lens"][::7] = 1
    o, lse = _decode(d, dev)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE


@pytest.mark.parametrize("path,G", [("split", 4), ("split", 1), ("split", 8), ("fused", 4)])
def test_decode_large_negative_logits(dev, orc, path, G):
    """Every score of every head far below -1e30 (scale 1e32, q.k < 0): softmax is
    still defined (one-hot on each head's largest score), so O is that key's value
    row and LSE that score, on every decode path (the VALU split kernel for G <= 4,
    the MFMA one above, the fused one for more than 1024 sequences)."""
    Hkv, D, ps = 2, 64, 16
    S = _decode_batch(dev, path, Hkv)
    announce(f"decode large negative logits {path} S={S} G={G}")
    d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1,
                               ctx_hi=300 if path == "split" else 40, max_pages=math.ceil(300 / ps), seed=130 + G)
    d["q"] = -d["q"].abs()
    kp = d["k_pool"].abs() + 0.01
    # one position per sequence gets a key a quarter as long, so its score is the
    # largest by a wide margin for every query head (fp32 and fp64 then agree on
    # the argmax whatever the rounding of the dot products)
    for s in range(S):
        n = int(d["context_lens"][s])
        t = (7919 * s) % n
        kp[int(d["block_table"][s, t // ps]), :, t % ps] *= 0.25
    d["k_pool"] = kp
    scale = 1e32
    for s in range(S):
        n = int(d["context_lens"][s])
        if n < 2:
            continue
        pos = torch.arange(n)
        rows = d["block_table"][s, pos // ps].long()
        kk = kp[rows, :, pos % ps].double()  # [n, Hkv, D]
        sc = torch.einsum("nhd,hgd->nhg", kk, d["q"][s].double().reshape(Hkv, G, D)).reshape(n, -1)
        top = torch.topk(sc, 2, dim=0).values
        assert float((top[0] - top[1]).min()) > 1e-3 * float(sc.abs().max()), s
    o, lse = _decode(d, dev, scale=scale)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], scale)
    assert float(np.max(rlse)) < -1e30
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE, ("LSE", rel_err(lse, rlse))


def test_prepared_decode_reissues_the_same_call(dev):
    """PreparedPagedDecode checks and marshals once; each call re-issues attn_paged_decode
    on the same tensors, so new contents written into them between calls are picked up,
    and every result equals the plain call's bit for bit."""
    announce("prepared decode")
    d = si.paged_decode_inputs(S=12, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=900, max_pages=64, seed=24)
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    plan = attn.PreparedPagedDecode(x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"])
    for i in range(3):
        if i:
            x["q"].mul_(-0.5).add_(0.25)  # new contents, same storage
            x["context_lens"].sub_(1).clamp_(min=1)
        o, lse = plan()
        want_o, want_lse = attn.attn_paged_decode(x["q"], x["k_pool"], x["v_pool"], x["block_table"],
                                                  x["context_lens"])
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_lse), i


def test_decode_shared_workspace(dev, orc):
    """Calls of different sizes sharing one workspace that starts out as NaN: its
    contents on entry do not matter, and each call's partials and slot records
    overwrite whatever an earlier, larger or smaller, call left there."""
    Hkv, G, D, ps, maxp = 4, 4, 64, 16, 64
    nb = attn.attn_paged_decode_workspace_bytes(40, Hkv * G, Hkv, D, ps, maxp)
    ws = torch.full((nb // 4,), float("nan"), device=dev)
    for i, S in enumerate((40, 7, 33, 1, 40, 2)):
        announce(f"decode shared workspace call {i} S={S}")
        d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1, ctx_hi=1000,
                                   max_pages=maxp, seed=900 + i)
        o, lse = _decode(d, dev, workspace=ws)
        ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
        assert rel_err(o, ro) <= TOL_DECODE, (S, rel_err(o, ro))
        assert rel_err(lse, rlse) <= TOL_DECODE


def test_decode_matches_causal_last_row(dev):
    """Decode over a contiguous sequence equals the causal forward's last row."""
    announce("decode vs causal last row")
    T, D, Hq, Hkv = 300, 64, 8, 2
    host = si.causal_inputs(1, Hq, Hkv, T, D, seed=31, with_do=False)
    x = _to(host, dev)
    o, lse = _run_fwd(x)
    ps = 16
    npg = math.ceil(T / ps)
    kp = torch.zeros(npg, Hkv, ps, D)
    vp = torch.zeros(npg, Hkv, ps, D)
    for t in range(T):
        kp[t // ps, :, t % ps] = host["k"][0, :, t]
        vp[t // ps, :, t % ps] = host["v"][0, :, t]
    d = {"q": host["q"][0, :, T - 1].unsqueeze(0).contiguous(), "k_pool": kp, "v_pool": vp,
         "block_table": torch.arange(npg, dtype=torch.int32).unsqueeze(0),
         "context_lens": torch.tensor([T], dtype=torch.int32)}
    od, lsed = _decode(d, dev)
    assert rel_err(od[0], o[0, :, T - 1]) <= TOL_O
    assert rel_err(lsed[0], lse[0, :, T - 1]) <= TOL_LSE


@pytest.mark.parametrize("S,Hkv,G,ctx_hi", [(1, 4, 4, 9000), (3, 8, 2, 3000), (7, 3, 5, 1500), (150, 1, 16, 200),
                                            (700, 1, 4, 120), (1024, 2, 4, 64), (1024, 8, 1, 40)])
def test_decode_split_layouts(dev, orc, S, Hkv, G, ctx_hi):
    """Split-path layouts: one long sequence (its groups spread over the whole grid),
    two columns of KV heads (Hkv = 8), a partial column (Hkv = 3), many short
    sequences over one KV head (several 64-sequence chunks of the partition), and
    up to the largest batch the split path takes (1024 sequences: more sequences than
    work-groups, so a work-group holds partials of several sequences)."""
    D, ps = 64, 16
    announce(f"decode split layout S={S} Hkv={Hkv} G={G}")
    d = si.paged_decode_inputs(S=S, Hq=Hkv * G, Hkv=Hkv, D=D, page_size=ps, ctx_lo=1, ctx_hi=ctx_hi,
                               max_pages=math.ceil(ctx_hi / ps), seed=500 + S + Hkv)
    o, lse = _decode(d, dev)
    ro, rlse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
    assert rel_err(o, ro) <= TOL_DECODE, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_DECODE
