"""Seeded synthetic inputs: determinism and the workloads' shapes/structure."""
import math

import torch

import synthetic_inputs as si


def test_causal_inputs_deterministic_and_shaped():
    for name, c in si.CAUSAL_WORKLOADS.items():
        if c["T"] > 1024:
            continue  # the 8192-token inputs are large; their shapes are checked below
        a = si.causal_workload(name)
        b = si.causal_workload(name)
        for key in a:
            assert torch.equal(a[key], b[key]), (name, key)
            assert a[key].dtype == torch.float32 and a[key].is_contiguous()
        assert a["q"].shape == (c["B"], c["Hq"], c["T"], c["D"])
        assert a["k"].shape == (c["B"], c["Hkv"], c["T"], c["D"])
        assert ("dout" in a) == c["backward"]


def test_dout_std_of_the_1024_token_workload():
    d = si.causal_workload("mha_b4_h8_t1024_d64")
    assert abs(float(d["dout"].std()) - 0.1) < 0.002
    assert abs(float(d["q"].std()) - 1.0) < 0.01


def test_gqa_workload_shapes():
    c = si.CAUSAL_WORKLOADS["gqa_b1_hq16_hkv4_t8192_d64"]
    assert c["Hq"] % c["Hkv"] == 0 and c["Hq"] // c["Hkv"] == 4 and not c["backward"]


def test_decode_inputs_structure():
    name = next(iter(si.DECODE_WORKLOADS))
    c = si.DECODE_WORKLOADS[name]
    d = si.decode_workload(name)
    d2 = si.decode_workload(name)
    for key in ("q", "k_pool", "v_pool", "block_table", "context_lens"):
        assert torch.equal(d[key], d2[key])
    ctx = d["context_lens"]
    assert ctx.dtype == torch.int32 and ctx.shape == (c["S"],)
    assert int(ctx.min()) >= c["ctx_lo"] and int(ctx.max()) <= c["ctx_hi"]
    n = [math.ceil(int(x) / c["page_size"]) for x in ctx]
    assert d["pages_used"] == sum(n) and d["num_pages"] == sum(n) + 1
    bt = d["block_table"]
    assert bt.shape == (c["S"], c["max_pages"]) and bt.dtype == torch.int32
    used = torch.cat([bt[s, : n[s]] for s in range(c["S"])])
    # every physical page except the padding page is used exactly once
    assert torch.equal(torch.sort(used).values, torch.arange(sum(n), dtype=torch.int32))
    for s in range(c["S"]):
        assert torch.all(bt[s, n[s]:] == d["poison_page"])
    assert d["k_pool"].shape == (sum(n) + 1, c["Hkv"], c["page_size"], c["D"])
