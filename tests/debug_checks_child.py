"""Child process of tests/test_gpu_debug_checks.py, run with ATTN_DEBUG_CHECKS=1 (the
library reads it once per process).  Prints one line per case and exits non-zero on
the first mismatch."""
import math
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import causal_self_attention_amd as attn  # noqa: E402
import synthetic_inputs as si  # noqa: E402
from oracle import oracle  # noqa: E402

assert os.environ.get("ATTN_DEBUG_CHECKS") == "1"
dev = torch.device("cuda:0")


def rel(a, b):
    import numpy as np
    a = a.detach().double().cpu().numpy()
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def expect_refusal(label, fn, fragments, untouched):
    before = [t.clone() for t in untouched]
    try:
        fn()
    except attn.AttnError as e:
        torch.cuda.synchronize()
        assert e.status == attn.ATTN_INVALID_ARGUMENT, (label, e)
        for f in fragments:
            assert f in e.message, (label, e.message)
        for a, b in zip(untouched, before):
            assert torch.equal(a, b), (label, "an output changed although nothing may be launched")
        print(f"{label}: refused: {e.message}", flush=True)
        return
    raise AssertionError(f"{label}: not refused")


# decode: a valid call passes the check and matches the oracle
h = si.paged_decode_inputs(S=9, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=500, max_pages=40, seed=81)
d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in h.items()}
o, lse = attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
torch.cuda.synchronize()
ro, _ = oracle.paged_decode(h["q"], h["k_pool"], h["v_pool"], h["block_table"], h["context_lens"])
assert rel(o, ro) <= 1e-5
print("decode: valid call checked and correct", flush=True)

o_s = torch.full_like(d["q"], 7.0)
l_s = torch.full((9, 16), 7.0, device=dev)
n_pages = h["num_pages"]
# a table entry in use outside the pool (sequence 3, its logical page 2 exists: length >= 33)
bt = d["block_table"].clone()
d["context_lens"][3] = max(int(d["context_lens"][3]), 40)
bt[3, 2] = n_pages + 5
expect_refusal("decode bad page", lambda: attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], bt,
                                                                  d["context_lens"], o=o_s, lse=l_s),
               ["block_table[3, 2]", str(n_pages + 5)], [o_s, l_s])
bt2 = d["block_table"].clone()
bt2[5, 0] = -1
expect_refusal("decode negative page", lambda: attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], bt2,
                                                                       d["context_lens"], o=o_s, lse=l_s),
               ["block_table[5, 0]", "-1"], [o_s, l_s])
# lengths: 0 and past the table's capacity
for s_bad, val in ((0, 0), (7, 40 * 16 + 1)):
    ctx = d["context_lens"].clone()
    ctx[s_bad] = val
    expect_refusal(f"decode length {val}", lambda: attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"],
                                                                           d["block_table"], ctx, o=o_s, lse=l_s),
                   [f"context_lens[{s_bad}] = {val}"], [o_s, l_s])
# the no-allocation variant checks too
expect_refusal("noalloc bad page", lambda: attn.attn_paged_decode_noalloc(d["q"], d["k_pool"], d["v_pool"], bt,
                                                                          d["context_lens"], o_s, l_s),
               ["block_table[3, 2]"], [o_s, l_s])
# an entry past the sequence's pages is not read, so it may hold anything
bt3 = d["block_table"].clone()
s0 = 2
npg = math.ceil(int(d["context_lens"][s0]) / 16)
bt3[s0, npg:] = 10 ** 6
o3, _ = attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], bt3, d["context_lens"])
o4, _ = attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
torch.cuda.synchronize()
assert torch.equal(o3, o4)
print("decode: entries past a sequence's pages are not checked (never read)", flush=True)

# prefill: broken ragged offsets and a bad page
p = si.paged_prefill_inputs(S=3, Hq=8, Hkv=2, D=64, page_size=16, cached_lo=0, cached_hi=90, new_lo=1, new_hi=80,
                            max_pages=12, seed=10)
x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
op, _ = attn.attn_paged_prefill(*(x[k] for k in ("q", "k_pool", "v_pool", "block_table", "context_lens",
                                                 "token_start")))
torch.cuda.synchronize()
rop, _ = oracle.paged_prefill(p["q"], p["k_pool"], p["v_pool"], p["block_table"], p["context_lens"],
                              p["token_start"])
assert rel(op, rop) <= 1e-4
print("prefill: valid call checked and correct", flush=True)
o_p = torch.full_like(x["q"], 7.0)
ts = x["token_start"].clone()
ts[3] += 1  # the last offset is not N
expect_refusal("prefill offsets", lambda: attn.attn_paged_prefill(x["q"], x["k_pool"], x["v_pool"],
                                                                   x["block_table"], x["context_lens"], ts, o=o_p,
                                                                   with_lse=False),
               ["token_start", "sequence 2"], [o_p])
btp = x["block_table"].clone()
btp[1, 0] = 10 ** 6
expect_refusal("prefill bad page", lambda: attn.attn_paged_prefill(x["q"], x["k_pool"], x["v_pool"], btp,
                                                                    x["context_lens"], x["token_start"], o=o_p,
                                                                    with_lse=False),
               ["block_table[1, 0]"], [o_p])
ctxp = x["context_lens"].clone()
ctxp[0] = int(x["token_start"][1]) - 1  # fewer cached positions than new tokens
expect_refusal("prefill short length", lambda: attn.attn_paged_prefill(x["q"], x["k_pool"], x["v_pool"],
                                                                        x["block_table"], ctxp, x["token_start"],
                                                                        o=o_p, with_lse=False),
               ["context_lens[0]"], [o_p])
print("ALL DEBUG CHECKS OK", flush=True)
