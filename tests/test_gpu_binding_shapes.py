"""The binding refuses caller-provided outputs of the wrong shape before anything is
launched (the C ABI receives only their pointers and writes as many elements as the
inputs imply, so a short buffer would be written past its end), and refuses K, V whose
batch, length or head width disagree with Q (they would be read past their end).  Every
refusal is a ValueError and leaves the buffers untouched."""
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import announce, require_gpu

pytestmark = pytest.mark.gpu


def _refused(fn, *untouched):
    before = [t.clone() for t in untouched]
    with pytest.raises(ValueError):
        fn()
    torch.cuda.synchronize()
    for a, b in zip(untouched, before):
        assert torch.equal(a, b)


def test_wrong_output_shapes_are_refused():
    dev = require_gpu()
    announce("binding: wrong output shapes")
    c = {k: v.to(dev) for k, v in si.causal_inputs(2, 4, 2, 100, 32, seed=5).items()}
    q, k, v, do = c["q"], c["k"], c["v"], c["dout"]
    short = torch.full((2, 4, 99, 32), 7.0, device=dev)
    lse_short = torch.full((2, 4, 99), 7.0, device=dev)
    _refused(lambda: attn.attn_causal_fwd(q, k, v, o=short), short)
    _refused(lambda: attn.attn_causal_fwd(q, k, v, lse=lse_short), lse_short)
    _refused(lambda: attn.attn_causal_fwd(q, k[:, :, :99].contiguous(), v[:, :, :99].contiguous()))
    o, lse = attn.attn_causal_fwd(q, k, v)
    dk_short = torch.full((2, 2, 99, 32), 7.0, device=dev)
    _refused(lambda: attn.attn_causal_bwd(q, k, v, o, lse, do, dq=short), short)
    _refused(lambda: attn.attn_causal_bwd(q, k, v, o, lse, do, dk=dk_short), dk_short)
    _refused(lambda: attn.attn_causal_bwd(q, k, v, o, lse, do, dv=dk_short), dk_short)
    p_short = torch.full((2, 4, 100, 99), 7.0, device=dev)
    _refused(lambda: attn.attn_materialized_fwd(q, k, v, p=p_short), p_short)
    _refused(lambda: attn.attn_materialized_fwd(q, k, v, o=short), short)
    _, _, p = attn.attn_materialized_fwd(q, k, v)
    _refused(lambda: attn.attn_materialized_bwd(q, k, v, o, p, do, dq=short), short)
    _refused(lambda: attn.attn_materialized_bwd(q, k, v, o[:, :, :99].contiguous(), p, do))

    d = si.paged_decode_inputs(S=5, Hq=8, Hkv=2, D=64, page_size=16, ctx_lo=1, ctx_hi=300, max_pages=20, seed=6)
    x = {k_: (t.to(dev) if isinstance(t, torch.Tensor) else t) for k_, t in d.items()}
    args = (x["q"], x["k_pool"], x["v_pool"], x["block_table"], x["context_lens"])
    o_short = torch.full((5, 8, 63), 7.0, device=dev)
    l_short = torch.full((5, 7), 7.0, device=dev)
    o_ok = torch.full((5, 8, 64), 7.0, device=dev)
    _refused(lambda: attn.attn_paged_decode(*args, o=o_short), o_short)
    _refused(lambda: attn.attn_paged_decode(*args, lse=l_short), l_short)
    _refused(lambda: attn.PreparedPagedDecode(*args, o=o_short), o_short)
    _refused(lambda: attn.attn_paged_decode_noalloc(*args, o_short), o_short)
    _refused(lambda: attn.attn_paged_decode_noalloc(*args, o_ok, l_short), o_ok, l_short)

    pf = si.paged_prefill_inputs(S=2, Hq=8, Hkv=2, D=64, page_size=16, cached_lo=0, cached_hi=50, new_lo=1, new_hi=40,
                                 max_pages=8, seed=7)
    y = {k_: (t.to(dev) if isinstance(t, torch.Tensor) else t) for k_, t in pf.items()}
    pargs = (y["q"], y["k_pool"], y["v_pool"], y["block_table"], y["context_lens"], y["token_start"])
    po_short = torch.full((pf["N"] - 1, 8, 64), 7.0, device=dev)
    pl_short = torch.full((pf["N"], 7), 7.0, device=dev)
    _refused(lambda: attn.attn_paged_prefill(*pargs, o=po_short), po_short)
    _refused(lambda: attn.attn_paged_prefill(*pargs, lse=pl_short), pl_short)
