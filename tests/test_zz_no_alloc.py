"""The no-allocation paged decode (attn_paged_decode_noalloc), called through the C
ABI, against attn_paged_decode with a caller workspace: the same kernels, so the
same bits, on two calls in a row (the second smaller, so it reuses what the first
left in the static scratch), each also within the decode tolerance of the oracle.
A batch whose partials exceed the scratch is refused with a clear message.  After
the first call on the device (its once-per-device set-up looks up the scratch's
address, which places the static array on the device), no call changes the
device's free memory."""
import ctypes
import math

import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_DECODE, announce, rel_err, require_gpu

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _noalloc(d, o, lse, scale, stream):
    S, Hq, D = d["q"].shape
    num_pages, Hkv, ps, _ = d["k_pool"].shape
    return attn.lib().attn_paged_decode_noalloc(
        _ptr(d["q"]), _ptr(d["k_pool"]), _ptr(d["v_pool"]), _ptr(d["block_table"]), _ptr(d["context_lens"]), S, Hq,
        Hkv, D, ps, d["block_table"].shape[1], num_pages, ctypes.c_float(scale), _ptr(o), _ptr(lse),
        ctypes.c_void_p(stream.cuda_stream))


def _to(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_noalloc_decode_matches_workspace_decode(orc):
    dev = require_gpu()
    stream = torch.cuda.current_stream(dev)
    name = next(iter(si.DECODE_WORKLOADS))
    cases = [("workload", si.decode_workload(name)),
             ("smaller", si.paged_decode_inputs(S=5, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=700,
                                                max_pages=48, seed=71))]
    set_up = False
    for label, host in cases:
        announce(f"noalloc decode {label} S={host['q'].shape[0]}")
        d = _to(host, dev)
        S, Hq, D = d["q"].shape
        scale = 1.0 / math.sqrt(D)
        want_o, want_lse = attn.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                                  d["context_lens"], scale=scale)
        o = torch.full_like(d["q"], float("nan"))
        lse = torch.full((S, Hq), float("nan"), device=dev)
        torch.cuda.synchronize()
        if not set_up:  # the first call on the device: its set-up
            assert _noalloc(d, o, lse, scale, stream) == attn.ATTN_OK, attn.attn_last_error()
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            set_up = True
        # read right before the call: torch's own kernels load their code lazily on
        # first use, and its allocator takes new segments, which also take device memory
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info(dev)[0]
        st = _noalloc(d, o, lse, scale, stream)
        assert st == attn.ATTN_OK, attn.attn_last_error()
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info(dev)[0] == free_before, "the call changed the device's free memory"
        assert torch.equal(o, want_o) and torch.equal(lse, want_lse), label
        ro, rlse = orc.paged_decode(host["q"], host["k_pool"], host["v_pool"], host["block_table"],
                                    host["context_lens"], scale)
        assert rel_err(o, ro) <= TOL_DECODE, (label, rel_err(o, ro))
        assert rel_err(lse, rlse) <= TOL_DECODE, (label, rel_err(lse, rlse))
        # without lse
        o2 = torch.full_like(d["q"], float("nan"))
        assert _noalloc(d, o2, None, scale, stream) == attn.ATTN_OK, attn.attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o2, want_o), label


def test_noalloc_decode_refuses_batches_beyond_the_scratch():
    """1024 sequences of 128 query heads at d = 128 need far more than the static
    scratch: refused before anything is launched (the buffers are real and valid,
    so nothing could go wrong even if it were launched)."""
    dev = require_gpu()
    announce("noalloc decode over-size refusal")
    S, Hq, Hkv, D, ps = 1024, 128, 8, 128, 16
    d = {"q": torch.zeros((S, Hq, D), device=dev), "k_pool": torch.zeros((1, Hkv, ps, D), device=dev),
         "v_pool": torch.zeros((1, Hkv, ps, D), device=dev),
         "block_table": torch.zeros((S, 1), device=dev, dtype=torch.int32),
         "context_lens": torch.ones((S,), device=dev, dtype=torch.int32)}
    o = torch.zeros_like(d["q"])
    st = _noalloc(d, o, None, 0.1, torch.cuda.current_stream(dev))
    assert st == attn.ATTN_WORKSPACE_TOO_SMALL, (st, attn.attn_last_error())
    msg = attn.attn_last_error()
    assert "scratch" in msg and str(attn.ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES) in msg, msg
    # the binding's wrapper raises with the same message
    with pytest.raises(attn.AttnError):
        attn.attn_paged_decode_noalloc(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], o)
    # more than 1024 sequences take the fused path, which needs no scratch
    S2 = 1025
    e = {"q": torch.randn((S2, 8, 64), device=dev), "k_pool": torch.randn((S2, 2, 16, 64), device=dev),
         "v_pool": torch.randn((S2, 2, 16, 64), device=dev),
         "block_table": torch.arange(S2, device=dev, dtype=torch.int32).reshape(S2, 1),
         "context_lens": torch.full((S2,), 16, device=dev, dtype=torch.int32)}
    o2 = torch.empty_like(e["q"])
    assert _noalloc(e, o2, None, 0.125, torch.cuda.current_stream(dev)) == attn.ATTN_OK, attn.attn_last_error()
    want, _ = attn.attn_paged_decode(e["q"], e["k_pool"], e["v_pool"], e["block_table"], e["context_lens"],
                                     scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o2, want)
