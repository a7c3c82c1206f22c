"""Several host threads, each on its own HIP stream, calling the library at once.

The C boundary keeps its error text per thread and reads each device's compute-unit
count once; the kernels share no global state.  So concurrent calls on different
streams, with their own outputs and workspaces, must give what the same calls give
one at a time: bitwise for the forward, dK, dV and the decode, and within rounding
for dQ (its float atomics may add in another order).
"""
import threading

import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import announce, rel_err, require_gpu

pytestmark = pytest.mark.gpu


def test_threads_on_separate_streams():
    dev = require_gpu()
    announce("threads on separate streams")
    x = {k: v.to(dev) for k, v in si.causal_inputs(2, 4, 2, 300, 64, seed=61).items()}
    d = si.paged_decode_inputs(S=12, Hq=8, Hkv=2, D=64, page_size=16, ctx_lo=1, ctx_hi=900, max_pages=64, seed=62)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}

    def run(stream=None):
        o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], stream=stream)
        dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], stream=stream)
        od, ld = attn.attn_paged_decode(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"], dd["context_lens"],
                                        stream=stream)
        return o, lse, dq, dk, dv, od, ld

    ref = run()
    torch.cuda.synchronize()

    errors, results = [], {}

    def worker(tid):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                for _ in range(4):
                    out = run(stream=s)
            s.synchronize()
            results[tid] = out
        except Exception as e:  # reported below, in the test's own thread
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    assert len(results) == 3
    names = ("o", "lse", "dq", "dk", "dv", "decode o", "decode lse")
    for tid, out in results.items():
        for name, got, want in zip(names, out, ref):
            if name == "dq":
                assert rel_err(got, want) <= 1e-5, (tid, name, rel_err(got, want))
            else:
                assert torch.equal(got, want), (tid, name)


def test_non_current_stream_with_allocation_churn():
    """Calls on a stream that is not the current one, while the current stream keeps
    allocating and overwriting memory of the workspaces' sizes: the binding's outputs
    and workspaces belong to the call's stream, so the caching allocator cannot hand
    a workspace dropped on return to the current stream's work while the call's
    kernels still use it.  Every result equals the same call made on the current
    stream (bitwise; dQ within rounding)."""
    dev = require_gpu()
    announce("non-current stream with allocation churn on the current stream")
    x = {k: v.to(dev) for k, v in si.causal_inputs(4, 8, 2, 1024, 64, seed=63).items()}
    d = si.paged_decode_inputs(S=32, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=512, ctx_hi=4096, max_pages=256,
                               seed=64)
    dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}

    def run(stream=None):
        o, lse = attn.attn_causal_fwd(x["q"], x["k"], x["v"], stream=stream)
        dq, dk, dv = attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], stream=stream)
        od, ld = attn.attn_paged_decode(dd["q"], dd["k_pool"], dd["v_pool"], dd["block_table"], dd["context_lens"],
                                        stream=stream)
        return o, lse, dq, dk, dv, od, ld

    ref = run()
    torch.cuda.synchronize()
    sizes = [attn.attn_causal_bwd_workspace_bytes(4, 8, 2, 1024, 64),
             attn.attn_paged_decode_workspace_bytes(32, 16, 4, 64, 16, 256)]
    s = torch.cuda.Stream(device=dev)
    assert s != torch.cuda.current_stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    outs = []
    for _ in range(6):
        outs.append(run(stream=s))
        for nb in sizes * 3:  # the current stream reuses freed memory of these sizes at once
            junk = torch.empty((nb // 4,), device=dev)
            junk.fill_(float("nan"))
            del junk
    s.synchronize()
    torch.cuda.synchronize()
    names = ("o", "lse", "dq", "dk", "dv", "decode o", "decode lse")
    for i, out in enumerate(outs):
        for name, got, want in zip(names, out, ref):
            if name == "dq":
                assert rel_err(got, want) <= 1e-5, (i, name, rel_err(got, want))
            else:
                assert torch.equal(got, want), (i, name)
