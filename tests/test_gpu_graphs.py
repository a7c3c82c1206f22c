"""The calls under HIP graph capture (torch.cuda.graph): every call is asynchronous on
the caller's stream and, given its outputs and workspaces, allocates and synchronizes
nothing, so a forward + backward, a paged decode through both entry points (the
no-allocation one holds its partial results in the library's static scratch) and a
batched prefill can be captured once and replayed.  The graph is replayed several times
with new input contents copied into its static inputs and eager work of the program's
own between the replays (other calls, on other buffers, and a synchronization); every
replay is checked against eager calls on the same inputs: the same bits for O, LSE, dK,
dV and the decode and prefill outputs, dQ (float atomics) within 1e-6 of its largest
magnitude."""

import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import announce, rel_err, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed):
    c = si.causal_inputs(2, 4, 2, 300, 64, seed=seed)
    d = si.paged_decode_inputs(S=9, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=700, max_pages=48, seed=seed)
    p = si.paged_prefill_inputs(S=3, Hq=8, Hkv=2, D=64, page_size=16, cached_lo=0, cached_hi=200, new_lo=1,
                                new_hi=100, max_pages=20, seed=seed)
    return c, d, p


def test_graph_capture_and_replay():
    dev = require_gpu()
    announce("graph capture of fwd+bwd, decode (both entries), prefill")
    c0, d0, p0 = _inputs(500)
    C = {k: v.to(dev) for k, v in c0.items()}
    Dd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d0.items()}
    Pp = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p0.items()}
    B, Hq, T, D = C["q"].shape
    Hkv = C["k"].shape[1]
    o, lse = torch.empty_like(C["q"]), torch.empty((B, Hq, T), device=dev)
    dq, dk, dv = torch.empty_like(C["q"]), torch.empty_like(C["k"]), torch.empty_like(C["v"])
    bws = torch.empty((max(attn.attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D), 256) // 4,), device=dev)
    S, dHq, dD = Dd["q"].shape
    dws = torch.empty((attn.attn_paged_decode_workspace_bytes(S, dHq, Dd["k_pool"].shape[1], dD, 16,
                                                              Dd["block_table"].shape[1]) // 4,), device=dev)
    do_, dl_ = torch.empty_like(Dd["q"]), torch.empty((S, dHq), device=dev)
    na_o, na_l = torch.empty_like(Dd["q"]), torch.empty((S, dHq), device=dev)
    po, pl = torch.empty_like(Pp["q"]), torch.empty((Pp["q"].shape[0], Pp["q"].shape[1]), device=dev)

    def calls():
        attn.attn_causal_fwd(C["q"], C["k"], C["v"], o=o, lse=lse)
        attn.attn_causal_bwd(C["q"], C["k"], C["v"], o, lse, C["dout"], dq=dq, dk=dk, dv=dv, workspace=bws)
        attn.attn_paged_decode(Dd["q"], Dd["k_pool"], Dd["v_pool"], Dd["block_table"], Dd["context_lens"], o=do_,
                               lse=dl_, workspace=dws)
        attn.attn_paged_decode_noalloc(Dd["q"], Dd["k_pool"], Dd["v_pool"], Dd["block_table"], Dd["context_lens"],
                                       na_o, na_l)
        attn.attn_paged_prefill(Pp["q"], Pp["k_pool"], Pp["v_pool"], Pp["block_table"], Pp["context_lens"],
                                Pp["token_start"], o=po, lse=pl)

    def snapshot():
        return [t.clone() for t in (o, lse, dq, dk, dv, do_, dl_, na_o, na_l, po, pl)]

    # warm up on the capture's side stream (first calls set up the static scratch address)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    other = {k: v.to(dev) for k, v in si.causal_inputs(1, 2, 2, 200, 32, seed=9).items()}
    for rep, seed in enumerate((501, 502, 503, 501)):
        # new contents for the static inputs (same shapes, tables and lengths)
        c = si.causal_inputs(B, Hq, Hkv, T, D, seed=seed)
        for k in ("q", "k", "v", "dout"):
            C[k].copy_(c[k])
        gen = torch.Generator("cpu").manual_seed(seed)
        Dd["q"].copy_(torch.randn(tuple(Dd["q"].shape), generator=gen))
        Pp["q"].copy_(torch.randn(tuple(Pp["q"].shape), generator=gen))
        Dd["k_pool"].copy_(torch.randn(tuple(Dd["k_pool"].shape), generator=gen))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        # the program's own eager work between replays, on other buffers
        attn.attn_causal_fwd(other["q"], other["k"], other["v"])
        torch.cuda.synchronize()
        calls()  # eager, same inputs and outputs
        torch.cuda.synchronize()
        want = snapshot()
        names = ("O", "LSE", "dQ", "dK", "dV", "decode O", "decode LSE", "noalloc O", "noalloc LSE", "prefill O",
                 "prefill LSE")
        for nm, a, b in zip(names, got, want):
            if nm == "dQ":
                assert rel_err(a, b) <= 1e-6, (rep, nm, rel_err(a, b))
            else:
                assert torch.equal(a, b), (rep, nm)
        assert torch.isfinite(got[0]).all() and torch.isfinite(got[5]).all()
