#!/usr/bin/env python3
"""Benchmark of the causal attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  causal forward + backward on the 1024-token workload (B=4, H=8, T=1024,
  d=64, fp32), then one batched paged decode (32 sequences, Hq=16, Hkv=4,
  d=64, 16-token pages, context lengths uniform in [512, 4096]).
All inputs are generated once and already resident in HBM when timing starts.
Before the warm-up steps, `--settle-steps` untimed steps (150 by default, ~30 ms) let
the chip's clock finish its climb under load (from idle it rises from about 2.06 to
2.18 GHz over the first ~20 ms); `settle_steps` in the line records how many ran.

Printed: one JSON line.  `value` is the causal forward+backward rate in
algorithmic TFLOP/s (14*d per unmasked query-key pair: QK^T and PV forward;
QK^T recompute, dV, dP, dK, dQ backward) over the event time from before the
forward to after the backward (the two calls issued back to back); separate
breakdown steps with an event between the calls give the per-call times (means,
medians and minima; `frac_by_medians` is the fraction from median(fwd) +
median(bwd)); `back_to_back_us` times the same pairs issued back to back between two
events, with no marker between the calls, as a training loop issues them.  The
decode rate is the algorithmic HBM bytes per call over the average time of
back-to-back decode calls between two events (the step's decode call, event to
event, is reported beside it); `decode_sweep` adds the same shape with one
16-position group per sequence (the fixed cost of a call), a 256-sequence batch,
and the workload's rate beyond that fixed cost.  The 8192-token grouped-query forward and backward, the materialized path, a batched
paged prefill of a ragged 8-sequence batch and the latency of a K/V append (the
step before decode) are reported beside it, and so are the 16- and 256-token
workloads' forward and backward times.  Each decode call reads a different one of
several pool replicas so the 256 MB last-level cache cannot serve a repeated pool.

`roofline` describes the dominant kernel (the backward: its delta/zero-fill
pass plus the main KV-parallel kernel, launched together by attn_causal_bwd),
measured with HIP events on the launch stream.  `cpu_baseline` is the CPU
oracle (plain double-precision materialised attention) timed on this host on
the full 1024-token forward+backward; `cpu_oracle_beside` times it on the
other workloads (the 8192-token forward once, the others as the median of 3)
with the same algorithmic counts.
"""
import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s (fp32, % MFMA peak); paged-decode HBM GB/s"
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
# HBM bytes per attn_causal_bwd launch on the 1024-token workload, from FETCH_SIZE (x2.00)
# and WRITE_SIZE (x1.00) counter passes; valid only for the kernel source they were taken on.
BWD_TRAFFIC_BYTES = 166.0e6
BWD_TRAFFIC_SOURCE_SHA256_PREFIX = "4898045732492846"
CAUSAL = "mha_b4_h8_t1024_d64"
SMALL = ("mha_b1_h2_t16_d8", "mha_b8_h4_t256_d32")
GQA = "gqa_b1_hq16_hkv4_t8192_d64"
DECODE = "paged_decode_s32_hq16_hkv4_d64_p16"
PREFILL = "paged_prefill_s8_hq16_hkv4_d64_p16"


def causal_flops(B, Hq, T, D):
    pairs = B * Hq * T * (T + 1) // 2
    return 4 * D * pairs, 10 * D * pairs


def decode_bytes(d, Hq, Hkv, D):
    ctx = [int(c) for c in d["context_lens"]]
    S = len(ctx)
    pages = sum(math.ceil(c / d["page_size"]) for c in ctx)
    kv = sum(ctx) * Hkv * D * 4 * 2          # every K and V row once per KV head
    qo = 2 * S * Hq * D * 4                  # q in, o out
    return kv + qo + S * Hq * 4 + pages * 4 + S * 4  # + lse, used table entries, lengths


def bwd_traffic():
    """Counter-measured bytes per backward launch, or None if the kernel source changed."""
    import hashlib
    path = os.path.join(ROOT, "causal_self_attention_amd", "csrc", "attn_bwd.hip")
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return BWD_TRAFFIC_BYTES if digest.startswith(BWD_TRAFFIC_SOURCE_SHA256_PREFIX) else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-steps", type=int, default=150,
                    help="untimed steps before the warm-up ones, while the chip's clock rises under load")
    ap.add_argument("--decode-replicas", type=int, default=4)
    ap.add_argument("--gqa-iters", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only fill, sum and copy a buffer of this many MiB (plain kernels of known "
                         "traffic, to scale hardware byte counters) and exit")
    ap.add_argument("--only", choices=["all", "bwd", "gqa", "decode", "prefill"], default="all",
                    help="'bwd': run only the timed steps of forward + backward; 'gqa': only the 8192-token "
                         "grouped-query forward and backward, --gqa-iters times each; 'decode': only --steps "
                         "decode calls on the pool replicas; 'prefill': only --steps prefill calls (for counter "
                         "passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU (got --gpus {args.gpus}); "
              "sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_self_attention_amd as attn
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    if args.calibrate_copy_mb:
        # known traffic: the fill writes n*4 bytes, each sum reads n*4 bytes, each copy
        # reads and writes n*4 bytes
        n = args.calibrate_copy_mb * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        tot = torch.empty((), device=dev)
        for _ in range(3):
            torch.sum(src, dim=(0,), out=tot)
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_bytes": n * 4, "fill": 1, "sum": 3, "copy": 3}), flush=True)
        return

    if args.only == "gqa":
        gcfg = si.CAUSAL_WORKLOADS[GQA]
        gh = si.causal_inputs(gcfg["B"], gcfg["Hq"], gcfg["Hkv"], gcfg["T"], gcfg["D"], gcfg["seed"], with_do=True)
        gx = {k: v.to(dev) for k, v in gh.items()}
        go = torch.empty_like(gx["q"])
        glse = torch.empty((gcfg["B"], gcfg["Hq"], gcfg["T"]), device=dev)
        gdq, gdk, gdv = torch.empty_like(gx["q"]), torch.empty_like(gx["k"]), torch.empty_like(gx["v"])
        gws = torch.empty((attn.attn_causal_bwd_workspace_bytes(gcfg["B"], gcfg["Hq"], gcfg["Hkv"], gcfg["T"],
                                                                gcfg["D"]) // 4,), device=dev)
        for _ in range(args.gqa_iters):
            attn.attn_causal_fwd(gx["q"], gx["k"], gx["v"], o=go, lse=glse, stream=stream)
            attn.attn_causal_bwd(gx["q"], gx["k"], gx["v"], go, glse, gx["dout"], dq=gdq, dk=gdk, dv=gdv,
                                 workspace=gws, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"only": "gqa", "iters": args.gqa_iters}), flush=True)
        return

    if args.only == "prefill":
        ph = si.prefill_workload(PREFILL)
        pdev = {k: ph[k].to(dev) for k in ("q", "k_pool", "v_pool", "block_table", "context_lens", "token_start")}
        po = torch.empty_like(pdev["q"])
        plse = torch.empty((ph["N"], si.PREFILL_WORKLOADS[PREFILL]["Hq"]), device=dev)
        for _ in range(args.steps):
            attn.attn_paged_prefill(pdev["q"], pdev["k_pool"], pdev["v_pool"], pdev["block_table"],
                                    pdev["context_lens"], pdev["token_start"], o=po, lse=plse, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"only": "prefill", "calls": args.steps}), flush=True)
        return

    # ---- inputs and outputs, resident before timing ----
    cfg = si.CAUSAL_WORKLOADS[CAUSAL]
    B, Hq, Hkv, T, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["D"]
    host = si.causal_workload(CAUSAL)
    x = {k: v.to(dev) for k, v in host.items()}
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, Hq, T), device=dev)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    ws = torch.empty((attn.attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D) // 4,), device=dev)
    fwd_flops, bwd_flops = causal_flops(B, Hq, T, D)

    dcfg = si.DECODE_WORKLOADS[DECODE]
    dh = si.decode_workload(DECODE)
    dq_ = dh["q"].to(dev)
    bt = dh["block_table"].to(dev)
    ctx = dh["context_lens"].to(dev)
    pools = []
    for r in range(max(1, args.decode_replicas)):
        pools.append((dh["k_pool"].to(dev), dh["v_pool"].to(dev)))
    do_ = torch.empty_like(dq_)
    dlse = torch.empty((dcfg["S"], dcfg["Hq"]), device=dev)
    dws = torch.empty((attn.attn_paged_decode_workspace_bytes(dcfg["S"], dcfg["Hq"], dcfg["Hkv"], dcfg["D"],
                                                              dcfg["page_size"], dcfg["max_pages"]) // 4,),
                      device=dev)
    dbytes = decode_bytes(dh, dcfg["Hq"], dcfg["Hkv"], dcfg["D"])
    torch.cuda.synchronize()
    if args.only == "decode":
        plans = [attn.PreparedPagedDecode(dq_, kp, vp, bt, ctx, o=do_, lse=dlse, workspace=dws, stream=stream)
                 for kp, vp in pools]
        for i in range(args.steps):
            plans[i % len(plans)]()
        torch.cuda.synchronize()
        print(json.dumps({"only": "decode", "calls": args.steps, "bytes_per_call": dbytes}), flush=True)
        return

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        attn.attn_causal_fwd(x["q"], x["k"], x["v"], o=o, lse=lse, stream=stream)
        if ev is not None and len(ev) == 4:  # breakdown: an event between the two calls
            ev[1].record(stream)
        attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], dq=dq, dk=dk, dv=dv, workspace=ws,
                             stream=stream)
        if ev is not None:
            ev[-2].record(stream)
        if args.only == "all":
            kp, vp = pools[i % len(pools)]
            attn.attn_paged_decode(dq_, kp, vp, bt, ctx, o=do_, lse=dlse, workspace=dws, stream=stream)
        if ev is not None:
            ev[-1].record(stream)

    # Clock settle: from idle (any pause of 0.2 s or more) the chip's core clock climbs from
    # about 2.06 to 2.18 GHz over the first ~20 ms of this load, and a forward + backward pair
    # from about 185 to 163 us; these untimed steps run before the warm-up ones so that the
    # timed steps measure the settled state rather than the climb.
    for i in range(args.settle_steps):
        step(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed steps: one event before the forward, one after the backward (the pass itself,
    # back to back as a training step issues it), one after the decode
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.only == "bwd":
        print(json.dumps({"only": "bwd", "steps": args.steps}), flush=True)
        return
    t_fb = [e[0].elapsed_time(e[1]) for e in evs]
    t_dec = [e[1].elapsed_time(e[2]) for e in evs]
    t_step = [e[0].elapsed_time(e[2]) for e in evs]
    K = args.steps

    # breakdown steps (after the timed ones): an event between the forward and the
    # backward too, for the per-kernel times and the backward's roofline
    nb = max(10, K // 2)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    for i in range(nb):
        step(K + i, bev[i])
    torch.cuda.synchronize()
    t_fwd = [e[0].elapsed_time(e[1]) for e in bev]
    t_bwd = [e[1].elapsed_time(e[2]) for e in bev]
    sum_fwd, sum_bwd = sum(t_fwd), sum(t_bwd)

    # the same pass back to back: K forward + backward pairs between two events, with no
    # marker between the calls (as a training loop issues them); reported beside `value`
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(K):
        attn.attn_causal_fwd(x["q"], x["k"], x["v"], o=o, lse=lse, stream=stream)
        attn.attn_causal_bwd(x["q"], x["k"], x["v"], o, lse, x["dout"], dq=dq, dk=dk, dv=dv, workspace=ws,
                             stream=stream)
    b1.record(stream)
    torch.cuda.synchronize()
    fb_b2b_s = b0.elapsed_time(b1) / K * 1e-3

    # headline: fwd+bwd algorithmic TFLOP/s over the event time of the two calls
    value = (fwd_flops + bwd_flops) * K / (sum(t_fb) * 1e-3) / 1e12
    bwd_avg_s = sum_bwd / nb * 1e-3
    bwd_tflops = bwd_flops / bwd_avg_s / 1e12
    fwd_avg_s = sum_fwd / nb * 1e-3
    # decode on its own: back-to-back calls between two events (each on the next pool
    # replica), so that no event marker sits between the calls; the in-step time above
    # (event after the backward to event after the decode) is reported beside it
    # (prepared calls: the arguments are checked once, so that Python's per-call checks
    # do not starve the device of work between two 30 us calls)
    nd = max(20, 2 * K) if args.only == "all" else 0
    if nd:
        plans = [attn.PreparedPagedDecode(dq_, kp, vp, bt, ctx, o=do_, lse=dlse, workspace=dws, stream=stream)
                 for kp, vp in pools]
        for plan in plans:
            plan()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(nd):
            plans[i % len(plans)]()
        d1.record(stream)
        torch.cuda.synchronize()
        dec_avg_s = d0.elapsed_time(d1) / nd * 1e-3
    else:
        dec_avg_s = sum(t_dec) / K * 1e-3
    dec_step_s = sum(t_dec) / K * 1e-3
    dec_gbps = dbytes / dec_avg_s / 1e9

    # the 8192-token grouped-query forward (O + LSE), timed separately, then its
    # backward (dO drawn after Q, K, V with the same generator)
    gcfg = si.CAUSAL_WORKLOADS[GQA]
    gh = si.causal_inputs(gcfg["B"], gcfg["Hq"], gcfg["Hkv"], gcfg["T"], gcfg["D"], gcfg["seed"], with_do=True)
    gx = {k: v.to(dev) for k, v in gh.items()}
    go = torch.empty_like(gx["q"])
    glse = torch.empty((gcfg["B"], gcfg["Hq"], gcfg["T"]), device=dev)
    attn.attn_causal_fwd(gx["q"], gx["k"], gx["v"], o=go, lse=glse, stream=stream)
    torch.cuda.synchronize()
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.gqa_iters)]
    for a, b in gev:
        a.record(stream)
        attn.attn_causal_fwd(gx["q"], gx["k"], gx["v"], o=go, lse=glse, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    g_ms = statistics.median(a.elapsed_time(b) for a, b in gev)
    g_flops, g_bflops = causal_flops(gcfg["B"], gcfg["Hq"], gcfg["T"], gcfg["D"])
    gdq, gdk, gdv = torch.empty_like(gx["q"]), torch.empty_like(gx["k"]), torch.empty_like(gx["v"])
    gws = torch.empty((attn.attn_causal_bwd_workspace_bytes(gcfg["B"], gcfg["Hq"], gcfg["Hkv"], gcfg["T"],
                                                            gcfg["D"]) // 4,), device=dev)
    attn.attn_causal_bwd(gx["q"], gx["k"], gx["v"], go, glse, gx["dout"], dq=gdq, dk=gdk, dv=gdv, workspace=gws,
                         stream=stream)
    torch.cuda.synchronize()
    for a, b in gev:
        a.record(stream)
        attn.attn_causal_bwd(gx["q"], gx["k"], gx["v"], go, glse, gx["dout"], dq=gdq, dk=gdk, dv=gdv,
                             workspace=gws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    gb_ms = statistics.median(a.elapsed_time(b) for a, b in gev)
    del gx, go, glse, gdq, gdk, gdv, gws

    # the materialized path on the 1024-token workload: O, LSE and P [B,H,T,T] forward,
    # the VJP from the stored P
    mp = torch.empty((B, Hq, T, T), device=dev)
    mdq, mdk, mdv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    mev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(10)]
    for it in range(12):
        ev = mev[it - 2] if it >= 2 else None
        if ev:
            ev[0].record(stream)
        attn.attn_materialized_fwd(x["q"], x["k"], x["v"], o=o, lse=lse, p=mp, stream=stream)
        if ev:
            ev[1].record(stream)
        attn.attn_materialized_bwd(x["q"], x["k"], x["v"], o, mp, x["dout"], dq=mdq, dk=mdk, dv=mdv, workspace=ws,
                                   stream=stream)
        if ev:
            ev[2].record(stream)
    torch.cuda.synchronize()
    m_fwd_us = statistics.median(e[0].elapsed_time(e[1]) for e in mev) * 1e3
    m_bwd_us = statistics.median(e[1].elapsed_time(e[2]) for e in mev) * 1e3
    p_bytes = B * Hq * T * T * 4
    del mp, mdq, mdk, mdv

    # decode cost structure: the workload's shape with one 16-position group per sequence
    # (what a call costs besides streaming K/V) and a 256-sequence batch with the
    # workload's length distribution, each timed back to back like the decode above
    def decode_back_to_back(d, reps, calls=20):
        q2, bt2, ctx2 = d["q"].to(dev), d["block_table"].to(dev), d["context_lens"].to(dev)
        pools2 = [(d["k_pool"].to(dev), d["v_pool"].to(dev)) for _ in range(reps)]
        o2 = torch.empty_like(q2)
        l2 = torch.empty(q2.shape[:2], device=dev)
        ws2 = torch.empty((attn.attn_paged_decode_workspace_bytes(q2.shape[0], dcfg["Hq"], dcfg["Hkv"], dcfg["D"],
                                                                  dcfg["page_size"], bt2.shape[1]) // 4,),
                          device=dev)
        plans2 = [attn.PreparedPagedDecode(q2, kp2, vp2, bt2, ctx2, o=o2, lse=l2, workspace=ws2, stream=stream)
                  for kp2, vp2 in pools2]
        for i in range(3):
            plans2[i % reps]()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(calls):
            plans2[i % reps]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls * 1e3, decode_bytes(d, dcfg["Hq"], dcfg["Hkv"], dcfg["D"])

    sweep = {}
    if args.only == "all":
        d_one = si.paged_decode_inputs(dcfg["S"], dcfg["Hq"], dcfg["Hkv"], dcfg["D"], dcfg["page_size"], 16, 16,
                                       dcfg["max_pages"], dcfg["seed"])
        one_us, one_bytes = decode_back_to_back(d_one, 1)
        d_256 = si.paged_decode_inputs(256, dcfg["Hq"], dcfg["Hkv"], dcfg["D"], dcfg["page_size"], dcfg["ctx_lo"],
                                       dcfg["ctx_hi"], dcfg["max_pages"], dcfg["seed"])
        big_us, big_bytes = decode_back_to_back(d_256, 1)
        del d_one, d_256
        sweep = {
            "one_group_per_sequence": {"S": dcfg["S"], "us": round(one_us, 2), "bytes_per_call": one_bytes},
            "s256": {"us": round(big_us, 2), "bytes_per_call": big_bytes, "gbps": round(big_bytes / big_us / 1e3, 1),
                     "frac_of_hbm_peak": round(big_bytes / big_us / 1e3 / PEAK_HBM_GBPS, 4)},
            "workload_beyond_fixed_gbps": round((dbytes - one_bytes) / (dec_avg_s * 1e6 - one_us) / 1e3, 1),
        }

    # the step before decode: lease + append one token's K/V for every sequence of the
    # decode workload's shape, into an empty cache (pages leased every 16th call)
    S_, Hkv_, D_, ps_ = dcfg["S"], dcfg["Hkv"], dcfg["D"], dcfg["page_size"]
    n_app = 64
    cache = attn.PagedKvCache(S_, Hkv_, D_, ps_, n_app // ps_ + 1, S_ * (n_app // ps_ + 1), dev)
    g_ = torch.Generator("cpu").manual_seed(6)
    kn = torch.randn((S_, Hkv_, D_), generator=g_).to(dev)
    vn = torch.randn((S_, Hkv_, D_), generator=g_).to(dev)
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_app)]
    torch.cuda.synchronize()
    for a, b in aev:
        a.record(stream)
        attn.attn_kv_append(kn, vn, cache, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    if cache.status() != attn.ATTN_KV_OK:
        raise RuntimeError("kv append refused during the bench")
    app_us = statistics.median(a.elapsed_time(b) for a, b in aev) * 1e3
    app_bytes = 2 * 2 * S_ * Hkv_ * D_ * 4  # new K and V rows read once and written once

    # batched prefill over the paged cache: the ragged 8-sequence workload (new tokens
    # already in the cache), O + LSE; 4*d flops per (new token, visible position, head)
    pcfg = si.PREFILL_WORKLOADS[PREFILL]
    ph = si.prefill_workload(PREFILL)
    pdev = {k: ph[k].to(dev) for k in ("q", "k_pool", "v_pool", "block_table", "context_lens", "token_start")}
    po = torch.empty_like(pdev["q"])
    plse = torch.empty((ph["N"], pcfg["Hq"]), device=dev)
    pts, pctx = ph["token_start"].tolist(), ph["context_lens"].tolist()
    p_pairs = 0
    for s_ in range(pcfg["S"]):
        n_ = pts[s_ + 1] - pts[s_]
        c_ = pctx[s_]
        p_pairs += sum(c_ - n_ + j + 1 for j in range(n_))
    p_flops = 4 * pcfg["D"] * pcfg["Hq"] * p_pairs
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(12)]
    torch.cuda.synchronize()
    for a, b in pev:
        a.record(stream)
        attn.attn_paged_prefill(pdev["q"], pdev["k_pool"], pdev["v_pool"], pdev["block_table"],
                                pdev["context_lens"], pdev["token_start"], o=po, lse=plse, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    pre_us = statistics.median(a.elapsed_time(b) for a, b in pev[2:]) * 1e3
    del pdev, po, plse

    # the 16- and 256-token workloads (parity cases, timed too): median over 20 calls of
    # the forward and of the backward, events around each call (the 16-token one is a
    # few microseconds of launches)
    small = {}
    for sname in SMALL:
        sc = si.CAUSAL_WORKLOADS[sname]
        sx = {k: v.to(dev) for k, v in si.causal_workload(sname).items()}
        s_o = torch.empty_like(sx["q"])
        s_l = torch.empty((sc["B"], sc["Hq"], sc["T"]), device=dev)
        s_dq, s_dk, s_dv = torch.empty_like(sx["q"]), torch.empty_like(sx["k"]), torch.empty_like(sx["v"])
        s_ws = torch.empty((max(attn.attn_causal_bwd_workspace_bytes(sc["B"], sc["Hq"], sc["Hkv"], sc["T"], sc["D"]),
                                256) // 4,), device=dev)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(20)]
        torch.cuda.synchronize()
        for it in range(25):
            ev = sev[it - 5] if it >= 5 else None
            if ev:
                ev[0].record(stream)
            attn.attn_causal_fwd(sx["q"], sx["k"], sx["v"], o=s_o, lse=s_l, stream=stream)
            if ev:
                ev[1].record(stream)
            attn.attn_causal_bwd(sx["q"], sx["k"], sx["v"], s_o, s_l, sx["dout"], dq=s_dq, dk=s_dk, dv=s_dv,
                                 workspace=s_ws, stream=stream)
            if ev:
                ev[2].record(stream)
        torch.cuda.synchronize()
        f_us = statistics.median(e[0].elapsed_time(e[1]) for e in sev) * 1e3
        b_us = statistics.median(e[1].elapsed_time(e[2]) for e in sev) * 1e3
        sf, sb = causal_flops(sc["B"], sc["Hq"], sc["T"], sc["D"])
        small[sname] = {"fwd_us_median": round(f_us, 2), "bwd_us_median": round(b_us, 2),
                        "fwd_bwd_us": round(f_us + b_us, 2), "flops": sf + sb,
                        "fwd_bwd_tflops": round((sf + sb) / ((f_us + b_us) * 1e-6) / 1e12, 4),
                        "frac_of_fp32_mfma_peak": round((sf + sb) / ((f_us + b_us) * 1e-6) / 1e12
                                                        / PEAK_FP32_MFMA_TFLOPS, 5)}
        del sx, s_o, s_l, s_dq, s_dk, s_dv, s_ws

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": args.settle_steps,
        "ms_per_step": round(sum(t_step) / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{CAUSAL} causal fwd+bwd + {DECODE} paged decode (one step)",
            "causal": {"B": B, "Hq": Hq, "Hkv": Hkv, "T": T, "D": D, "scale": 1 / math.sqrt(D)},
            "decode": {k: dcfg[k] for k in ("S", "Hq", "Hkv", "D", "page_size", "ctx_lo", "ctx_hi", "max_pages")},
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "attn_causal_bwd (attn_bwd_pre + attn_bwd_main)",
            "bound": "mfma",
            "achieved": round(bwd_tflops, 3),
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(bwd_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
            "traffic": bwd_traffic(),
            "flops_per_launch": bwd_flops,
            "avg_launch_us": round(bwd_avg_s * 1e6, 2),
        },
        "fwd_bwd": {
            "us": round(sum(t_fb) / K * 1e3, 2), "us_median": round(statistics.median(t_fb) * 1e3, 2),
            "breakdown_steps": nb, "fwd_us": round(fwd_avg_s * 1e6, 2), "bwd_us": round(bwd_avg_s * 1e6, 2),
            "fwd_tflops": round(fwd_flops / fwd_avg_s / 1e12, 3), "bwd_tflops": round(bwd_tflops, 3),
            "fwd_bwd_tflops": round(value, 3), "frac_of_fp32_mfma_peak": round(value / PEAK_FP32_MFMA_TFLOPS, 4),
            "fwd_us_median": round(statistics.median(t_fwd) * 1e3, 2),
            "bwd_us_median": round(statistics.median(t_bwd) * 1e3, 2),
            "us_min": round(min(t_fb) * 1e3, 2), "fwd_us_min": round(min(t_fwd) * 1e3, 2),
            "bwd_us_min": round(min(t_bwd) * 1e3, 2),
            "back_to_back_us": round(fb_b2b_s * 1e6, 2),
            "back_to_back_frac": round((fwd_flops + bwd_flops) / fb_b2b_s / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
            # the same fraction from median(fwd) + median(bwd) of the breakdown steps
            "frac_by_medians": round((fwd_flops + bwd_flops) / ((statistics.median(t_fwd) + statistics.median(t_bwd))
                                                                * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
        },
        "decode": {
            "us": round(dec_avg_s * 1e6, 2), "calls_back_to_back": nd,
            "us_in_step": round(dec_step_s * 1e6, 2), "us_in_step_median": round(statistics.median(t_dec) * 1e3, 2),
            "bytes_per_call": dbytes, "gbps": round(dec_gbps, 1),
            "frac_of_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4), "pool_replicas": len(pools),
        },
        "gqa_t8192_fwd": {
            "ms_median": round(g_ms, 4), "tflops": round(g_flops / (g_ms * 1e-3) / 1e12, 3),
            "frac_of_fp32_mfma_peak": round(g_flops / (g_ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
        },
        "gqa_t8192_fwd_bwd": {
            "fwd_ms_median": round(g_ms, 4), "bwd_ms_median": round(gb_ms, 4),
            "bwd_tflops": round(g_bflops / (gb_ms * 1e-3) / 1e12, 3),
            "tflops": round((g_flops + g_bflops) / ((g_ms + gb_ms) * 1e-3) / 1e12, 3),
            "frac_of_fp32_mfma_peak": round((g_flops + g_bflops) / ((g_ms + gb_ms) * 1e-3) / 1e12
                                            / PEAK_FP32_MFMA_TFLOPS, 4),
        },
        "materialized": {
            "workload": CAUSAL, "fwd_us_median": round(m_fwd_us, 2), "bwd_us_median": round(m_bwd_us, 2),
            "p_bytes": p_bytes, "fwd_p_store_gbps": round(p_bytes / (m_fwd_us * 1e-6) / 1e9, 1),
            "bwd_tflops": round(bwd_flops / (m_bwd_us * 1e-6) / 1e12, 3),
        },
        "decode_sweep": sweep,
        "small_workloads": small,
        "paged_prefill": {
            "workload": PREFILL, "new_tokens": ph["N"], "us_median": round(pre_us, 2), "flops": p_flops,
            "tflops": round(p_flops / (pre_us * 1e-6) / 1e12, 3),
            "frac_of_fp32_mfma_peak": round(p_flops / (pre_us * 1e-6) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
        },
        "kv_append": {
            "us_median": round(app_us, 2), "bytes_per_call": app_bytes,
            "gbps": round(app_bytes / (app_us * 1e-6) / 1e9, 2), "calls": n_app,
            "note": "lease + append of one token for 32 sequences; one launch (the lease work-group copies the rows), latency bound",
        },
        "wall_s_timed_region": round(wall, 4),
    }

    if not args.no_cpu_baseline:
        from oracle import oracle as oracle_mod
        orc = oracle_mod.default()
        runs = []
        for _ in range(max(1, args.cpu_runs)):
            t = time.perf_counter()
            orc.causal_fwd(host["q"], host["k"], host["v"])
            orc.causal_bwd(host["q"], host["k"], host["v"], host["dout"])
            runs.append(time.perf_counter() - t)
        cpu_s = statistics.median(runs)
        line["cpu_baseline"] = {
            "value": round((fwd_flops + bwd_flops) / cpu_s / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"full {CAUSAL} forward+backward (materialised, double), median of {len(runs)} runs, "
                      f"{cpu_s:.2f} s each; host {cpu_model()}",
        }

        # the oracle beside the other workloads, same algorithmic counts as the GPU lines:
        # the small ones and the decode one warm-up and the median of 3, the 8192-token
        # forward one run
        def med3(fn):
            fn()
            ts_ = []
            for _ in range(3):
                t = time.perf_counter()
                fn()
                ts_.append(time.perf_counter() - t)
            return statistics.median(ts_)

        beside = {"cores": orc.num_threads(), "host": cpu_model()}
        for sname in SMALL:
            hs = si.causal_workload(sname)
            sc = si.CAUSAL_WORKLOADS[sname]
            t_s = med3(lambda: (orc.causal_fwd(hs["q"], hs["k"], hs["v"]),
                                orc.causal_bwd(hs["q"], hs["k"], hs["v"], hs["dout"])))
            sf, sb = causal_flops(sc["B"], sc["Hq"], sc["T"], sc["D"])
            beside[sname] = {"fwd_bwd_s": round(t_s, 6), "gflops": round((sf + sb) / t_s / 1e9, 3),
                             "runs": "1 warm-up + median of 3"}
        gcfg = si.CAUSAL_WORKLOADS[GQA]
        gh4 = si.causal_inputs(gcfg["B"], gcfg["Hq"], gcfg["Hkv"], gcfg["T"], gcfg["D"], gcfg["seed"],
                               with_do=False)
        t = time.perf_counter()
        orc.causal_fwd(gh4["q"], gh4["k"], gh4["v"])
        t4 = time.perf_counter() - t
        beside[GQA] = {"fwd_s": round(t4, 3), "gflops": round(g_flops / t4 / 1e9, 3), "runs": "1 run",
                       "gpu_speedup": round(t4 / (g_ms * 1e-3), 1)}
        t5 = med3(lambda: orc.paged_decode(dh["q"], dh["k_pool"], dh["v_pool"], dh["block_table"],
                                           dh["context_lens"]))
        beside[DECODE] = {"s": round(t5, 4), "gbps": round(dbytes / t5 / 1e9, 3), "runs": "1 warm-up + median of 3",
                          "gpu_speedup": round(t5 / dec_avg_s, 1)}
        line["cpu_oracle_beside"] = beside
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
