"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and builds index tables; it holds none of
the attention arithmetic, so both the CPU oracle and the HIP library can be fed
from it without sharing any of the method's code.

Every tensor is drawn on the CPU with ``torch.Generator('cpu').manual_seed(seed)``
in a fixed order, so the same seed always gives the same bytes.
"""
import math

import torch

# The five workloads, named by what they are.  Causal ones draw Q, K, V and then
# dO (if there is a backward pass) from N(0,1); dO of the 1024-token case has
# standard deviation 0.1.  The seed of each workload is fixed here.
CAUSAL_WORKLOADS = {
    "mha_b1_h2_t16_d8": dict(B=1, Hq=2, Hkv=2, T=16, D=8, do_std=1.0, backward=True, seed=1),
    "mha_b8_h4_t256_d32": dict(B=8, Hq=4, Hkv=4, T=256, D=32, do_std=1.0, backward=True, seed=2),
    "mha_b4_h8_t1024_d64": dict(B=4, Hq=8, Hkv=8, T=1024, D=64, do_std=0.1, backward=True, seed=3),
    "gqa_b1_hq16_hkv4_t8192_d64": dict(B=1, Hq=16, Hkv=4, T=8192, D=64, do_std=1.0,
                                       backward=False, seed=4),
}

# Paged decode: 32 sequences of one query token, context lengths uniform in
# [512, 4096], K/V in 16-token pages scattered through one shared pool by a
# seeded permutation.
DECODE_WORKLOADS = {
    "paged_decode_s32_hq16_hkv4_d64_p16": dict(S=32, Hq=16, Hkv=4, D=64, page_size=16,
                                               ctx_lo=512, ctx_hi=4096, max_pages=256, seed=5),
}


# Batched prefill into a paged cache (ragged): sequences with a cached prefix of
# U{cached_lo..cached_hi} positions each bring U{new_lo..new_hi} new tokens.
PREFILL_WORKLOADS = {
    "paged_prefill_s8_hq16_hkv4_d64_p16": dict(S=8, Hq=16, Hkv=4, D=64, page_size=16, cached_lo=0,
                                               cached_hi=2048, new_lo=128, new_hi=1024, max_pages=192,
                                               seed=6),
}


def causal_inputs(B, Hq, Hkv, T, D, seed, do_std=1.0, with_do=True):
    """Q [B,Hq,T,D], K, V [B,Hkv,T,D] and (optionally) dO [B,Hq,T,D], fp32, CPU.

    Draw order: Q, K, V, dO.  dO is N(0,1) scaled by ``do_std``.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, Hq, T, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, T, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, T, D), generator=g, dtype=torch.float32)
    out = {"q": q, "k": k, "v": v}
    if with_do:
        dout = torch.randn((B, Hq, T, D), generator=g, dtype=torch.float32)
        if do_std != 1.0:
            dout = dout * float(do_std)
        out["dout"] = dout
    return out


def causal_workload(name):
    """Inputs of one named causal workload (see CAUSAL_WORKLOADS)."""
    c = CAUSAL_WORKLOADS[name]
    return causal_inputs(c["B"], c["Hq"], c["Hkv"], c["T"], c["D"], c["seed"],
                         do_std=c["do_std"], with_do=c["backward"])


def paged_decode_inputs(S, Hq, Hkv, D, page_size, ctx_lo, ctx_hi, max_pages, seed,
                        pool_shuffle=True):
    """Context lengths, block tables and pools for batched single-token decode.

    Draw order: context lengths (uniform integers in [ctx_lo, ctx_hi]), the page
    permutation, Q [S,Hq,D], K pool, V pool [num_pages,Hkv,page_size,D].
    Sequence s owns ceil(ctx_s/page_size) logical pages; logical page p of s is
    physical page perm[offset_s + p].  The pool holds one extra page (index
    ``poison_page``) that pads every block table row past its last used page;
    a correct decode never reads it.
    """
    if ctx_hi > max_pages * page_size:
        raise ValueError("ctx_hi exceeds the block table's capacity")
    g = torch.Generator("cpu").manual_seed(int(seed))
    ctx = torch.randint(ctx_lo, ctx_hi + 1, (S,), generator=g, dtype=torch.int64)
    n_pages = [int(math.ceil(int(c) / page_size)) for c in ctx]
    total = sum(n_pages)
    perm = torch.randperm(total, generator=g) if pool_shuffle else torch.arange(total)
    block_table = torch.full((S, max_pages), total, dtype=torch.int32)
    off = 0
    for s, n in enumerate(n_pages):
        block_table[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    q = torch.randn((S, Hq, D), generator=g, dtype=torch.float32)
    k_pool = torch.randn((total + 1, Hkv, page_size, D), generator=g, dtype=torch.float32)
    v_pool = torch.randn((total + 1, Hkv, page_size, D), generator=g, dtype=torch.float32)
    return {
        "q": q, "k_pool": k_pool, "v_pool": v_pool, "block_table": block_table,
        "context_lens": ctx.to(torch.int32), "page_size": page_size, "num_pages": total + 1,
        "poison_page": total, "pages_used": total,
    }


def decode_workload(name):
    """Inputs of one named decode workload (see DECODE_WORKLOADS)."""
    c = DECODE_WORKLOADS[name]
    return paged_decode_inputs(c["S"], c["Hq"], c["Hkv"], c["D"], c["page_size"], c["ctx_lo"],
                               c["ctx_hi"], c["max_pages"], c["seed"])


def paged_prefill_inputs(S, Hq, Hkv, D, page_size, cached_lo, cached_hi, new_lo, new_hi, max_pages, seed,
                         pool_shuffle=True):
    """A ragged prefill batch over a paged cache whose new tokens are already appended.

    Draw order: cached lengths c_s (uniform integers in [cached_lo, cached_hi]), new
    token counts n_s (uniform in [new_lo, new_hi]), the page permutation, Q [N,Hq,D]
    (N = sum n_s, sequence by sequence), K pool, V pool [num_pages,Hkv,page_size,D].
    context_lens = c_s + n_s; token_start [S+1] = 0, n_0, n_0 + n_1, ...  Pages are
    laid out as in paged_decode_inputs (shuffled, one extra padding page).
    """
    if cached_hi + new_hi > max_pages * page_size:
        raise ValueError("cached_hi + new_hi exceeds the block table's capacity")
    g = torch.Generator("cpu").manual_seed(int(seed))
    cached = torch.randint(cached_lo, cached_hi + 1, (S,), generator=g, dtype=torch.int64)
    new = torch.randint(new_lo, new_hi + 1, (S,), generator=g, dtype=torch.int64)
    ctx = cached + new
    n_pages = [int(math.ceil(int(c) / page_size)) for c in ctx]
    total = sum(n_pages)
    perm = torch.randperm(total, generator=g) if pool_shuffle else torch.arange(total)
    block_table = torch.full((S, max_pages), total, dtype=torch.int32)
    off = 0
    for s, n in enumerate(n_pages):
        block_table[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    N = int(new.sum())
    token_start = torch.zeros((S + 1,), dtype=torch.int32)
    token_start[1:] = torch.cumsum(new, 0).to(torch.int32)
    q = torch.randn((N, Hq, D), generator=g, dtype=torch.float32)
    k_pool = torch.randn((total + 1, Hkv, page_size, D), generator=g, dtype=torch.float32)
    v_pool = torch.randn((total + 1, Hkv, page_size, D), generator=g, dtype=torch.float32)
    return {
        "q": q, "k_pool": k_pool, "v_pool": v_pool, "block_table": block_table,
        "context_lens": ctx.to(torch.int32), "token_start": token_start, "page_size": page_size,
        "num_pages": total + 1, "poison_page": total, "N": N,
    }


def prefill_workload(name):
    """Inputs of one named prefill workload (see PREFILL_WORKLOADS)."""
    c = PREFILL_WORKLOADS[name]
    return paged_prefill_inputs(c["S"], c["Hq"], c["Hkv"], c["D"], c["page_size"], c["cached_lo"],
                                c["cached_hi"], c["new_lo"], c["new_hi"], c["max_pages"], c["seed"])


def gather_sequence(k_pool, v_pool, block_table, ctx, s, page_size):
    """Contiguous [n,Hkv,D] copies of sequence s's K/V, by indexing only.

    Used to hand the same gathered KV to a dense decode; it is an index gather,
    not attention arithmetic.
    """
    n = int(ctx[s])
    pos = torch.arange(n)
    phys = block_table[s].to(torch.int64)[pos // page_size]
    off = pos % page_size
    kseq = k_pool[phys, :, off, :]
    vseq = v_pool[phys, :, off, :]
    return kseq.contiguous(), vseq.contiguous()
