"""The batched prefill's work order, as integer arithmetic on the host (CPU only).

A prefill work item is one 64-token block qb of the new tokens of sequence s (for every
query head).  Block qb of a sequence with n new tokens and ctx cached positions (the new
ones included) reaches position L = min(base + min(64 qb + 64, n) - 1, ctx - 1), with
base = ctx - n, and visits L / 64 + 1 key tiles.  The kernel ranks the blocks of the whole
batch heaviest first (most tiles; ties by sequence, then block) and finds the block of
rank `item` without a sort: by bisection on t of the number of blocks with at least t
tiles, which has a closed form per sequence, then the rank among the blocks with exactly
the found count.  This model repeats that arithmetic as the kernel writes it and checks,
on random ragged batches (empty sequences, one-token sequences and long cached prefixes
included), that it yields every block exactly once, in exactly the order of a plain sort
by (-tiles, sequence, block), and nothing past the last block.
"""
import random

BM = BN = 64


def seq_blocks(n, ctx):
    return {"nb": (n + BM - 1) // BM, "n": n, "base": max(ctx - n, 0), "ctxm1": ctx - 1}


def tiles(q, qb):
    last = min(q["base"] + min(BM * qb + BM, q["n"]) - 1, q["ctxm1"])
    return max(last, 0) // BN + 1


def cnt_ge(q, t):
    if t <= 1:
        return q["nb"]
    P = BN * (t - 1)
    R = P - q["base"] + 1
    if q["nb"] == 0 or q["ctxm1"] < P or q["n"] < R:
        return 0
    return q["nb"] - (0 if R <= BM else (R - 1) // BM)


def select(seqs, item):
    """(sequence, block) of rank `item`, or None past the last block -- as in the kernel."""
    def total_ge(t):
        return sum(cnt_ge(q, t) for q in seqs)
    if item >= total_ge(1):
        return None
    tmax = max((max(min(q["base"] + q["n"] - 1, q["ctxm1"]), 0) // BN + 1) if q["nb"] > 0 else 0 for q in seqs)
    lo, hi = 1, tmax
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if total_ge(mid) > item:
            lo = mid
        else:
            hi = mid - 1
    k = item - (total_ge(lo + 1) if lo < tmax else 0)
    carry = 0
    for s, q in enumerate(seqs):
        ge = cnt_ge(q, lo)
        eq = ge - cnt_ge(q, lo + 1)
        if k < carry + eq:
            return s, (q["nb"] - ge) + (k - carry)
        carry += eq
    raise AssertionError("no block found")


def test_prefill_order_matches_a_sort():
    rng = random.Random(7)
    for trial in range(400):
        S = rng.randint(1, 20)
        seqs = []
        for _ in range(S):
            kind = rng.random()
            n = 0 if kind < 0.1 else (1 if kind < 0.2 else rng.randint(1, 700))
            cached = rng.choice([0, 0, rng.randint(0, 3000)])
            seqs.append(seq_blocks(n, cached + n))
        blocks = [(s, qb) for s, q in enumerate(seqs) for qb in range(q["nb"])]
        expect = sorted(blocks, key=lambda sb: (-tiles(seqs[sb[0]], sb[1]), sb[0], sb[1]))
        got = [select(seqs, i) for i in range(len(blocks))]
        assert got == expect, (trial, seqs)
        assert select(seqs, len(blocks)) is None
        for s, q in enumerate(seqs):   # the closed form against counting
            for t in range(1, 60):
                assert cnt_ge(q, t) == sum(1 for qb in range(q["nb"]) if tiles(q, qb) >= t), (q, t)
