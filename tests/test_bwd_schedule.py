"""The causal backward's work cut, as integer arithmetic on the host (CPU only).

The backward's work for one (batch, KV head) is the list of steps (key block kb, query
head, query tile >= kb), key block after key block in the paired order 0, n-1, 1, n-2, ...
(two neighbours hold G (n + 1) steps together).  When the key-block grid fits on the chip
at once the list is cut into `runs` equal runs, one per work-group: half a pair each
(runs = n), or finer (runs > n) when half pairs would leave CUs idle.  This model repeats
the kernels' arithmetic (the run of a work-group, its first position in the pair order,
the segments it walks, the preprocess's zeroed rows and the post kernel's view of a
shared key block) and checks, for every n < 130 key blocks and G <= 8 query heads per KV
head, that:
  * the work-groups of a (batch, KV head) take every run exactly once;
  * every step of every key block belongs to exactly one run, runs walk their segments in
    list order, and a key block shared by several runs is the first or the last segment
    of each of them (two workspace slots per run suffice);
  * with half pairs a run has at most two segments and only key blocks below n / 2 are
    ever shared, so zeroing the first (n / 2) 64 keys of dK, dV before the atomic adds
    covers every shared block, and each shared block has exactly two addends (the same
    bits in either order);
  * with finer runs the post kernel finds, for each key block, exactly the runs that hold
    a piece of it, in run order, and which of a run's two slots holds it.
"""
import pytest


def pair_order(n, G):
    pair_len = G * (n + 1)

    def kb_at(pi):
        return n - 1 - (pi >> 1) if pi & 1 else pi >> 1

    def start_at(pi):
        pr = pi >> 1
        return pr * pair_len + (G * (n - pr) if pi & 1 else 0)

    return pair_len, kb_at, start_at


def run_of_workgroup(x, grid, runs, nbkv):
    """(run, bkv) of work-group x: neighbouring runs for x and x + grid/2 when runs is even."""
    if runs % 2 == 0:
        half = grid // 2
        hi = 1 if x >= half else 0
        j = x - hi * half
        return 2 * (j // nbkv) + 1 - hi, j % nbkv
    return x // nbkv, x % nbkv


def walk(n, G, runs, run):
    """The segments of a run: (key block, first step, end step within the block, whole?)."""
    pair_len, kb_at, start_at = pair_order(n, G)
    total = G * n * (n + 1) // 2
    s_begin, s_end = run * total // runs, (run + 1) * total // runs
    if s_begin >= s_end:
        return [], None
    pr = s_begin // pair_len
    pi = 2 * pr + (1 if s_begin - pr * pair_len >= G * (n - pr) else 0)
    first_pi = pi
    segs = []
    s = s_begin
    while s < s_end:
        kb = kb_at(pi)
        kb_first = start_at(pi)
        kb_end = kb_first + G * (n - kb)
        assert kb_first <= s < kb_end
        seg_end = min(s_end, kb_end)
        segs.append((kb, s - kb_first, seg_end - kb_first, s == kb_first and seg_end == kb_end, pi))
        s = seg_end
        pi += 1
    return segs, first_pi


def post_view(n, G, runs, kb):
    """The post kernel's view of key block kb: runs r0 .. r1 and r0's slot."""
    pair_len = G * (n + 1)
    pi = 2 * kb if 2 * kb < n else 2 * (n - 1 - kb) + 1
    pr = pi >> 1
    bs = pr * pair_len + (G * (n - pr) if pi & 1 else 0)
    be = bs + G * (n - kb)
    total = G * n * (n + 1) // 2
    r0 = ((bs + 1) * runs - 1) // total
    r1 = (be * runs - 1) // total
    w0 = 0 if r0 * total // runs == bs else 1
    return r0, r1, w0


def check(n, G, runs, nbkv=3):
    grid = runs * nbkv
    seen = sorted(run_of_workgroup(x, grid, runs, nbkv) for x in range(grid))
    assert seen == [(r, b) for r in range(runs) for b in range(nbkv)]

    pieces = {kb: [] for kb in range(n)}
    for run in range(runs):
        segs, first_pi = walk(n, G, runs, run)
        if runs == n:
            assert len(segs) <= 2
        for i, (kb, j0, j1, whole, pi) in enumerate(segs):
            pieces[kb].append((j0, j1, run, pi != first_pi))
            if not whole:
                assert i == 0 or i == len(segs) - 1, (n, G, runs, run, segs)
    for kb, v in pieces.items():
        v.sort()
        assert v[0][0] == 0 and v[-1][1] == G * (n - kb), (n, G, runs, kb, v)
        for a, b in zip(v, v[1:]):
            assert a[1] == b[0], (n, G, runs, kb, v)          # contiguous, no overlap
        assert [p[2] for p in v] == sorted(p[2] for p in v)   # in run order
        if len(v) > 1:
            if runs == n:
                assert len(v) == 2 and kb < n // 2, (n, G, kb, v)
                assert kb * 64 + 64 <= (n // 2) * 64            # inside the zeroed rows
            else:
                r0, r1, w0 = post_view(n, G, runs, kb)
                assert [p[2] for p in v] == list(range(r0, r1 + 1)), (n, G, runs, kb, v, r0, r1)
                assert w0 == (1 if v[0][3] else 0)               # r0's slot: its last segment or its first
                assert all(not p[3] for p in v[1:])              # the block is the first segment of later runs


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_half_pairs(G):
    for n in range(1, 130):
        check(n, G, n)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_finer_runs(G):
    for n in range(1, 70):
        total = G * n * (n + 1) // 2
        for runs in sorted({n + 1, 2 * n, 3 * n + 1, min(512, total // 2)}):
            if runs > n and total // runs >= 2:   # at least two steps per run, as the launcher picks
                check(n, G, runs)
