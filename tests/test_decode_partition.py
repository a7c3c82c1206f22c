"""The paged decode's split partition, as integer arithmetic on the host (CPU only).

The split kernels cut the list of all sequences' 16-position groups, with a charge of
C units before each sequence's groups, into equal shares: work-group w of n takes places
[w V / n, (w+1) V / n) of the charged list (V = N + C S), i.e. the groups whose place
u + C (s + 1) falls there, and sequence s's partials go to the consecutive slots of the
work-groups that hold its groups.  This model repeats that arithmetic (first_group, owner,
the slot counts and bases) exactly as the kernels write it, for C = 0 (plain equal
shares) and the library's C = 2, and checks on random length mixes (empty and very
unequal sequences included) that the shares cover every group once, in order; that owner()
agrees with the shares; that a sequence's slot count is the number of work-groups holding
its groups and all slots fit in n + S - 1; and that the charged load of every share
(groups plus C per sequence start it holds) is equal to within 2 C + 1 when every length is
at least 1, as decode requires (the shares' places differ by at most one, and a sequence's
C charge units may straddle two shares)."""
import random

import pytest


def partition(lengths, nwg, C):
    S = len(lengths)
    groups = [(x + 15) // 16 for x in lengths]
    incl, acc = [], 0
    for g in groups:
        acc += g
        incl.append(acc)                      # P_{s+1}
    total = acc
    V = total + C * S
    n = min(nwg, total)

    def start(s):
        return 0 if s == 0 else incl[s - 1]

    def owner(u, s):
        v = u + C * (s + 1)
        return ((v + 1) * n - 1) // V

    def first_group(v):
        k = sum(1 for s in range(S) if incl[s] + C * (s + 1) <= v)
        if k >= S:
            return total
        return max(start(k), v - C * (k + 1))

    shares = [(first_group(w * V // n), first_group((w + 1) * V // n)) for w in range(n)]
    cnt = [owner(incl[s] - 1, s) - owner(start(s), s) + 1 if groups[s] else 0 for s in range(S)]
    base = [sum(cnt[:s]) for s in range(S)]
    return dict(S=S, groups=groups, incl=incl, total=total, n=n, shares=shares, cnt=cnt, base=base,
                owner=owner, start=start)


def _seq_of(incl, u):
    return next(s for s, e in enumerate(incl) if u < e)


def _cases():
    r = random.Random(77)
    out = []
    for _ in range(60):
        S = r.choice([1, 2, 3, 7, 32, 100, 333, 1024])
        kind = r.randrange(4)
        if kind == 0:
            lengths = [r.randint(512, 4096) for _ in range(S)]
        elif kind == 1:
            lengths = [r.randint(1, 40) for _ in range(S)]
        elif kind == 2:
            lengths = [r.choice([0, 1, 16, 17, 5000]) for _ in range(S)]
        else:
            lengths = [int(r.expovariate(1 / 800)) for _ in range(S)]
        out.append((lengths, r.choice([64, 256, 512, 1024])))
    return out


@pytest.mark.parametrize("C", [0, 2])
def test_decode_partition_invariants(C):
    for lengths, nwg in _cases():
        p = partition(lengths, nwg, C)
        if p["total"] == 0:
            continue
        S, incl, n = p["S"], p["incl"], p["n"]
        # the shares cover groups 0 .. total-1 once, in order (some may be empty when C > 0)
        assert p["shares"][0][0] == 0 and p["shares"][-1][1] == p["total"]
        for (a, b), (c, d) in zip(p["shares"], p["shares"][1:]):
            assert a <= b == c <= d
        if C == 0:
            assert all(a < b for a, b in p["shares"])
        # owner() names the share that holds each group
        for w, (a, b) in enumerate(p["shares"]):
            for u in range(a, b):
                assert p["owner"](u, _seq_of(incl, u)) == w
        # slots: a sequence's count is the number of shares holding its groups
        for s in range(S):
            holders = {w for w, (a, b) in enumerate(p["shares"]) if max(a, p["start"](s)) < min(b, incl[s])}
            assert p["cnt"][s] == len(holders)
            if holders:
                assert min(holders) == p["owner"](p["start"](s), s)
        assert sum(p["cnt"]) <= n + S - 1
        # balance of the charged load (for valid lengths, all >= 1: an empty sequence's
        # charge units take places without work): groups plus C per sequence start held
        if min(lengths) < 1:
            continue
        loads = []
        for a, b in p["shares"]:
            starts = sum(1 for s in range(S) if p["groups"][s] and a <= p["start"](s) < b)
            loads.append((b - a) + C * starts)
        assert max(loads) - min(loads) <= 2 * C + 1, (max(loads), min(loads))
