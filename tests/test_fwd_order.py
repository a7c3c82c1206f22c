"""The forward's work order, as integer arithmetic on the host (CPU only).

A forward work-group x first maps to a work item through the XCD-grouped order (the G
query heads that read one K/V head go to work-groups on one XCD, x % 8, in consecutive
dispatch slots; padding work-groups past the last group get -1), then to a rank through
the snake order (ids dealt to the CUs in rounds of ncu, every second round reversed;
rank 0 is the longest causal prefix).  This model repeats both maps as the kernels write
them and checks, over grids up to 4096 items and G up to 16, that every item and every
rank is taken exactly once; that the G items of a group share an XCD; that the group order
is kept to within 8 groups; and that when the grid fills the chip exactly twice (n = 2 ncu,
the case the snake order serves) the two work-groups x and x + ncu that share a CU hold
ranks that add up to 2 ncu - 1, i.e. a heavy block with its light partner, also after the
XCD map when ncu is a multiple of 8 G.
"""
import pytest

XCDS = 8


def xcd_grouped_item(x, G, ngroups):
    if G == 1:
        return x if x < ngroups else -1
    slot = x // XCDS
    grp = (slot // G) * XCDS + x % XCDS
    return grp * G + slot % G if grp < ngroups else -1


def xcd_grouped_grid(G, ngroups):
    return ngroups if G == 1 else (ngroups + XCDS - 1) // XCDS * XCDS * G


def snake_rank(i, n, ncu):
    rnd = i // ncu
    base = rnd * ncu
    m = min(n - base, ncu)
    return base + (m - 1 - (i - base)) if rnd & 1 else i


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
def test_xcd_grouped_items_are_a_bijection(G):
    for ngroups in list(range(1, 70)) + [255, 256, 257, 1000]:
        grid = xcd_grouped_grid(G, ngroups)
        items = [xcd_grouped_item(x, G, ngroups) for x in range(grid)]
        real = sorted(i for i in items if i >= 0)
        assert real == list(range(ngroups * G)), (G, ngroups)
        assert grid - len(real) < XCDS * G                      # padding below one set of 8 groups
        xcds_of_group = {}
        for x, it in enumerate(items):
            if it >= 0:
                xcds_of_group.setdefault(it // G, set()).add(x % XCDS)
                # groups kept in order to within 8
                assert abs(it // G - x // (XCDS * G) * XCDS) < XCDS
        # the G items of a group on one XCD
        assert all(len(v) == 1 for v in xcds_of_group.values())


@pytest.mark.parametrize("ncu", [1, 7, 8, 64, 256])
def test_snake_rank_is_a_permutation(ncu):
    for n in list(range(1, 3 * ncu + 5, max(1, ncu // 7))) + [2 * ncu]:
        ranks = sorted(snake_rank(i, n, ncu) for i in range(n))
        assert ranks == list(range(n)), (n, ncu)


@pytest.mark.parametrize("G", [1, 2, 4])
def test_co_resident_pairs_are_heavy_with_light(G):
    ncu = 256
    n = 2 * ncu
    grid = xcd_grouped_grid(G, n // G)
    rank_of = {}
    for x in range(grid):
        it = xcd_grouped_item(x, G, n // G)
        if it >= 0:
            rank_of[x] = snake_rank(it, n, ncu)
    assert sorted(rank_of.values()) == list(range(n))
    for x in range(ncu):
        assert rank_of[x] + rank_of[x + ncu] == n - 1, (G, x)
