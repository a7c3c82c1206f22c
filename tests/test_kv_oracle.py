"""Pins of the paged K/V cache model (oracle/kv_cache.py), all on the CPU.

What pins it, independently of its own code:
  * the defining property of a cache: what is read back through the page table
    equals the stream that was appended (tracked here with plain lists);
  * page accounting: live pages are distinct, none is on the free stack, and
    live + free = num_pages after every operation;
  * a small example worked out by hand (page ids written below as numbers);
  * the error cases change nothing;
  * two plausible mistakes (lease order reversed, release order reversed) fail
    the hand-worked example.
"""
import numpy as np
import pytest

from oracle.kv_cache import (KV_OK, KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL, KV_STACK_OVERFLOW,
                             KvCacheModel)


def _rows(rng, S, Hkv, D):
    return rng.standard_normal((S, Hkv, D)).astype(np.float32)


def _check_accounting(m):
    live = [p for (_, _, p) in m.live_pages()]
    assert len(live) == len(set(live)), "a physical page is held twice"
    free = set(int(x) for x in m.free_pages[:m.free_count])
    assert not (free & set(live)), "a live page is on the free stack"
    assert m.free_count + len(live) == m.num_pages
    assert all(0 <= p < m.num_pages for p in live)


def _snapshot(m):
    return (m.k_pool.copy(), m.v_pool.copy(), m.block_table.copy(), m.context_lens.copy(),
            m.free_pages.copy(), m.free_count)


def _same(a, b):
    return all(np.array_equal(x, y) if isinstance(x, np.ndarray) else x == y for x, y in zip(a, b))


@pytest.mark.parametrize("page_size", [16, 32])
def test_gathered_stream_equals_appended_stream(page_size):
    rng = np.random.default_rng(3)
    S, Hkv, D, max_pages, num_pages = 5, 2, 8, 4, 12
    m = KvCacheModel(S, Hkv, D, page_size, max_pages, num_pages)
    streams = [([], []) for _ in range(S)]
    for step in range(150):
        if step % 23 == 22:  # release a few sequences now and then
            ids = sorted(rng.choice(S, size=int(rng.integers(1, S)), replace=False).tolist())
            assert m.release(ids) == KV_OK
            for s in ids:
                streams[s] = ([], [])
        else:
            kn, vn = _rows(rng, S, Hkv, D), _rows(rng, S, Hkv, D)
            before = _snapshot(m)
            st = m.append(kn, vn)
            if st == KV_OK:
                for s in range(S):
                    streams[s][0].append(kn[s])
                    streams[s][1].append(vn[s])
            else:  # a refused append changes nothing
                assert st in (KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL)
                assert _same(before, _snapshot(m))
                ids = list(range(S))
                assert m.release(ids) == KV_OK
                streams = [([], []) for _ in range(S)]
        _check_accounting(m)
        for s in range(S):
            ks, vs = m.gather(s)
            assert ks.shape[0] == len(streams[s][0])
            if ks.shape[0]:
                assert np.array_equal(ks, np.stack(streams[s][0]))
                assert np.array_equal(vs, np.stack(streams[s][1]))


def _hand_example(model_cls):
    """S=3 sequences, 16-position pages, 2 pages per sequence, 4 pages in the pool.
    Returns the list of observations compared with the hand-worked values."""
    m = model_cls(3, 1, 4, 16, 2, 4)
    obs = []
    z = np.zeros((3, 1, 4), dtype=np.float32)
    obs.append(m.append(z, z))                        # t = 0 for all: three leases
    obs.append(m.block_table[:, 0].tolist())
    obs.append(m.free_count)
    for _ in range(15):                               # t = 1 .. 15: no lease
        m.append(z, z)
    obs.append(m.append(z, z))                        # t = 16: three needed, one free
    obs.append(m.context_lens.tolist())
    obs.append(m.release([1]))                        # pushes page 1
    obs.append((m.free_pages[:m.free_count].tolist(), m.context_lens.tolist()))
    obs.append(m.release([0, 2]))                     # pushes pages 0, then 2
    obs.append(m.free_pages[:m.free_count].tolist())
    obs.append(m.append(z, z))                        # all start again: three leases from the top
    obs.append(m.block_table[:, 0].tolist())
    return obs


# Worked by hand: the stack starts as [3, 2, 1, 0] (top last).  The first append
# leases to sequences 0, 1, 2 in order: pages 0, 1, 2, leaving [3].  At t = 16 all
# three need a page and only one is free: refused, lengths stay 16.  Releasing
# sequence 1 pushes its page 1: [3, 1]; releasing 0 and 2 pushes 0 then 2:
# [3, 1, 0, 2].  The next append gives sequence 0 the top (2), then 0, then 1.
HAND = [KV_OK, [0, 1, 2], 1, KV_POOL_EXHAUSTED, [16, 16, 16], KV_OK, ([3, 1], [16, 0, 16]), KV_OK,
        [3, 1, 0, 2], KV_OK, [2, 0, 1]]


def test_hand_worked_example():
    assert _hand_example(KvCacheModel) == HAND


class _ReversedLease(KvCacheModel):
    """Mutant: sequences that start a page lease in reverse index order."""

    def append(self, k_new, v_new):
        lengths = [int(t) for t in self.context_lens]
        starting = [s for s in range(self.S) if lengths[s] % self.page_size == 0]
        if any(t >= self.page_size * self.max_pages for t in lengths):
            return KV_SEQUENCE_FULL
        if len(starting) > self.free_count:
            return KV_POOL_EXHAUSTED
        for r, s in enumerate(reversed(starting)):
            self.block_table[s, lengths[s] // self.page_size] = self.free_pages[self.free_count - 1 - r]
        self.free_count -= len(starting)
        for s in range(self.S):
            t = lengths[s]
            page = int(self.block_table[s, t // self.page_size])
            self.k_pool[page, :, t % self.page_size, :] = k_new[s]
            self.v_pool[page, :, t % self.page_size, :] = v_new[s]
            self.context_lens[s] = t + 1
        return KV_OK


class _ReversedRelease(KvCacheModel):
    """Mutant: released sequences are pushed in reverse list order."""

    def release(self, seq_ids):
        return super().release(list(reversed(seq_ids)))


@pytest.mark.parametrize("mutant", [_ReversedLease, _ReversedRelease])
def test_hand_example_catches_mutants(mutant):
    assert _hand_example(mutant) != HAND


def test_full_sequence_is_refused_and_changes_nothing():
    m = KvCacheModel(1, 1, 4, 16, 1, 2)
    z = np.ones((1, 1, 4), dtype=np.float32)
    for _ in range(16):
        assert m.append(z, z) == KV_OK
    before = _snapshot(m)
    assert m.append(z, z) == KV_SEQUENCE_FULL
    assert _same(before, _snapshot(m))


def test_release_overflow_is_refused_and_changes_nothing():
    m = KvCacheModel(1, 1, 4, 16, 1, 1)
    z = np.ones((1, 1, 4), dtype=np.float32)
    assert m.append(z, z) == KV_OK and m.free_count == 0
    m.free_count = 1  # a corrupted count: the page would be pushed a second time
    before = _snapshot(m)
    assert m.release([0]) == KV_STACK_OVERFLOW
    assert _same(before, _snapshot(m))


# ----------------------------------------------------------------------------
# ragged multi-token append (the step before a batched prefill)
# ----------------------------------------------------------------------------
def test_append_tokens_gathered_stream_and_accounting():
    """Ragged appends (some sequences adding nothing, some crossing several pages):
    what is read back equals what was appended, and the page accounting holds."""
    rng = np.random.default_rng(11)
    S, Hkv, D, ps, max_pages, num_pages = 4, 2, 4, 16, 6, 20
    m = KvCacheModel(S, Hkv, D, ps, max_pages, num_pages)
    streams = [([], []) for _ in range(S)]
    for step in range(60):
        if step % 17 == 16:
            ids = sorted(rng.choice(S, size=int(rng.integers(1, S)), replace=False).tolist())
            assert m.release(ids) == KV_OK
            for s in ids:
                streams[s] = ([], [])
            continue
        counts = rng.integers(0, 40, size=S)
        ts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        kn = rng.standard_normal((int(ts[-1]), Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((int(ts[-1]), Hkv, D)).astype(np.float32)
        before = _snapshot(m)
        st = m.append_tokens(kn, vn, ts)
        if st == KV_OK:
            for s in range(S):
                streams[s][0].extend(kn[ts[s]:ts[s + 1]])
                streams[s][1].extend(vn[ts[s]:ts[s + 1]])
        else:
            assert st in (KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL)
            assert _same(before, _snapshot(m)), "a refused append changed the state"
        _check_accounting(m)
        for s in range(S):
            ks, vs = m.gather(s)
            assert len(ks) == len(streams[s][0])
            if len(ks):
                assert np.array_equal(ks, np.stack(streams[s][0])) and np.array_equal(vs, np.stack(streams[s][1]))


def test_append_tokens_one_each_is_append():
    """One new row per sequence: the same state as the single-token append."""
    rng = np.random.default_rng(12)
    S, Hkv, D, ps = 3, 2, 4, 16
    a = KvCacheModel(S, Hkv, D, ps, 3, 8)
    b = KvCacheModel(S, Hkv, D, ps, 3, 8)
    ts = np.arange(S + 1, dtype=np.int32)
    for _ in range(40):
        kn, vn = _rows(rng, S, Hkv, D), _rows(rng, S, Hkv, D)
        assert a.append(kn, vn) == b.append_tokens(kn, vn, ts)
        assert _same(_snapshot(a), _snapshot(b))


def test_append_tokens_worked_example():
    """Lengths [15, 0, 32], page 16, 8 pages, stack top = page 0.  Adding [3, 20, 0]
    rows: sequence 0 needs logical page 1 (positions 16, 17), sequence 1 logical pages
    0 and 1, sequence 2 nothing -> pages 0 | 1, 2 from the top, in that order."""
    m = KvCacheModel(3, 1, 4, 16, 4, 8)
    m.context_lens[:] = [15, 0, 32]
    m.block_table[0, 0] = 7
    m.block_table[2, :2] = [6, 5]
    m.free_pages[:5] = [4, 3, 2, 1, 0]
    m.free_count = 5
    ts = np.array([0, 3, 23, 23], dtype=np.int32)
    kn = np.arange(23 * 4, dtype=np.float32).reshape(23, 1, 4)
    assert m.append_tokens(kn, -kn, ts) == KV_OK
    assert m.block_table[0, :2].tolist() == [7, 0]
    assert m.block_table[1, :2].tolist() == [1, 2]
    assert m.block_table[2, :2].tolist() == [6, 5]
    assert m.context_lens.tolist() == [18, 20, 32] and m.free_count == 2
    assert np.array_equal(m.k_pool[7, 0, 15], kn[0, 0]) and np.array_equal(m.k_pool[0, 0, 1], kn[2, 0])
    assert np.array_equal(m.k_pool[2, 0, 3], kn[3 + 19, 0]) and np.array_equal(m.v_pool[1, 0, 0], -kn[3, 0])


def test_append_tokens_refusals_change_nothing():
    m = KvCacheModel(2, 1, 4, 16, 2, 3)
    ts = np.array([0, 33, 33], dtype=np.int32)  # 33 > 2 pages of 16
    before = _snapshot(m)
    assert m.append_tokens(np.zeros((33, 1, 4), np.float32), np.zeros((33, 1, 4), np.float32), ts) == KV_SEQUENCE_FULL
    assert _same(before, _snapshot(m))
    ts = np.array([0, 32, 64], dtype=np.int32)  # 4 pages needed, 3 free
    assert m.append_tokens(np.zeros((64, 1, 4), np.float32), np.zeros((64, 1, 4), np.float32), ts) == KV_POOL_EXHAUSTED
    assert _same(before, _snapshot(m))
