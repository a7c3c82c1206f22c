"""GPU parity of the paged K/V cache calls (attn_kv_append, attn_kv_release)
against the plain model in oracle/kv_cache.py, and of decode over an appended
cache against the dense oracle.

The cache operations move data and integers, so the bar is bit-exact: after
every call the pools, page tables, lengths, the live part of the free stack, its
count and the status word equal the model's.
"""
import math

import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
from gpu_common import TOL_DECODE, announce, rel_err, require_gpu
from oracle.kv_cache import KV_OK, KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL, KV_STACK_OVERFLOW, KvCacheModel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _assert_same_state(c, m, where):
    torch.cuda.synchronize()
    fc = int(c.free_count.item())
    assert int(c.kv_status.item()) == m.status, (where, "status", int(c.kv_status.item()), m.status)
    assert fc == m.free_count, (where, "free_count", fc, m.free_count)
    assert np.array_equal(c.context_lens.cpu().numpy(), m.context_lens), (where, "context_lens")
    assert np.array_equal(c.block_table.cpu().numpy(), m.block_table), (where, "block_table")
    assert np.array_equal(c.free_pages.cpu().numpy()[:fc], m.free_pages[:fc]), (where, "free stack")
    assert np.array_equal(c.k_pool.cpu().numpy(), m.k_pool), (where, "k_pool")
    assert np.array_equal(c.v_pool.cpu().numpy(), m.v_pool), (where, "v_pool")


# single-token appends up to 1024 sequences and 4096 float4 rows take the one-launch path
# (lease and copy in one work-group); the second-to-last case is exactly at both limits,
# the two before it past the row limit, the last past the sequence limit
KV_CASES = [(37, 4, 64, 16, 6, 120), (37, 2, 8, 64, 2, 40), (9, 2, 128, 32, 5, 30), (100, 8, 64, 16, 3, 250),
            (40, 16, 128, 16, 4, 150), (1024, 1, 16, 16, 2, 1500), (1500, 1, 16, 16, 2, 2100)]


@pytest.mark.parametrize("S,Hkv,D,ps,max_pages,num_pages", KV_CASES)
def test_kv_calls_match_model(dev, S, Hkv, D, ps, max_pages, num_pages):
    """Random appends and releases, including refused appends (pool exhausted,
    sequence full); the last case has more sequences than one scan block."""
    announce(f"kv append/release S={S} Hkv={Hkv} D={D} page={ps}")
    rng = np.random.default_rng(S + D + ps)
    c = attn.PagedKvCache(S, Hkv, D, ps, max_pages, num_pages, dev)
    m = KvCacheModel(S, Hkv, D, ps, max_pages, num_pages)
    steps = 3 * ps * max_pages if S < 1000 else 2 * ps + 3
    saw = set()
    for step in range(steps):
        if rng.random() < 0.03:
            k = int(rng.integers(0, max(1, S // 3) + 1))
            ids = np.sort(rng.choice(S, size=k, replace=False)).astype(np.int32)
            c.release(torch.from_numpy(ids).to(dev))
            m.release(ids.tolist())
        else:
            kn = rng.standard_normal((S, Hkv, D)).astype(np.float32)
            vn = rng.standard_normal((S, Hkv, D)).astype(np.float32)
            c.append(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev))
            m.append(kn, vn)
        saw.add(m.status)
        if step % 7 == 0 or m.status != KV_OK:
            _assert_same_state(c, m, step)
    _assert_same_state(c, m, "end")
    if S < 1000:
        assert saw & {KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL}, "no refused append was exercised"


def test_release_overflow_changes_nothing(dev):
    announce("kv release overflow")
    c = attn.PagedKvCache(2, 1, 16, 16, 2, 2, dev)
    m = KvCacheModel(2, 1, 16, 16, 2, 2)
    x = np.ones((2, 1, 16), dtype=np.float32)
    c.append(torch.from_numpy(x).to(dev), torch.from_numpy(x).to(dev))
    m.append(x, x)
    # both pages are leased; a count claiming both are free again (as if pushed twice)
    # makes releasing sequence 0 overflow the stack, which must be refused
    c.free_count.fill_(2)
    m.free_count = 2
    ids = torch.tensor([0], dtype=torch.int32, device=dev)
    c.release(ids)
    assert m.release([0]) == KV_STACK_OVERFLOW
    _assert_same_state(c, m, "overflow")


def test_release_of_nothing_is_ok(dev):
    c = attn.PagedKvCache(2, 1, 16, 16, 2, 4, dev)
    c.kv_status.fill_(7)
    c.release(torch.empty((0,), dtype=torch.int32, device=dev))
    assert c.status() == KV_OK and int(c.free_count.item()) == 4


@pytest.mark.parametrize("G,ps", [(4, 16), (1, 64)])
def test_decode_over_appended_cache(dev, orc, G, ps):
    """Decode reads exactly what the appends wrote: build contexts of mixed lengths
    with appends and releases, then compare decode with the oracle on the model."""
    S, Hkv, D, max_pages = 8, 2, 64, 40
    announce(f"decode over appended cache G={G} page={ps}")
    num_pages = S * max_pages
    rng = np.random.default_rng(11 + G)
    c = attn.PagedKvCache(S, Hkv, D, ps, max_pages, num_pages, dev)
    m = KvCacheModel(S, Hkv, D, ps, max_pages, num_pages)
    for step in range(300):
        if step in (40, 170):
            ids = np.array([1, 4, 6] if step == 40 else [0, 3], dtype=np.int32)
            c.release(torch.from_numpy(ids).to(dev))
            m.release(ids.tolist())
        kn = rng.standard_normal((S, Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((S, Hkv, D)).astype(np.float32)
        c.append(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev))
        assert m.append(kn, vn) == KV_OK
    _assert_same_state(c, m, "built")
    q = torch.randn((S, Hkv * G, D), generator=torch.Generator("cpu").manual_seed(5))
    o, lse = attn.attn_paged_decode(q.to(dev), c.k_pool, c.v_pool, c.block_table, c.context_lens)
    torch.cuda.synchronize()
    ro, rlse = orc.paged_decode(q, m.k_pool, m.v_pool, m.block_table, m.context_lens)
    assert rel_err(o, ro) <= TOL_DECODE and rel_err(lse, rlse) <= TOL_DECODE
    # and the dense decode over each sequence's appended stream
    for s in range(S):
        ks, vs = m.gather(s)
        rd, _ = orc.decode_dense(q[s], torch.from_numpy(ks), torch.from_numpy(vs), 1.0 / math.sqrt(D))
        assert rel_err(o[s], rd) <= TOL_DECODE, s
