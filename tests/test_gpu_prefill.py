"""GPU parity of batched prefill over a paged cache (attn_paged_prefill) and of
the ragged multi-token append before it (attn_kv_append_tokens).

Prefill outputs are compared with the oracle (oracle_paged_prefill, float64) at
the forward's bars: O and LSE within 1e-4 (max-abs error relative to the
reference's largest magnitude).  The append moves data and integers, so its bar
is bit-exact against the plain model in oracle/kv_cache.py.
"""
import math

import numpy as np
import pytest
import torch

import causal_self_attention_amd as attn
import synthetic_inputs as si
from gpu_common import TOL_LSE, TOL_O, announce, rel_err, require_gpu
from oracle.kv_cache import KV_OK, KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL, KvCacheModel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _prefill(d, dev, scale=None, with_lse=True):
    o, lse = attn.attn_paged_prefill(d["q"].to(dev), d["k_pool"].to(dev), d["v_pool"].to(dev),
                                     d["block_table"].to(dev), d["context_lens"].to(dev),
                                     d["token_start"].to(dev), scale=scale, with_lse=with_lse)
    torch.cuda.synchronize()
    return o, lse


def _batch(S, Hq, Hkv, D, ps, cached, new, seed, shuffle=True):
    """A ragged batch with given cached and new lengths (pages shuffled, one padding page)."""
    g = torch.Generator("cpu").manual_seed(seed)
    ctx = [c + n for c, n in zip(cached, new)]
    n_pages = [-(-c // ps) for c in ctx]
    total = sum(n_pages)
    maxp = max(n_pages) + 1
    perm = torch.randperm(total, generator=g) if shuffle else torch.arange(total)
    bt = torch.full((S, maxp), total, dtype=torch.int32)
    off = 0
    for s, n in enumerate(n_pages):
        bt[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    N = sum(new)
    ts = torch.zeros((S + 1,), dtype=torch.int32)
    ts[1:] = torch.cumsum(torch.tensor(new), 0).to(torch.int32)
    return {"q": torch.randn((N, Hq, D), generator=g), "k_pool": torch.randn((total + 1, Hkv, ps, D), generator=g),
            "v_pool": torch.randn((total + 1, Hkv, ps, D), generator=g), "block_table": bt,
            "context_lens": torch.tensor(ctx, dtype=torch.int32), "token_start": ts, "page_size": ps,
            "poison_page": total}


def _check(d, dev, orc):
    o, lse = _prefill(d, dev)
    ro, rlse = orc.paged_prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                                 d["token_start"])
    assert rel_err(o, ro) <= TOL_O, ("O", rel_err(o, ro))
    assert rel_err(lse, rlse) <= TOL_LSE, ("LSE", rel_err(lse, rlse))
    return o, lse


RAGGED = [
    # (Hq, Hkv, D, page, cached lengths, new lengths)
    (16, 4, 64, 16, [0, 17, 100, 64, 300, 5], [33, 1, 0, 130, 64, 200]),
    (8, 8, 32, 32, [1, 250, 0], [64, 65, 127]),
    (4, 1, 128, 64, [90, 0], [100, 1]),
    (6, 2, 16, 16, [0, 0, 7], [1, 63, 9]),
    (2, 2, 8, 16, [40, 3], [129, 2]),
    (16, 2, 64, 32, [1000, 0, 2047, 333], [257, 300, 1, 64]),
]


@pytest.mark.parametrize("Hq,Hkv,D,ps,cached,new", RAGGED)
def test_prefill_ragged(dev, orc, Hq, Hkv, D, ps, cached, new):
    announce(f"prefill ragged Hq={Hq} Hkv={Hkv} D={D} page={ps} cached={cached} new={new}")
    d = _batch(len(new), Hq, Hkv, D, ps, cached, new, seed=sum(cached) + D)
    o, lse = _check(d, dev, orc)
    o2, lse2 = _prefill(d, dev, with_lse=False)  # without lse: the same bits
    assert lse2 is None and torch.equal(o, o2)
    o3, lse3 = _prefill(d, dev)                   # run to run: the same bits
    assert torch.equal(o, o3) and torch.equal(lse, lse3)


def test_prefill_workload(dev, orc):
    """The 8-sequence workload (4172 new tokens, contexts up to 2737 positions) in the
    configuration the bench times: whole O and LSE against the oracle's batched prefill,
    and sampled rows against a second route, each row as a one-token prefill at its own
    position."""
    name = next(iter(si.PREFILL_WORKLOADS))
    announce(f"prefill workload {name}")
    d = si.prefill_workload(name)
    o, lse = _prefill(d, dev)
    wo, wlse = orc.paged_prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                                 d["token_start"])
    assert rel_err(o, wo) <= TOL_O, ("O", rel_err(o, wo))
    assert rel_err(lse, wlse) <= TOL_LSE, ("LSE", rel_err(lse, wlse))
    ts, ctx = d["token_start"].tolist(), d["context_lens"].tolist()
    rows, seqs, pos = [], [], []
    for s in range(len(ctx)):
        n = ts[s + 1] - ts[s]
        for j in sorted({0, 1, n // 3, n // 2, n - 2, n - 1}):
            rows.append(ts[s] + j)
            seqs.append(s)
            pos.append(ctx[s] - n + j)
    sub_ts = torch.arange(len(rows) + 1, dtype=torch.int32)
    ro, rlse = orc.paged_prefill(d["q"][rows], d["k_pool"], d["v_pool"], d["block_table"][seqs],
                                 torch.tensor([p + 1 for p in pos], dtype=torch.int32), sub_ts)
    assert rel_err(o[rows], ro) <= TOL_O, ("O", rel_err(o[rows], ro))
    assert rel_err(lse[rows], rlse) <= TOL_LSE


def test_prefill_one_token_each_is_decode(dev, orc):
    announce("prefill one token per sequence vs decode")
    d = si.paged_decode_inputs(S=9, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=700, max_pages=48, seed=81)
    d["token_start"] = torch.arange(10, dtype=torch.int32)
    o, lse = _check(d, dev, orc)
    od, lsed = attn.attn_paged_decode(d["q"].to(dev), d["k_pool"].to(dev), d["v_pool"].to(dev),
                                      d["block_table"].to(dev), d["context_lens"].to(dev))
    torch.cuda.synchronize()
    assert rel_err(o, od) <= 1e-5 and rel_err(lse, lsed) <= 1e-5


def test_prefill_whole_sequences_are_causal_forward(dev):
    """No cached prefix: each sequence's rows are the causal forward over its tokens."""
    announce("prefill whole sequences vs causal forward")
    T, Hq, Hkv, D, ps = 300, 8, 2, 64, 16
    host = si.causal_inputs(1, Hq, Hkv, T, D, seed=82, with_do=False)
    npg = math.ceil(T / ps)
    kp = torch.zeros(npg, Hkv, ps, D)
    vp = torch.zeros(npg, Hkv, ps, D)
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(83))
    for t in range(T):
        kp[perm[t // ps], :, t % ps] = host["k"][0, :, t]
        vp[perm[t // ps], :, t % ps] = host["v"][0, :, t]
    d = {"q": host["q"][0].transpose(0, 1).contiguous(), "k_pool": kp, "v_pool": vp,
         "block_table": perm.to(torch.int32).unsqueeze(0), "context_lens": torch.tensor([T], dtype=torch.int32),
         "token_start": torch.tensor([0, T], dtype=torch.int32)}
    o, lse = _prefill(d, dev)
    of, lsef = attn.attn_causal_fwd(host["q"].to(dev), host["k"].to(dev), host["v"].to(dev))
    torch.cuda.synchronize()
    assert rel_err(o, of[0].transpose(0, 1)) <= TOL_O
    assert rel_err(lse, lsef[0].transpose(0, 1)) <= TOL_LSE


def test_prefill_poisoned_tail_and_padding(dev):
    """NaN in pool slots past each context and in the padding page changes nothing."""
    announce("prefill poison")
    d = _batch(4, 8, 2, 64, 16, [5, 0, 30, 100], [40, 17, 2, 64], seed=84)
    o, lse = _prefill(d, dev)
    kp, vp = d["k_pool"].clone(), d["v_pool"].clone()
    kp[d["poison_page"]] = float("nan")
    vp[d["poison_page"]] = float("nan")
    for s in range(4):
        n = int(d["context_lens"][s])
        last = int(d["block_table"][s, (n - 1) // 16])
        kp[last, :, (n - 1) % 16 + 1:] = float("nan")
        vp[last, :, (n - 1) % 16 + 1:] = float("nan")
    p = dict(d)
    p["k_pool"], p["v_pool"] = kp, vp
    o2, lse2 = _prefill(p, dev)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def _assert_same_state(c, m, where):
    torch.cuda.synchronize()
    fc = int(c.free_count.item())
    assert int(c.kv_status.item()) == m.status, (where, "status", int(c.kv_status.item()), m.status)
    assert fc == m.free_count, (where, "free_count")
    assert np.array_equal(c.context_lens.cpu().numpy(), m.context_lens), (where, "context_lens")
    assert np.array_equal(c.block_table.cpu().numpy(), m.block_table), (where, "block_table")
    assert np.array_equal(c.free_pages.cpu().numpy()[:fc], m.free_pages[:fc]), (where, "free stack")
    assert np.array_equal(c.k_pool.cpu().numpy(), m.k_pool), (where, "k_pool")
    assert np.array_equal(c.v_pool.cpu().numpy(), m.v_pool), (where, "v_pool")


@pytest.mark.parametrize("S,Hkv,D,ps,max_pages,num_pages", [(5, 4, 64, 16, 12, 40), (70, 2, 32, 32, 4, 150)])
def test_append_tokens_then_prefill(dev, orc, S, Hkv, D, ps, max_pages, num_pages):
    """Ragged appends (bit-exact against the model, refusals included), each followed
    by a prefill of the appended tokens over the cache (against the oracle)."""
    announce(f"append_tokens + prefill S={S} Hkv={Hkv} D={D} page={ps}")
    rng = np.random.default_rng(S + D)
    Hq = 2 * Hkv
    c = attn.PagedKvCache(S, Hkv, D, ps, max_pages, num_pages, dev)
    m = KvCacheModel(S, Hkv, D, ps, max_pages, num_pages)
    saw = set()
    for step in range(12):
        counts = rng.integers(0, 2 * ps + 5, size=S)
        counts[rng.random(S) < 0.3] = 0
        ts = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        N = int(ts[-1])
        kn = rng.standard_normal((N, Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((N, Hkv, D)).astype(np.float32)
        ts_d = torch.from_numpy(ts).to(dev)
        c.append_tokens(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev), ts_d)
        st = m.append_tokens(kn, vn, ts)
        saw.add(st)
        _assert_same_state(c, m, f"step {step}")
        if st != KV_OK:
            if step % 3 == 2:  # make room now and then
                ids = np.sort(rng.choice(S, size=max(1, S // 2), replace=False)).astype(np.int32)
                c.release(torch.from_numpy(ids).to(dev))
                m.release(ids.tolist())
                _assert_same_state(c, m, f"release {step}")
            continue
        if N == 0:
            continue
        q = rng.standard_normal((N, Hq, D)).astype(np.float32)
        o, lse = attn.attn_paged_prefill(torch.from_numpy(q).to(dev), c.k_pool, c.v_pool, c.block_table,
                                         c.context_lens, ts_d)
        torch.cuda.synchronize()
        ro, rlse = orc.paged_prefill(q, m.k_pool, m.v_pool, m.block_table, m.context_lens, ts)
        assert rel_err(o, ro) <= TOL_O and rel_err(lse, rlse) <= TOL_LSE, ("prefill after append", step)
    assert KV_OK in saw
    assert saw & {KV_POOL_EXHAUSTED, KV_SEQUENCE_FULL}, "no refused append was exercised"


def test_prefill_many_sequences(dev, orc):
    """More sequences than one wave's lanes (the block search spans several 64-sequence
    chunks), with empty ones mixed in."""
    announce("prefill S=100")
    rng = np.random.default_rng(90)
    S = 100
    cached = rng.integers(0, 200, size=S).tolist()
    new = rng.integers(0, 70, size=S).tolist()
    new[5] = 0
    new[-1] = 1
    d = _batch(S, 4, 2, 32, 16, cached, new, seed=91)
    _check(d, dev, orc)


def test_append_tokens_nothing_new(dev):
    """N = 0: every sequence adds no row; the state is unchanged and the status OK."""
    announce("append_tokens N=0")
    c = attn.PagedKvCache(3, 2, 16, 16, 2, 4, dev)
    m = KvCacheModel(3, 2, 16, 16, 2, 4)
    ts = torch.zeros((4,), dtype=torch.int32, device=dev)
    empty = torch.zeros((0, 2, 16), device=dev)
    c.append_tokens(empty, empty, ts)
    m.append_tokens(np.zeros((0, 2, 16), np.float32), np.zeros((0, 2, 16), np.float32), np.zeros(4, np.int32))
    _assert_same_state(c, m, "N=0")
