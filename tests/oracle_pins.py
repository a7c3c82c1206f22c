"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.oracle.Oracle`` and raises
AssertionError when the oracle disagrees with what the pages and the
mathematics fix:

* brute force: pure-Python scalar loops on tiny inputs, in a different form
  (no max subtraction; the backward in its per-pair scalar form with
  Delta_i = <dO_i, O_i>);
* central finite differences of L = sum(dO * O) -- the gradient check the
  riftco-transformer learn/neural_network page ("Source map") names;
* closed forms: T = 1, Q = 0 (uniform prefix averages), scale = 0, a rational
  example with known probabilities, and the page's large-logit softmax input;
* invariants: rows of P sum to one with zeros above the diagonal ("exact
  causal probabilities"), causality under perturbation and NaN poisoning of
  future keys, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, LSE bounds;
* GQA: grouped attention equals multi-head attention on repeat-interleaved K/V;
* decode: dense decode equals the last row of the causal forward, and paged
  decode equals dense decode on the gathered sequence for any page shuffle;
* prefill: each new token's row equals the causal forward's row at its position
  over the gathered sequence, brute force agrees on tiny ragged batches, and one
  new token per sequence is decode.

The mutation test (test_oracle_mutants.py) builds broken copies of the oracle
and checks that each one trips at least one of these pins.
"""
import json
import math
import os

import numpy as np
import torch

import synthetic_inputs as si

RTOL_EXACT = 1e-12


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    return float(np.max(np.abs(a - b)) / den) if a.size else 0.0


def _rand(shape, seed, std=1.0):
    r = np.random.default_rng(seed)
    return r.standard_normal(shape) * std


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------
def _brute_fwd(q, k, v, scale):
    """Scalar loops; softmax without max subtraction (inputs are small)."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, T))
    p = np.zeros((B, Hq, T, T))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                w = []
                for j in range(i + 1):
                    s = 0.0
                    for c in range(D):
                        s += q[b, h, i, c] * k[b, g, j, c]
                    w.append(math.exp(scale * s))
                z = sum(w)
                lse[b, h, i] = math.log(z)
                for j in range(i + 1):
                    p[b, h, i, j] = w[j] / z
                    for c in range(D):
                        o[b, h, i, c] += w[j] / z * v[b, g, j, c]
    return o, lse, p


def _brute_bwd(q, k, v, dout, scale):
    """dQ_i = scale sum_j P_ij (dO_i.v_j - dO_i.O_i) k_j, dK_j likewise with q_i,
    dV_j = sum_i P_ij dO_i, each summed over the query heads of a KV head."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o, _, p = _brute_fwd(q, k, v, scale)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(k.shape)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                do_o = sum(dout[b, h, i, c] * o[b, h, i, c] for c in range(D))
                for j in range(i + 1):
                    do_v = sum(dout[b, h, i, c] * v[b, g, j, c] for c in range(D))
                    w = p[b, h, i, j] * (do_v - do_o)
                    for c in range(D):
                        dq[b, h, i, c] += scale * w * k[b, g, j, c]
                        dk[b, g, j, c] += scale * w * q[b, h, i, c]
                        dv[b, g, j, c] += p[b, h, i, j] * dout[b, h, i, c]
    return dq, dk, dv


BRUTE_SHAPES = [  # (B, Hq, Hkv, T, D)
    (1, 2, 2, 16, 8),   # the 16-token, 8-wide workload's shape
    (2, 4, 2, 7, 4),    # GQA, G = 2
    (1, 4, 1, 5, 3),    # all query heads share one KV head
    (1, 3, 3, 1, 2),    # a single position
]


def pin_bruteforce_forward(orc):
    for n, (B, Hq, Hkv, T, D) in enumerate(BRUTE_SHAPES):
        q = _rand((B, Hq, T, D), 10 + n)
        k = _rand((B, Hkv, T, D), 20 + n)
        v = _rand((B, Hkv, T, D), 30 + n)
        scale = 1.0 / math.sqrt(D)
        o, lse, p = orc.causal_fwd(q, k, v, scale, return_p=True)
        bo, blse, bp = _brute_fwd(q, k, v, scale)
        assert _rel(o, bo) < RTOL_EXACT, ("O", (B, Hq, Hkv, T, D), _rel(o, bo))
        assert _rel(lse, blse) < RTOL_EXACT, ("LSE", (B, Hq, Hkv, T, D))
        assert _rel(p, bp) < RTOL_EXACT, ("P", (B, Hq, Hkv, T, D))


def pin_bruteforce_backward(orc):
    for n, (B, Hq, Hkv, T, D) in enumerate(BRUTE_SHAPES):
        q = _rand((B, Hq, T, D), 40 + n)
        k = _rand((B, Hkv, T, D), 50 + n)
        v = _rand((B, Hkv, T, D), 60 + n)
        do = _rand((B, Hq, T, D), 70 + n)
        scale = 1.0 / math.sqrt(D)
        dq, dk, dv = orc.causal_bwd(q, k, v, do, scale)
        bq, bk, bv = _brute_bwd(q, k, v, do, scale)
        for name, a, b in (("dQ", dq, bq), ("dK", dk, bk), ("dV", dv, bv)):
            assert _rel(a, b) < 1e-11, (name, (B, Hq, Hkv, T, D), _rel(a, b))


# ----------------------------------------------------------------------------
# central finite differences
# ----------------------------------------------------------------------------
def _fd_check(orc, B, Hq, Hkv, T, D, seed, tol=1e-7):
    q = _rand((B, Hq, T, D), seed)
    k = _rand((B, Hkv, T, D), seed + 1)
    v = _rand((B, Hkv, T, D), seed + 2)
    do = _rand((B, Hq, T, D), seed + 3)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = orc.causal_bwd(q, k, v, do, scale)

    def loss(qq, kk, vv):
        o, _ = orc.causal_fwd(qq, kk, vv, scale)
        return float(np.sum(do * o))

    for name, x, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
        fd = np.zeros_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            x0 = flat[idx]
            h = 1e-6 * max(1.0, abs(x0))
            flat[idx] = x0 + h
            lp = loss(q, k, v)
            flat[idx] = x0 - h
            lm = loss(q, k, v)
            flat[idx] = x0
            fd.reshape(-1)[idx] = (lp - lm) / (2 * h)
        err = _rel(grad, fd)
        assert err < tol, (name, (B, Hq, Hkv, T, D), err)


def pin_finite_differences(orc):
    _fd_check(orc, 1, 2, 2, 16, 8, seed=101)   # the 16-token, 8-wide shape
    _fd_check(orc, 1, 4, 2, 6, 4, seed=202)    # GQA, G = 2


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def pin_single_position(orc):
    """T = 1: the only key is the diagonal one, P = 1, so O = V exactly,
    LSE = scale <q, k>, dV = dO and dQ = dK = 0 (each dS row is 1*(dP - dP))."""
    q = _rand((2, 4, 1, 8), 1)
    k = _rand((2, 2, 1, 8), 2)
    v = _rand((2, 2, 1, 8), 3)
    do = _rand((2, 4, 1, 8), 4)
    scale = 0.37
    o, lse = orc.causal_fwd(q, k, v, scale)
    kv_of = np.array([0, 0, 1, 1])
    assert np.array_equal(o, v[:, kv_of]), "T=1: O must equal V exactly"
    want = scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, kv_of, 0])
    assert _rel(lse[:, :, 0], want) < RTOL_EXACT, "T=1: LSE = scale q.k"
    dq, dk, dv = orc.causal_bwd(q, k, v, do, scale)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    assert _rel(dv, do[:, [0, 2]] + do[:, [1, 3]]) < RTOL_EXACT


def _prefix_mean_expectations(q, k, v, do, scale):
    """When every score in a row is equal, P_ij = 1/(i+1) for j <= i."""
    B, Hq, T, D = q.shape
    G = Hq // k.shape[1]
    cnt = np.arange(1, T + 1, dtype=np.float64)
    o = np.zeros(q.shape)
    dq = np.zeros(q.shape)
    dv = np.zeros(k.shape)
    for h in range(Hq):
        g = h // G
        o[:, h] = np.cumsum(v[:, g], axis=1) / cnt[None, :, None]
        for i in range(T):
            w = np.einsum("bd,bjd->bj", do[:, h, i], v[:, g, : i + 1] - o[:, h, i][:, None, :])
            dq[:, h, i] = scale / (i + 1) * np.einsum("bj,bjd->bd", w, k[:, g, : i + 1])
        # dV_j = sum_{i >= j} dO_i / (i+1)
        contrib = do[:, h] / cnt[None, :, None]
        dv[:, g] += np.flip(np.cumsum(np.flip(contrib, axis=1), axis=1), axis=1)
    lse = np.broadcast_to(np.log(cnt), (B, Hq, T))
    return o, lse, dq, dv


def pin_uniform_rows(orc):
    """Q = 0 (any scale) or scale = 0 (any Q): all scores of a row are 0, so O_i is
    the mean of v_0..v_i, LSE_i = ln(i+1), dV_j = sum_{i>=j} dO_i/(i+1); dK = 0
    because every dS_ij multiplies q_i = 0 or scale = 0."""
    B, Hq, Hkv, T, D = 2, 4, 2, 9, 5
    k = _rand((B, Hkv, T, D), 5)
    v = _rand((B, Hkv, T, D), 6)
    do = _rand((B, Hq, T, D), 7)
    for q, scale in ((np.zeros((B, Hq, T, D)), 0.5), (_rand((B, Hq, T, D), 8), 0.0)):
        o, lse = orc.causal_fwd(q, k, v, scale)
        eo, else_, edq, edv = _prefix_mean_expectations(q, k, v, do, scale)
        assert _rel(o, eo) < RTOL_EXACT, "uniform rows: O = prefix mean"
        assert _rel(lse, else_) < RTOL_EXACT, "uniform rows: LSE = ln(i+1)"
        dq, dk, dv = orc.causal_bwd(q, k, v, do, scale)
        assert np.max(np.abs(dk)) < 1e-14, "uniform rows: dK = 0"
        assert _rel(dv, edv) < RTOL_EXACT, "uniform rows: dV"
        if scale == 0.0:
            assert np.max(np.abs(dq)) < 1e-14
        else:
            assert _rel(dq, edq) < 1e-11, "Q = 0: dQ closed form"


def pin_rational_example(orc):
    """d = 1, scale = 1, q_i = 1, k = (0, ln 2, ln 3): the scores of row i are
    ln(j+1), so P has rows (1), (1/3, 2/3), (1/6, 2/6, 3/6) and LSE = ln 1, ln 3,
    ln 6.  With v = (1, 2, 3): O = 1, 5/3, 7/3."""
    q = np.ones((1, 1, 3, 1))
    k = np.array([0.0, math.log(2.0), math.log(3.0)]).reshape(1, 1, 3, 1)
    v = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    o, lse, p = orc.causal_fwd(q, k, v, 1.0, return_p=True)
    ep = np.array([[1, 0, 0], [1 / 3, 2 / 3, 0], [1 / 6, 2 / 6, 3 / 6]])
    assert _rel(p[0, 0], ep) < 1e-15
    assert _rel(lse[0, 0], np.log([1.0, 3.0, 6.0])) < 1e-15
    assert _rel(o[0, 0, :, 0], [1.0, 5 / 3, 7 / 3]) < 1e-15


def pin_large_logits(orc):
    """The learn/neural_network page ("Stable softmax and cross-entropy") requires
    a finite softmax for the logits it prints (tests/golden/stable_softmax_large_logits.json);
    softmax is shift-invariant, so the last row, which sees all three, equals
    softmax(z - max z)."""
    with open(os.path.join(GOLDEN, "stable_softmax_large_logits.json")) as f:
        z = np.array(json.load(f)["logits"], dtype=np.float64)
    n = z.size
    q = np.ones((1, 1, n, 1))
    k = z.reshape(1, 1, n, 1)
    _, lse, p = orc.causal_fwd(q, k, np.zeros((1, 1, n, 1)), 1.0, return_p=True)
    e = np.exp(z - z.max())
    assert np.all(np.isfinite(p)) and np.all(np.isfinite(lse))
    assert _rel(p[0, 0, n - 1], e / e.sum()) < 1e-15
    assert abs(lse[0, 0, n - 1] - (z.max() + math.log(e.sum()))) < 1e-9


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def pin_probability_rows(orc):
    q = _rand((2, 4, 12, 6), 11)
    k = _rand((2, 2, 12, 6), 12)
    v = _rand((2, 2, 12, 6), 13)
    scale = 1.0 / math.sqrt(6)
    _, lse, p = orc.causal_fwd(q, k, v, scale, return_p=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-14, "rows of P sum to 1"
    assert np.all(np.triu(p, 1) == 0.0), "P_ij = 0 above the diagonal"
    assert np.all(p[..., np.arange(12), np.arange(12)] > 0.0), "diagonal key is kept"
    # max_j s_ij <= LSE_i <= max_j s_ij + ln(i+1)
    kv = k[:, [0, 0, 1, 1]]
    s = scale * np.einsum("bhid,bhjd->bhij", q, kv)
    s = np.where(np.tril(np.ones((12, 12), bool)), s, -np.inf)
    m = s.max(-1)
    assert np.all(lse >= m - 1e-12) and np.all(lse <= m + np.log(np.arange(1, 13)) + 1e-12)


def pin_causality(orc):
    """Rows i < s do not change, bit for bit, when K_s..., V_s... change or
    become NaN ("whole-model causality")."""
    B, Hq, Hkv, T, D = 1, 4, 2, 10, 4
    q = _rand((B, Hq, T, D), 21)
    k = _rand((B, Hkv, T, D), 22)
    v = _rand((B, Hkv, T, D), 23)
    do = _rand((B, Hq, T, D), 24)
    o, lse = orc.causal_fwd(q, k, v, 0.5)
    dq, _, _ = orc.causal_bwd(q, k, v, do, 0.5)
    for s in (1, 4, 9):
        for poison in (lambda a: a + 3.0, lambda a: a * np.nan):
            k2, v2 = k.copy(), v.copy()
            k2[:, :, s:] = poison(k2[:, :, s:])
            v2[:, :, s:] = poison(v2[:, :, s:])
            o2, lse2 = orc.causal_fwd(q, k2, v2, 0.5)
            assert np.array_equal(o2[:, :, :s], o[:, :, :s]), ("causality O", s)
            assert np.array_equal(lse2[:, :, :s], lse[:, :, :s]), ("causality LSE", s)
            dq2, _, _ = orc.causal_bwd(q, k2, v2, do, 0.5)
            assert np.array_equal(dq2[:, :, :s], dq[:, :, :s]), ("causality dQ", s)
        # changing a future row of the query must not move earlier rows either
        q2 = q.copy()
        q2[:, :, s:] += 1.0
        o3, _ = orc.causal_fwd(q2, k, v, 0.5)
        assert np.array_equal(o3[:, :, :s], o[:, :, :s])


def pin_gradient_sums(orc):
    """Each dS row sums to 0 (softmax is shift invariant), so sum_j dK_j = 0;
    sum_j P_ij = 1, so sum_j dV_j = sum over the group's heads of sum_i dO_i."""
    B, Hq, Hkv, T, D = 2, 6, 3, 11, 5
    q = _rand((B, Hq, T, D), 31)
    k = _rand((B, Hkv, T, D), 32)
    v = _rand((B, Hkv, T, D), 33)
    do = _rand((B, Hq, T, D), 34)
    dq, dk, dv = orc.causal_bwd(q, k, v, do, 0.4)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(dk)))
    want = do.sum(axis=2).reshape(B, Hkv, Hq // Hkv, D).sum(axis=2)
    assert _rel(dv.sum(axis=2), want) < 1e-13


def pin_gqa_identity(orc):
    """GQA(Q, K, V) = MHA(Q, repeat_interleave(K, G), repeat_interleave(V, G));
    dK, dV of GQA are the per-group sums of the MHA ones (query heads
    g*G .. g*G+G-1 share KV head g)."""
    B, Hq, Hkv, T, D = 2, 8, 2, 9, 4
    G = Hq // Hkv
    q = _rand((B, Hq, T, D), 41)
    k = _rand((B, Hkv, T, D), 42)
    v = _rand((B, Hkv, T, D), 43)
    do = _rand((B, Hq, T, D), 44)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse = orc.causal_fwd(q, k, v, 0.5)
    om, lsem = orc.causal_fwd(q, kr, vr, 0.5)
    assert np.array_equal(o, om) and np.array_equal(lse, lsem)
    dq, dk, dv = orc.causal_bwd(q, k, v, do, 0.5)
    dqm, dkm, dvm = orc.causal_bwd(q, kr, vr, do, 0.5)
    assert _rel(dq, dqm) < RTOL_EXACT
    assert _rel(dk, dkm.reshape(B, Hkv, G, T, D).sum(2)) < RTOL_EXACT
    assert _rel(dv, dvm.reshape(B, Hkv, G, T, D).sum(2)) < RTOL_EXACT


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def pin_decode_is_last_causal_row(orc):
    """A single query attending to n cached positions is the last row of the
    causal forward over those positions with the query placed at row n-1."""
    for (Hq, Hkv, n, D, seed) in ((4, 4, 13, 8, 51), (8, 2, 20, 4, 52), (3, 1, 1, 5, 53)):
        qd = _rand((Hq, D), seed)
        kseq = _rand((n, Hkv, D), seed + 1)
        vseq = _rand((n, Hkv, D), seed + 2)
        o, lse = orc.decode_dense(qd, kseq, vseq, 0.3)
        qc = _rand((1, Hq, n, D), seed + 3)
        qc[0, :, n - 1] = qd
        kc = np.transpose(kseq, (1, 0, 2))[None]
        vc = np.transpose(vseq, (1, 0, 2))[None]
        oc, lsec = orc.causal_fwd(qc, kc, vc, 0.3)
        assert _rel(o, oc[0, :, n - 1]) < RTOL_EXACT, ("decode vs causal row", Hq, Hkv, n)
        assert _rel(lse, lsec[0, :, n - 1]) < RTOL_EXACT


def pin_paged_equals_dense(orc):
    """Paged decode equals dense decode on the sequence gathered through the
    block table, and does not depend on where the pages sit in the pool."""
    for seed, shuffle in ((61, True), (62, False)):
        d = si.paged_decode_inputs(S=5, Hq=4, Hkv=2, D=8, page_size=4, ctx_lo=1, ctx_hi=23,
                                   max_pages=6, seed=seed, pool_shuffle=shuffle)
        o, lse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                  d["context_lens"], 0.35)
        for s in range(5):
            kseq, vseq = si.gather_sequence(d["k_pool"], d["v_pool"], d["block_table"],
                                            d["context_lens"], s, 4)
            od, lsed = orc.decode_dense(d["q"][s], kseq, vseq, 0.35)
            assert np.array_equal(o[s], od) and np.array_equal(lse[s], lsed), ("paged", s)
    # re-permute the pool: same logical sequences, different physical pages
    d = si.paged_decode_inputs(S=4, Hq=8, Hkv=2, D=4, page_size=4, ctx_lo=3, ctx_hi=24,
                               max_pages=6, seed=63)
    o, lse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                              d["context_lens"], 0.5)
    P = d["num_pages"]
    rng = np.random.default_rng(64)
    perm = rng.permutation(P)            # new physical page of old page p is perm[p]
    kp = np.empty_like(d["k_pool"].numpy())
    vp = np.empty_like(kp)
    kp[perm] = d["k_pool"].numpy()
    vp[perm] = d["v_pool"].numpy()
    bt = perm[d["block_table"].numpy()].astype(np.int32)
    o2, lse2 = orc.paged_decode(d["q"], kp, vp, bt, d["context_lens"], 0.5)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "pool permutation"
    # positions past the context (in the last page and in the padding page) are not read
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[perm[d["poison_page"]]] = np.nan
    vp2[perm[d["poison_page"]]] = np.nan
    ctx = d["context_lens"].numpy()
    for s in range(4):
        n = int(ctx[s])
        last = bt[s, (n - 1) // 4]
        kp2[last, :, (n - 1) % 4 + 1:] = np.nan
        vp2[last, :, (n - 1) % 4 + 1:] = np.nan
    o3, lse3 = orc.paged_decode(d["q"], kp2, vp2, bt, d["context_lens"], 0.5)
    assert np.array_equal(o3, o2) and np.array_equal(lse3, lse2), "poisoned tail/padding"


# ----------------------------------------------------------------------------
# batched prefill over a paged cache
# ----------------------------------------------------------------------------
def _prefill_case(S, Hq, Hkv, D, ps, cached, new, seed):
    """A ragged batch whose new tokens are the last rows of a full per-sequence Q."""
    ctx = [c + n for c, n in zip(cached, new)]
    maxp = max(1, max(-(-c // ps) for c in ctx))
    rng = np.random.default_rng(seed)
    n_pages = [-(-c // ps) for c in ctx]
    total = sum(n_pages)
    perm = rng.permutation(total)
    bt = np.full((S, maxp + 1), total, dtype=np.int32)
    off = 0
    for s in range(S):
        bt[s, :n_pages[s]] = perm[off:off + n_pages[s]]
        off += n_pages[s]
    kp = rng.standard_normal((total + 1, Hkv, ps, D))
    vp = rng.standard_normal((total + 1, Hkv, ps, D))
    qfull = [rng.standard_normal((c, Hq, D)) for c in ctx]
    q = np.concatenate([qf[c - n:] for qf, c, n in zip(qfull, ctx, new)], 0) if sum(new) else np.zeros((0, Hq, D))
    ts = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    return q, kp, vp, bt, np.array(ctx, dtype=np.int32), ts, qfull


def pin_prefill_rows_are_causal_rows(orc):
    """Token j of sequence s (position t = ctx - n + j) gets the causal forward's
    row t over the sequence gathered through its table, O and LSE."""
    for (S, Hq, Hkv, D, ps, cached, new, seed) in (
            (3, 4, 2, 8, 4, [0, 5, 9], [6, 3, 4], 71),
            (4, 2, 2, 5, 8, [17, 0, 1, 30], [2, 9, 0, 1], 72),
            (2, 6, 1, 4, 4, [3, 0], [1, 13], 73)):
        q, kp, vp, bt, ctx, ts, qfull = _prefill_case(S, Hq, Hkv, D, ps, cached, new, seed)
        o, lse = orc.paged_prefill(q, kp, vp, bt, ctx, ts, 0.4)
        for s in range(S):
            n = new[s]
            if n == 0:
                continue
            kseq, vseq = si.gather_sequence(torch.from_numpy(kp), torch.from_numpy(vp), torch.from_numpy(bt),
                                            torch.from_numpy(ctx), s, ps)
            qc = np.transpose(qfull[s], (1, 0, 2))[None]
            kc = np.transpose(kseq.numpy(), (1, 0, 2))[None]
            vc = np.transpose(vseq.numpy(), (1, 0, 2))[None]
            oc, lsec = orc.causal_fwd(qc, kc, vc, 0.4)
            c = int(ctx[s])
            rows = slice(int(ts[s]), int(ts[s + 1]))
            assert _rel(o[rows], np.transpose(oc[0, :, c - n:], (1, 0, 2))) < RTOL_EXACT, ("prefill row", s)
            assert _rel(lse[rows], lsec[0, :, c - n:].T) < RTOL_EXACT, ("prefill lse", s)


def pin_prefill_bruteforce(orc):
    """Scalar loops: every new token sums exp(scale q.k) over the positions up to its
    own (no max subtraction), read through the table one position at a time."""
    S, Hq, Hkv, D, ps = 3, 4, 2, 3, 4
    cached, new = [2, 0, 6], [3, 5, 1]
    q, kp, vp, bt, ctx, ts, _ = _prefill_case(S, Hq, Hkv, D, ps, cached, new, 74)
    o, lse = orc.paged_prefill(q, kp, vp, bt, ctx, ts, 0.7)
    G = Hq // Hkv
    for s in range(S):
        for j in range(new[s]):
            row = int(ts[s]) + j
            t = int(ctx[s]) - new[s] + j
            for h in range(Hq):
                g = h // G
                w, vals = [], []
                for pos in range(t + 1):
                    page = int(bt[s, pos // ps])
                    kr = kp[page, g, pos % ps]
                    w.append(math.exp(0.7 * sum(q[row, h, c] * kr[c] for c in range(D))))
                    vals.append(vp[page, g, pos % ps])
                z = sum(w)
                assert abs(lse[row, h] - math.log(z)) < 1e-12 * max(1.0, abs(math.log(z)))
                for c in range(D):
                    ref = sum(wi * vi[c] for wi, vi in zip(w, vals)) / z
                    assert abs(o[row, h, c] - ref) < 1e-12, ("prefill brute", s, j, h, c)


def pin_prefill_single_tokens_are_decode(orc):
    """One new token per sequence: prefill and paged decode give the same rows."""
    d = si.paged_decode_inputs(S=5, Hq=4, Hkv=2, D=8, page_size=4, ctx_lo=1, ctx_hi=23, max_pages=6, seed=75)
    o, lse = orc.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], 0.35)
    ts = np.arange(6, dtype=np.int32)
    op, lsep = orc.paged_prefill(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"], ts, 0.35)
    assert np.array_equal(o, op) and np.array_equal(lse, lsep)


ALL_PINS = [
    pin_bruteforce_forward,
    pin_bruteforce_backward,
    pin_finite_differences,
    pin_single_position,
    pin_uniform_rows,
    pin_rational_example,
    pin_large_logits,
    pin_probability_rows,
    pin_causality,
    pin_gradient_sums,
    pin_gqa_identity,
    pin_decode_is_last_causal_row,
    pin_paged_equals_dense,
    pin_prefill_rows_are_causal_rows,
    pin_prefill_bruteforce,
    pin_prefill_single_tokens_are_decode,
]
