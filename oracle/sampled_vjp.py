"""Single outputs of the causal attention VJP, each from its definition (test
infrastructure only; only ``tests/`` may use this module).

For the long-context sizes the full oracle cannot hold a [T,T] matrix per head in
seconds, so the tests compare the GPU's gradients there on sampled rows of dQ and
sampled key positions of dK, dV, each computed here on its own.

What is computed ("Execution Backends and the Python ABI", "What the Metal slice
does": the backward recomputes the probabilities from Q and K; "Architecture",
"Tensor conventions": key t_k is excluded from query t_q when t_k > t_q;
learn/neural_network, "Layer normalization": a broadcast input's gradient is
summed back to its own shape, here over the query heads sharing a key/value
head).  For query head h, query row i and its key/value head g = h // (Hq/Hkv):
  s_ij  = scale * q_hi . k_gj              (j <= i)
  P_ij  = exp(s_ij) / sum_{l <= i} exp(s_il)
  dP_ij = dO_hi . v_gj
  dS_ij = P_ij * (dP_ij - sum_{l <= i} P_il dP_il)
  dQ_hi = scale * sum_{j <= i} dS_ij k_gj
  dK_gj = scale * sum_{h in g} sum_{i >= j} dS_ij q_hi
  dV_gj = sum_{h in g} sum_{i >= j} P_ij dO_hi
Everything is float64 numpy, one query row at a time; the row's softmax is taken
after subtracting its maximum (the same value, without overflow).
"""
import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _row(q, k, v, dout, h, i, G, scale):
    """P_i., dS_i. over keys 0..i of query head h, row i."""
    g = h // G
    s = scale * (k[g, :i + 1] @ q[h, i])
    e = np.exp(s - s.max())
    p = e / e.sum()
    dp = v[g, :i + 1] @ dout[h, i]
    ds = p * (dp - p @ dp)
    return p, ds


def dq_rows(q, k, v, dout, rows, scale):
    """dQ[h, i] for every query head h and each i in rows: [Hq, len(rows), D].
    q, dout [Hq, T, D]; k, v [Hkv, T, D] (one batch element)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Hq, T, D = q.shape
    G = Hq // k.shape[0]
    out = np.zeros((Hq, len(rows), D))
    for h in range(Hq):
        for n, i in enumerate(rows):
            _, ds = _row(q, k, v, dout, h, i, G, scale)
            out[h, n] = scale * (ds @ k[h // G, :i + 1])
    return out


def dkv_cols(q, k, v, dout, cols, scale):
    """dK[g, j], dV[g, j] for every key/value head g and each key position j in
    cols: two arrays [Hkv, len(cols), D].  Visits the query rows i >= min(cols)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Hq, T, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    cols = list(cols)
    dk = np.zeros((Hkv, len(cols), D))
    dv = np.zeros((Hkv, len(cols), D))
    for h in range(Hq):
        g = h // G
        for i in range(min(cols), T):
            p, ds = _row(q, k, v, dout, h, i, G, scale)
            for n, j in enumerate(cols):
                if j <= i:
                    dk[g, n] += scale * ds[j] * q[h, i]
                    dv[g, n] += p[j] * dout[h, i]
    return dk, dv
