"""Materialized causal attention and its VJP with a cotangent on the
probabilities (test infrastructure only; only ``tests/`` may use this module).

What it follows: "Architecture", "Intentional limits" and "Execution Backends
and the Python ABI", "What the Metal slice does" -- the materialized path forms
the [B,H,T,T] probabilities, returns them with the context and keeps them for
the VJPs; "Architecture", "Tensor conventions" -- key t_k is excluded from query
t_q when t_k > t_q.  For the loss L = sum(dO * O) + sum(dPx * P), with
P = softmax_j(scale Q K^T masked) and O = P V, the chain rule gives
  dV = P^T dO,  dP = dO V^T + dPx,  dS_ij = P_ij (dP_ij - sum_l P_il dP_il),
  dQ = scale dS K,  dK = scale dS^T Q,
with dK, dV summed over the query heads that share a key/value head
(learn/neural_network, "Layer normalization": a broadcast input's gradient is
reduced back to its shape).  Plain float64 numpy, one (batch, head) at a time.
"""
import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def probabilities(q, k, scale):
    """P [B,Hq,T,T] of the masked, scaled scores (rows sum to 1, zeros above the diagonal)."""
    q, k = _f64(q), _f64(k)
    B, Hq, T, _ = q.shape
    G = Hq // k.shape[1]
    mask = np.triu(np.ones((T, T), dtype=bool), 1)  # j > i
    p = np.zeros((B, Hq, T, T))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // G].T)
            s[mask] = -np.inf
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p[b, h] = e / e.sum(axis=1, keepdims=True)
    return p


def forward(q, k, v, scale):
    """(O, P) of the materialized path."""
    v = _f64(v)
    p = probabilities(q, k, scale)
    B, Hq = p.shape[:2]
    G = Hq // v.shape[1]
    o = np.stack([np.stack([p[b, h] @ v[b, h // G] for h in range(Hq)]) for b in range(B)])
    return o, p


def backward(q, k, v, dout, dpx, scale):
    """(dQ, dK, dV) of L = sum(dout * O) + sum(dpx * P); dpx may be None."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    p = probabilities(q, k, scale)
    dpx = None if dpx is None else _f64(dpx)
    B, Hq, T, _ = q.shape
    G = Hq // k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            P = p[b, h]
            dv[b, g] += P.T @ dout[b, h]
            dP = dout[b, h] @ v[b, g].T
            if dpx is not None:
                dP = dP + dpx[b, h]
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ k[b, g])
            dk[b, g] += scale * (dS.T @ q[b, h])
    return dq, dk, dv
