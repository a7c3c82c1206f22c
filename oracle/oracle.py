"""ctypes front-end of the CPU oracle (test infrastructure only).

Wraps ``liboracle.so`` built from ``attn_oracle.c``.  Inputs may be numpy
arrays or CPU torch tensors of any float dtype; they are converted to float64
(exact for fp32 data) and every result comes back as float64 numpy arrays.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use this module.
"""
import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a, kind=_dp):
    return a.ctypes.data_as(kind) if a is not None else None


class Oracle:
    """One loaded copy of the oracle library (tests may load a mutated build)."""

    def __init__(self, lib_path: str = DEFAULT_LIB):
        if not os.path.exists(lib_path):
            raise FileNotFoundError(f"{lib_path} is missing; run oracle/build.py first")
        lib = ctypes.CDLL(lib_path)
        lib.oracle_causal_fwd.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_double, _dp, _dp, _dp]
        lib.oracle_causal_bwd.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_double, _dp, _dp, _dp]
        lib.oracle_decode_dense.argtypes = [_dp, _dp, _dp, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, _dp, _dp]
        lib.oracle_paged_decode.argtypes = [_dp, _dp, _dp, _ip, _ip, _i64, _i64, _i64, _i64,
                                            _i64, _i64, _i64, ctypes.c_double, _dp, _dp]
        lib.oracle_paged_prefill.argtypes = [_dp, _dp, _dp, _ip, _ip, _ip, _i64, _i64, _i64, _i64, _i64,
                                             _i64, _i64, _i64, ctypes.c_double, _dp, _dp]
        for fn in ("oracle_causal_fwd", "oracle_causal_bwd", "oracle_decode_dense",
                   "oracle_paged_decode", "oracle_paged_prefill", "oracle_num_threads"):
            getattr(lib, fn).restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    @staticmethod
    def _shapes(q, k):
        B, Hq, T, D = q.shape
        Bk, Hkv, Tk, Dk = k.shape
        if (Bk, Tk, Dk) != (B, T, D) or Hq % Hkv != 0:
            raise ValueError(f"incompatible shapes q{q.shape} k{k.shape}")
        return B, Hq, Hkv, T, D

    def causal_fwd(self, q, k, v, scale=None, return_p=False):
        """O [B,Hq,T,D], LSE [B,Hq,T] (and P [B,Hq,T,T] if asked), float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, T, D = self._shapes(q, k)
        if v.shape != k.shape:
            raise ValueError("v must have k's shape")
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        o = np.empty((B, Hq, T, D))
        lse = np.empty((B, Hq, T))
        p = np.empty((B, Hq, T, T)) if return_p else None
        rc = self.lib.oracle_causal_fwd(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, T, D, scale,
                                        _ptr(o), _ptr(lse), _ptr(p))
        if rc != 0:
            raise RuntimeError("oracle_causal_fwd failed")
        return (o, lse, p) if return_p else (o, lse)

    def causal_bwd(self, q, k, v, dout, scale=None):
        """dQ [B,Hq,T,D], dK, dV [B,Hkv,T,D] of L = sum(dout * O), float64."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, T, D = self._shapes(q, k)
        if dout.shape != q.shape or v.shape != k.shape:
            raise ValueError("dout must have q's shape and v k's shape")
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(k)
        rc = self.lib.oracle_causal_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, Hq, Hkv, T, D,
                                        scale, _ptr(dq), _ptr(dk), _ptr(dv))
        if rc != 0:
            raise RuntimeError("oracle_causal_bwd failed")
        return dq, dk, dv

    def decode_dense(self, q, kseq, vseq, scale=None):
        """One sequence: q [Hq,D]; kseq, vseq [n,Hkv,D] -> O [Hq,D], LSE [Hq]."""
        q, kseq, vseq = _f64(q), _f64(kseq), _f64(vseq)
        Hq, D = q.shape
        n, Hkv, Dk = kseq.shape
        if Dk != D or vseq.shape != kseq.shape:
            raise ValueError("incompatible shapes")
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        o = np.empty((Hq, D))
        lse = np.empty((Hq,))
        rc = self.lib.oracle_decode_dense(_ptr(q), _ptr(kseq), _ptr(vseq), n, Hq, Hkv, D, scale,
                                          _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError("oracle_decode_dense failed")
        return o, lse

    def paged_decode(self, q, k_pool, v_pool, block_table, context_lens, scale=None):
        """q [S,Hq,D]; pools [P,Hkv,page,D]; block_table [S,maxp]; ctx [S]."""
        q, k_pool, v_pool = _f64(q), _f64(k_pool), _f64(v_pool)
        bt, ctx = _i32(block_table), _i32(context_lens)
        S, Hq, D = q.shape
        P, Hkv, page, Dk = k_pool.shape
        if Dk != D or v_pool.shape != k_pool.shape or bt.shape[0] != S or ctx.shape != (S,):
            raise ValueError("incompatible shapes")
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        o = np.empty((S, Hq, D))
        lse = np.empty((S, Hq))
        rc = self.lib.oracle_paged_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(bt, _ip),
                                          _ptr(ctx, _ip), S, Hq, Hkv, D, page, bt.shape[1], P,
                                          scale, _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError("oracle_paged_decode failed (bad length or page index?)")
        return o, lse


    def paged_prefill(self, q, k_pool, v_pool, block_table, context_lens, token_start, scale=None):
        """q [N,Hq,D]; pools [P,Hkv,page,D]; block_table [S,maxp]; ctx [S]; token_start [S+1]."""
        q, k_pool, v_pool = _f64(q), _f64(k_pool), _f64(v_pool)
        bt, ctx, ts = _i32(block_table), _i32(context_lens), _i32(token_start)
        N, Hq, D = q.shape
        P, Hkv, page, Dk = k_pool.shape
        S = bt.shape[0]
        if Dk != D or v_pool.shape != k_pool.shape or ctx.shape != (S,) or ts.shape != (S + 1,):
            raise ValueError("incompatible shapes")
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        o = np.zeros((N, Hq, D))
        lse = np.zeros((N, Hq))
        rc = self.lib.oracle_paged_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(bt, _ip), _ptr(ctx, _ip),
                                           _ptr(ts, _ip), S, N, Hq, Hkv, D, page, bt.shape[1], P, scale,
                                           _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError("oracle_paged_prefill failed (bad table, length or page index?)")
        return o, lse


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def causal_fwd(*a, **kw):
    return default().causal_fwd(*a, **kw)


def causal_bwd(*a, **kw):
    return default().causal_bwd(*a, **kw)


def decode_dense(*a, **kw):
    return default().decode_dense(*a, **kw)


def paged_decode(*a, **kw):
    return default().paged_decode(*a, **kw)


def paged_prefill(*a, **kw):
    return default().paged_prefill(*a, **kw)
