"""Thin Python binding of libattn.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI; this
module only checks tensors, allocates outputs and workspaces with torch on the
inputs' device, and passes raw device pointers plus the current HIP stream.
There is no fallback: if the library is missing, loading fails loudly.

Same names as the C entry points (see include/attn.h).  Native failures raise
AttnError carrying the status code and the library's thread-local message, in
the manner of the Python client on "Execution Backends and the Python ABI",
"Python client".
"""
import contextlib
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIBRARY = os.path.join(HERE, "libattn.so")

ATTN_OK = 0
ATTN_INVALID_ARGUMENT = 1
ATTN_UNSUPPORTED = 2
ATTN_WORKSPACE_TOO_SMALL = 3
ATTN_DEVICE_ERROR = 4
ATTN_ABI_VERSION = 0x00010004

ATTN_KV_OK = 0
ATTN_KV_POOL_EXHAUSTED = 1
ATTN_KV_SEQUENCE_FULL = 2
ATTN_KV_STACK_OVERFLOW = 3

STATUS_NAMES = {
    ATTN_OK: "ATTN_OK",
    ATTN_INVALID_ARGUMENT: "ATTN_INVALID_ARGUMENT",
    ATTN_UNSUPPORTED: "ATTN_UNSUPPORTED",
    ATTN_WORKSPACE_TOO_SMALL: "ATTN_WORKSPACE_TOO_SMALL",
    ATTN_DEVICE_ERROR: "ATTN_DEVICE_ERROR",
}

# name -> (restype, argtypes); mirrors include/attn.h
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f = ctypes.c_float
_sz = ctypes.c_size_t
_st = ctypes.c_int32
SIGNATURES = {
    "attn_abi_version": (ctypes.c_uint32, []),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_causal_fwd": (_st, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f, _vp, _vp, _vp]),
    "attn_causal_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "attn_causal_bwd": (_st, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f,
                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "attn_paged_decode_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "attn_paged_decode": (_st, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                _f, _vp, _vp, _vp, _sz, _vp]),
    "attn_paged_decode_noalloc": (_st, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                        _f, _vp, _vp, _vp]),
    "attn_materialized_fwd": (_st, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f, _vp, _vp, _vp, _vp]),
    "attn_materialized_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "attn_materialized_bwd": (_st, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f,
                                    _vp, _vp, _vp, _vp, _sz, _vp]),
    "attn_kv_append": (_st, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp]),
    "attn_kv_release": (_st, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "attn_kv_append_tokens": (_st, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp]),
    "attn_paged_prefill": (_st, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _f, _vp, _vp, _vp]),
}


class AttnError(RuntimeError):
    def __init__(self, status, message):
        self.status = int(status)
        self.message = message
        super().__init__(f"{STATUS_NAMES.get(self.status, self.status)}: {message}")


_lib = None


def library_path() -> str:
    return os.environ.get("ATTN_LIBRARY", DEFAULT_LIBRARY)


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with causal_self_attention_amd/build.py "
                              "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.attn_abi_version() >> 16 != ATTN_ABI_VERSION >> 16:
            raise ImportError(f"{path}: ABI major mismatch ({handle.attn_abi_version():#x})")
        _lib = handle
    return _lib


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, lib().attn_last_error().decode(errors="replace"))


def _stream_ptr(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream, *given):
    """Context for the tensors this module allocates for a call (outputs and
    workspace): with an explicit stream they are allocated while that stream is
    current, so torch's caching allocator hands their memory to later allocations
    only in that stream's order -- after the call's kernels -- even when the
    workspace is dropped as soon as the call returns.  When the caller passed every
    buffer (`given` holds them; None marks one to allocate) nothing is allocated,
    and the stream switch, which costs microseconds of host time, is skipped."""
    if stream is None or all(t is not None for t in given):
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _dev(t, name, dtype=torch.float32):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _given(t, shape, name):
    """A caller-provided output must have exactly the shape the call writes: the C ABI
    takes only its pointer and writes as many elements as the inputs' sizes imply."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _causal_shapes(q, k, v):
    """B, Hq, Hkv, T, D of q [B,Hq,T,D] and k, v [B,Hkv,T,D]."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"expected q [B,Hq,T,D], k/v [B,Hkv,T,D]; got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Hq, T, D = q.shape
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return B, Hq, k.shape[1], T, D


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def attn_abi_version() -> int:
    return int(lib().attn_abi_version())


def attn_last_error() -> str:
    return lib().attn_last_error().decode(errors="replace")


def attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D) -> int:
    return int(lib().attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D))


def attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages_per_seq) -> int:
    return int(lib().attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages_per_seq))


def attn_causal_fwd(q, k, v, scale=None, o=None, lse=None, stream=None):
    """O [B,Hq,T,D] and LSE [B,Hq,T] of causal attention (async on the stream)."""
    dev = _same_device(q, k, v)
    B, Hq, Hkv, T, D = _causal_shapes(q, k, v)
    _given(o, q.shape, "o")
    _given(lse, (B, Hq, T), "lse")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with _alloc_on(stream, o, lse):
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq, T), device=dev, dtype=torch.float32)
    _check(lib().attn_causal_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, T, D, scale,
                                 _dev(o, "o"), _dev(lse, "lse"), _stream_ptr(stream, dev)))
    return o, lse


def attn_causal_bwd(q, k, v, o, lse, dout, scale=None, dq=None, dk=None, dv=None, workspace=None,
                    stream=None):
    """(dQ, dK, dV) of the loss sum(dout * O) (async on the stream)."""
    dev = _same_device(q, k, v, o, lse, dout)
    B, Hq, Hkv, T, D = _causal_shapes(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (B, Hq, T):
        raise ValueError("shape mismatch among q, k, v, o, lse, dout")
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _given(t, ref.shape, name)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    need = attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D)
    with _alloc_on(stream, dq, dk, dv, workspace):
        if dq is None:
            dq = torch.empty_like(q)
        if dk is None:
            dk = torch.empty_like(k)
        if dv is None:
            dv = torch.empty_like(v)
        if workspace is None:
            workspace = torch.empty((max(need, 256) // 4,), device=dev, dtype=torch.float32)
    _check(lib().attn_causal_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(lse, "lse"),
                                 _dev(dout, "dout"), B, Hq, Hkv, T, D, scale, _dev(dq, "dq"),
                                 _dev(dk, "dk"), _dev(dv, "dv"), _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev)))
    return dq, dk, dv


def attn_paged_decode(q, k_pool, v_pool, block_table, context_lens, scale=None, o=None, lse=None,
                      workspace=None, stream=None, with_lse=True):
    """O [S,Hq,D] (and LSE [S,Hq]) of one query token per sequence over a paged cache."""
    dev = _same_device(q, k_pool, v_pool, block_table, context_lens)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [S,Hq,D] and pools [num_pages,Hkv,page_size,D]")
    S, Hq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_pool.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("shape mismatch among q, pools, block_table, context_lens")
    max_pages = block_table.shape[1]
    _given(o, q.shape, "o")
    _given(lse, (S, Hq), "lse")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    need = attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages)
    with _alloc_on(stream, o, lse if with_lse else o, workspace):
        if o is None:
            o = torch.empty_like(q)
        if with_lse and lse is None:
            lse = torch.empty((S, Hq), device=dev, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty((max(need, 256) // 4,), device=dev, dtype=torch.float32)
    lse_p = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    _check(lib().attn_paged_decode(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                   _dev(block_table, "block_table", torch.int32),
                                   _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D,
                                   page_size, max_pages, num_pages, scale, _dev(o, "o"), lse_p,
                                   _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(),
                                   _stream_ptr(stream, dev)))
    return o, lse


class PreparedPagedDecode:
    """attn_paged_decode with its arguments checked and marshalled once: each call
    re-issues the C call on the same tensors (their contents may change between calls,
    their storage may not), for loops where the per-call Python checks would cost more
    host time than the kernels take (a 30 us decode issued back to back).  The tensors
    are kept alive by this object; `o` and `lse` hold each call's results."""

    def __init__(self, q, k_pool, v_pool, block_table, context_lens, scale=None, o=None, lse=None,
                 workspace=None, stream=None, with_lse=True):
        dev = _same_device(q, k_pool, v_pool, block_table, context_lens)
        if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
            raise ValueError("expected q [S,Hq,D] and pools [num_pages,Hkv,page_size,D]")
        S, Hq, D = q.shape
        num_pages, Hkv, page_size, Dk = k_pool.shape
        if Dk != D or block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
            raise ValueError("shape mismatch among q, pools, block_table, context_lens")
        max_pages = block_table.shape[1]
        scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
        need = attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages)
        with _alloc_on(stream, o, lse if with_lse else o, workspace):
            if o is None:
                o = torch.empty_like(q)
            if with_lse and lse is None:
                lse = torch.empty((S, Hq), device=dev, dtype=torch.float32)
            if workspace is None:
                workspace = torch.empty((max(need, 256) // 4,), device=dev, dtype=torch.float32)
        _given(o, q.shape, "o")
        _given(lse, (S, Hq), "lse")
        lse_p = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
        self.o, self.lse = o, lse
        self._keep = (q, k_pool, v_pool, block_table, context_lens, workspace)
        self._fn = lib().attn_paged_decode
        self._args = (_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                      _dev(block_table, "block_table", torch.int32), _dev(context_lens, "context_lens", torch.int32),
                      S, Hq, Hkv, D, page_size, max_pages, num_pages, scale, _dev(o, "o"), lse_p,
                      _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                      _stream_ptr(stream, dev))

    def __call__(self):
        _check(self._fn(*self._args))
        return self.o, self.lse


ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def attn_paged_decode_noalloc(q, k_pool, v_pool, block_table, context_lens, o, lse=None, scale=None, stream=None):
    """attn_paged_decode with no workspace: the library's static per-GPU scratch holds
    the partial results, and nothing is allocated, here or in the library (the caller
    passes the outputs o [S,Hq,D] and, optionally, lse [S,Hq]).  Calls on one GPU share
    that scratch, so overlapping calls race."""
    _same_device(q, k_pool, v_pool, block_table, context_lens, o)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [S,Hq,D] and pools [num_pages,Hkv,page_size,D]")
    S, Hq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_pool.shape
    if Dk != D or block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("shape mismatch among q, pools, block_table, context_lens")
    _given(o, q.shape, "o")
    _given(lse, (S, Hq), "lse")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lse_p = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    _check(lib().attn_paged_decode_noalloc(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                           _dev(block_table, "block_table", torch.int32),
                                           _dev(context_lens, "context_lens", torch.int32), S, Hq, Hkv, D,
                                           page_size, block_table.shape[1], num_pages, scale, _dev(o, "o"), lse_p,
                                           _stream_ptr(stream, q.device)))
    return o, lse


def attn_materialized_bwd_workspace_bytes(B, Hq, Hkv, T, D) -> int:
    return int(lib().attn_materialized_bwd_workspace_bytes(B, Hq, Hkv, T, D))


def attn_materialized_fwd(q, k, v, scale=None, o=None, lse=None, p=None, stream=None):
    """O [B,Hq,T,D], LSE [B,Hq,T] and the probabilities P [B,Hq,T,T] (async)."""
    dev = _same_device(q, k, v)
    B, Hq, Hkv, T, D = _causal_shapes(q, k, v)
    _given(o, q.shape, "o")
    _given(lse, (B, Hq, T), "lse")
    _given(p, (B, Hq, T, T), "p")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with _alloc_on(stream, o, lse, p):
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, Hq, T), device=dev, dtype=torch.float32)
        if p is None:
            p = torch.empty((B, Hq, T, T), device=dev, dtype=torch.float32)
    _check(lib().attn_materialized_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, T, D, scale,
                                       _dev(o, "o"), _dev(lse, "lse"), _dev(p, "p"), _stream_ptr(stream, dev)))
    return o, lse, p


def attn_materialized_bwd(q, k, v, o, p, dout, dp=None, scale=None, dq=None, dk=None, dv=None, workspace=None,
                          stream=None):
    """(dQ, dK, dV) of sum(dout * O) + sum(dp * P) using the stored probabilities p (async)."""
    dev = _same_device(q, k, v, o, p, dout)
    B, Hq, Hkv, T, D = _causal_shapes(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if p.shape != (B, Hq, T, T) or (dp is not None and dp.shape != p.shape):
        raise ValueError("p (and dp) must be [B, Hq, T, T]")
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _given(t, ref.shape, name)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    need = attn_materialized_bwd_workspace_bytes(B, Hq, Hkv, T, D)
    with _alloc_on(stream, dq, dk, dv, workspace):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        if workspace is None:
            workspace = torch.empty((max(need, 256) // 4,), device=dev, dtype=torch.float32)
    dp_p = _dev(dp, "dp") if dp is not None else ctypes.c_void_p(0)
    _check(lib().attn_materialized_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(p, "p"),
                                       _dev(dout, "dout"), dp_p, B, Hq, Hkv, T, D, scale, _dev(dq, "dq"),
                                       _dev(dk, "dk"), _dev(dv, "dv"), _dev(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev)))
    return dq, dk, dv


class PagedKvCache:
    """Device state of one layer's paged K/V cache (tensors only; every update runs
    in attn_kv_append / attn_kv_release).

    k_pool, v_pool [num_pages, Hkv, page_size, D]; block_table [S, max_pages] and
    context_lens [S] int32; free_pages [num_pages] int32 with free_count [1] (the
    free-page stack, top at free_count - 1); kv_status [1] int32.  Starts empty:
    every page free (the stack holds num_pages-1 .. 0, so page 0 is leased first),
    every length 0.
    """

    def __init__(self, S, Hkv, D, page_size, max_pages, num_pages, device):
        f32, i32 = torch.float32, torch.int32
        self.S, self.Hkv, self.D = int(S), int(Hkv), int(D)
        self.page_size, self.max_pages, self.num_pages = int(page_size), int(max_pages), int(num_pages)
        self.k_pool = torch.zeros((num_pages, Hkv, page_size, D), device=device, dtype=f32)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.block_table = torch.zeros((S, max_pages), device=device, dtype=i32)
        self.context_lens = torch.zeros((S,), device=device, dtype=i32)
        self.free_pages = torch.arange(num_pages - 1, -1, -1, device=device, dtype=i32)
        self.free_count = torch.full((1,), num_pages, device=device, dtype=i32)
        self.kv_status = torch.zeros((1,), device=device, dtype=i32)

    def append(self, k_new, v_new, stream=None):
        attn_kv_append(k_new, v_new, self, stream=stream)

    def append_tokens(self, k_new, v_new, token_start, stream=None):
        attn_kv_append_tokens(k_new, v_new, token_start, self, stream=stream)

    def release(self, seq_ids, stream=None):
        attn_kv_release(seq_ids, self, stream=stream)

    def status(self) -> int:
        """Outcome of the last call (synchronizes with the device)."""
        return int(self.kv_status.item())


def attn_kv_append(k_new, v_new, cache, stream=None):
    """Lease pages where needed and append k_new, v_new [S, Hkv, D] at each sequence's
    current length (async; the outcome lands in cache.kv_status)."""
    c = cache
    dev = _same_device(k_new, v_new, c.k_pool)
    if k_new.shape != (c.S, c.Hkv, c.D) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [{c.S}, {c.Hkv}, {c.D}], got {tuple(k_new.shape)}")
    _check(lib().attn_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"), c.S, c.Hkv, c.D, c.page_size,
                                c.max_pages, c.num_pages, _dev(c.k_pool, "k_pool"), _dev(c.v_pool, "v_pool"),
                                _dev(c.block_table, "block_table", torch.int32),
                                _dev(c.context_lens, "context_lens", torch.int32),
                                _dev(c.free_pages, "free_pages", torch.int32),
                                _dev(c.free_count, "free_count", torch.int32),
                                _dev(c.kv_status, "kv_status", torch.int32), _stream_ptr(stream, dev)))


def attn_kv_append_tokens(k_new, v_new, token_start, cache, stream=None):
    """Lease pages where needed and append, to each sequence s, the rows
    token_start[s] .. token_start[s+1]-1 of k_new, v_new [N, Hkv, D] (token_start: int32
    device tensor [S + 1]; async, the outcome lands in cache.kv_status)."""
    c = cache
    dev = _same_device(k_new, v_new, token_start, c.k_pool)
    if k_new.dim() != 3 or k_new.shape[1:] != (c.Hkv, c.D) or v_new.shape != k_new.shape:
        raise ValueError(f"k_new/v_new must be [N, {c.Hkv}, {c.D}], got {tuple(k_new.shape)}")
    if token_start.shape != (c.S + 1,):
        raise ValueError(f"token_start must be [{c.S + 1}]")
    N = k_new.shape[0]
    kp = _dev(k_new, "k_new") if N > 0 else ctypes.c_void_p(0)
    vp = _dev(v_new, "v_new") if N > 0 else ctypes.c_void_p(0)
    _check(lib().attn_kv_append_tokens(kp, vp, _dev(token_start, "token_start", torch.int32), c.S, N, c.Hkv, c.D,
                                       c.page_size, c.max_pages, c.num_pages, _dev(c.k_pool, "k_pool"),
                                       _dev(c.v_pool, "v_pool"), _dev(c.block_table, "block_table", torch.int32),
                                       _dev(c.context_lens, "context_lens", torch.int32),
                                       _dev(c.free_pages, "free_pages", torch.int32),
                                       _dev(c.free_count, "free_count", torch.int32),
                                       _dev(c.kv_status, "kv_status", torch.int32), _stream_ptr(stream, dev)))


def attn_paged_prefill(q, k_pool, v_pool, block_table, context_lens, token_start, scale=None, o=None, lse=None,
                       stream=None, with_lse=True):
    """O [N,Hq,D] (and LSE [N,Hq]) of the new tokens q [N,Hq,D] of a ragged batch over a
    paged cache: row token_start[s] + j is token j of sequence s, at position
    context_lens[s] - n_s + j, and attends to positions 0 .. that one (async)."""
    dev = _same_device(q, k_pool, v_pool, block_table, context_lens, token_start)
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("expected q [N,Hq,D] and pools [num_pages,Hkv,page_size,D]")
    N, Hq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_pool.shape
    S = block_table.shape[0]
    if Dk != D or block_table.dim() != 2 or context_lens.shape != (S,) or token_start.shape != (S + 1,):
        raise ValueError("shape mismatch among q, pools, block_table, context_lens, token_start")
    _given(o, q.shape, "o")
    _given(lse, (N, Hq), "lse")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with _alloc_on(stream, o, lse if with_lse else o):
        if o is None:
            o = torch.empty_like(q)
        if with_lse and lse is None:
            lse = torch.empty((N, Hq), device=dev, dtype=torch.float32)
    lse_p = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    _check(lib().attn_paged_prefill(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                    _dev(block_table, "block_table", torch.int32),
                                    _dev(context_lens, "context_lens", torch.int32),
                                    _dev(token_start, "token_start", torch.int32), S, N, Hq, Hkv, D, page_size,
                                    block_table.shape[1], num_pages, scale, _dev(o, "o"), lse_p,
                                    _stream_ptr(stream, dev)))
    return o, lse


def attn_kv_release(seq_ids, cache, stream=None):
    """Return the pages of sequences seq_ids (int32 device tensor of distinct indices)
    to the free stack and zero their lengths (async)."""
    c = cache
    dev = _same_device(seq_ids, c.k_pool)
    if seq_ids.dim() != 1:
        raise ValueError("seq_ids must be 1-D")
    n = seq_ids.numel()
    ids_p = _dev(seq_ids, "seq_ids", torch.int32) if n > 0 else ctypes.c_void_p(0)
    _check(lib().attn_kv_release(ids_p, n, c.S, c.page_size, c.max_pages, c.num_pages,
                                 _dev(c.block_table, "block_table", torch.int32),
                                 _dev(c.context_lens, "context_lens", torch.int32),
                                 _dev(c.free_pages, "free_pages", torch.int32),
                                 _dev(c.free_count, "free_count", torch.int32),
                                 _dev(c.kv_status, "kv_status", torch.int32), _stream_ptr(stream, dev)))
