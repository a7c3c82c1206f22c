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
ATTN_ABI_VERSION = 0x00010000

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
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"expected q [B,Hq,T,D], k/v [B,Hkv,T,D]; got {tuple(q.shape)}, {tuple(k.shape)}")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
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
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape or lse.shape != (B, Hq, T):
        raise ValueError("shape mismatch among q, k, v, o, lse, dout")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    need = attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D)
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
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((S, Hq), device=dev, dtype=torch.float32)
    need = attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page_size, max_pages)
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
