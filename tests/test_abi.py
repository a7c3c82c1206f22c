"""The C ABI without a GPU: the library loads, exports every function the header
declares, reports its version and workspace sizes, and rejects every invalid
argument with its status and a message before any HIP call.

Fake, never-dereferenced device addresses are used: validation fails before a
pointer is touched.  A valid call on a machine with no GPU returns
ATTN_DEVICE_ERROR instead of crashing.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import causal_self_attention_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def _exported_symbols(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    return {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}


@pytest.fixture(scope="module")
def L():
    return attn.lib()


def test_every_declared_function_is_exported(L):
    declared = _declared_functions()
    assert declared == sorted(attn._binding.SIGNATURES), "binding and header disagree"
    exported = _exported_symbols(attn.library_path())
    missing = [f for f in declared if f not in exported]
    assert not missing, f"declared in attn.h but not exported: {missing}"
    for f in declared:
        assert hasattr(L, f)


def test_header_is_c11_clean(tmp_path):
    src = tmp_path / "use_header.c"
    src.write_text('#include "attn.h"\nint main(void) { return ATTN_OK + (int)ATTN_ABI_VERSION * 0; }\n')
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                    os.path.join(ROOT, "include"), "-o", str(tmp_path / "a.out"), str(src)], check=True)


def test_version_and_status_values(L):
    assert attn.attn_abi_version() == attn.ATTN_ABI_VERSION == 0x00010004
    header = open(HEADER).read()
    for name in ("ATTN_OK", "ATTN_INVALID_ARGUMENT", "ATTN_UNSUPPORTED", "ATTN_WORKSPACE_TOO_SMALL",
                 "ATTN_DEVICE_ERROR"):
        m = re.search(name + r"\s*=\s*(\d+)", header)
        assert m and int(m.group(1)) == getattr(attn, name), name


def test_workspace_queries(L):
    def bwd_expect(B, Hq, Hkv, T, D):
        # Delta (rounded to 64 floats), then two dK, dV pieces [64, D] per run of the
        # finer cut (at most 512 work-groups, two steps each, only if finer than T/64)
        nkb = (T + 63) // 64
        fine = min(512 // (B * Hkv), Hq // Hkv * nkb * (nkb + 1) // 2 // 2)
        fine = fine if fine > nkb else 0
        floats = (B * Hq * T + 63) // 64 * 64 + B * Hkv * fine * 2 * 2 * 64 * D
        return (floats * 4 + 255) // 256 * 256
    assert attn.attn_causal_bwd_workspace_bytes(4, 8, 8, 1024, 64) == 4 * 8 * 1024 * 4  # no finer cut
    for args in ((4, 8, 2, 1024, 64), (1, 8, 8, 2048, 128), (1, 2, 2, 16, 8), (2, 4, 1, 200, 32), (1, 1, 1, 64, 8)):
        assert attn.attn_causal_bwd_workspace_bytes(*args) == bwd_expect(*args), args
    assert attn.attn_causal_bwd_workspace_bytes(1, 2, 2, 16, 8) == 256  # rounded up to 256
    assert attn.attn_causal_bwd_workspace_bytes(1, 3, 2, 16, 8) == 0    # Hq % Hkv != 0
    assert attn.attn_causal_bwd_workspace_bytes(0, 2, 2, 16, 8) == 0
    # partial (m, l, o[D]) records per query head for 1024 + S slots (the split grid plus
    # one boundary per sequence) and a first slot and slot count per sequence, 256-byte rounded
    def expect(S, Hq, Hkv, D, ps, maxp):
        b = (1024 + S) * Hq * (D + 2) * 4 + 2 * S * 4
        return -(-b // 256) * 256
    for args in ((32, 16, 4, 64, 16, 256), (32, 16, 4, 64, 16, 512), (32, 16, 4, 64, 16, 1),
                 (32, 16, 4, 64, 16, 100000), (3, 8, 8, 32, 64, 7), (1, 1, 1, 8, 16, 1)):
        assert attn.attn_paged_decode_workspace_bytes(*args) == expect(*args), args
    assert attn.attn_paged_decode_workspace_bytes(32, 16, 5, 64, 16, 256) == 0


# fake device addresses, 256-byte spaced far apart so ranges never overlap
def _p(i):
    return ctypes.c_void_p(0x100000000 * (i + 1))


def _fwd(L, q=_p(0), k=_p(1), v=_p(2), B=1, Hq=2, Hkv=2, T=16, D=8, scale=0.35, o=_p(3), lse=_p(4)):
    return L.attn_causal_fwd(q, k, v, B, Hq, Hkv, T, D, scale, o, lse, None)


def _bwd(L, B=1, Hq=2, Hkv=2, T=16, D=8, scale=0.35, ws_bytes=None, **ptrs):
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = attn.attn_causal_bwd_workspace_bytes(B, Hq, Hkv, T, D)
    return L.attn_causal_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], B, Hq, Hkv, T, D, scale,
                             p["dq"], p["dk"], p["dv"], p["ws"], ws_bytes, None)


def _dec(L, S=2, Hq=4, Hkv=2, D=64, page=16, maxp=8, npages=16, scale=0.125, ws_bytes=None, **ptrs):
    names = ["q", "kp", "vp", "bt", "ctx", "o", "lse", "ws"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = attn.attn_paged_decode_workspace_bytes(S, Hq, Hkv, D, page, maxp)
    return L.attn_paged_decode(p["q"], p["kp"], p["vp"], p["bt"], p["ctx"], S, Hq, Hkv, D, page, maxp, npages,
                               scale, p["o"], p["lse"], p["ws"], ws_bytes, None)


def _decna(L, S=2, Hq=4, Hkv=2, D=64, page=16, maxp=8, npages=16, scale=0.125, **ptrs):
    names = ["q", "kp", "vp", "bt", "ctx", "o", "lse"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.attn_paged_decode_noalloc(p["q"], p["kp"], p["vp"], p["bt"], p["ctx"], S, Hq, Hkv, D, page, maxp,
                                       npages, scale, p["o"], p["lse"], None)


def _matf(L, B=1, Hq=2, Hkv=2, T=16, D=8, scale=0.35, **ptrs):
    names = ["q", "k", "v", "o", "lse", "p"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.attn_materialized_fwd(p["q"], p["k"], p["v"], B, Hq, Hkv, T, D, scale, p["o"], p["lse"], p["p"], None)


def _matb(L, B=1, Hq=2, Hkv=2, T=16, D=8, scale=0.35, ws_bytes=None, **ptrs):
    names = ["q", "k", "v", "o", "p", "dout", "dp", "dq", "dk", "dv", "ws"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = attn.attn_materialized_bwd_workspace_bytes(B, Hq, Hkv, T, D)
    return L.attn_materialized_bwd(p["q"], p["k"], p["v"], p["o"], p["p"], p["dout"], p["dp"], B, Hq, Hkv, T, D,
                                   scale, p["dq"], p["dk"], p["dv"], p["ws"], ws_bytes, None)


def _pre(L, S=3, N=40, Hq=4, Hkv=2, D=64, page=16, maxp=8, npages=16, scale=0.125, **ptrs):
    names = ["q", "kp", "vp", "bt", "ctx", "ts", "o", "lse"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.attn_paged_prefill(p["q"], p["kp"], p["vp"], p["bt"], p["ctx"], p["ts"], S, N, Hq, Hkv, D, page, maxp,
                                npages, scale, p["o"], p["lse"], None)


def _appt(L, S=3, N=40, Hkv=2, D=64, page=16, maxp=4, npages=8, **ptrs):
    names = ["kn", "vn", "ts", "kp", "vp", "bt", "ctx", "free", "fc", "st"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.attn_kv_append_tokens(p["kn"], p["vn"], p["ts"], S, N, Hkv, D, page, maxp, npages, p["kp"], p["vp"],
                                   p["bt"], p["ctx"], p["free"], p["fc"], p["st"], None)


def _app(L, S=3, Hkv=2, D=64, page=16, maxp=4, npages=8, **ptrs):
    names = ["kn", "vn", "kp", "vp", "bt", "ctx", "free", "fc", "st"]
    p = {n: _p(i) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.attn_kv_append(p["kn"], p["vn"], S, Hkv, D, page, maxp, npages, p["kp"], p["vp"], p["bt"], p["ctx"],
                            p["free"], p["fc"], p["st"], None)


def _rel(L, n=2, S=3, page=16, maxp=4, npages=8, **ptrs):
    names = ["ids", "bt", "ctx", "free", "fc", "st"]
    p = {n_: _p(i) for i, n_ in enumerate(names)}
    p.update(ptrs)
    return L.attn_kv_release(p["ids"], n, S, page, maxp, npages, p["bt"], p["ctx"], p["free"], p["fc"], p["st"],
                             None)


def _expect(status, want, fragment):
    assert status == want, (status, attn.attn_last_error())
    msg = attn.attn_last_error()
    assert fragment.lower() in msg.lower(), msg


def test_fwd_invalid_arguments(L):
    _expect(_fwd(L, q=None), attn.ATTN_INVALID_ARGUMENT, "'q' is NULL")
    _expect(_fwd(L, lse=None), attn.ATTN_INVALID_ARGUMENT, "'lse' is NULL")
    _expect(_fwd(L, T=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_fwd(L, B=-1), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_fwd(L, Hq=3, Hkv=2), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_fwd(L, scale=float("nan")), attn.ATTN_INVALID_ARGUMENT, "scale")
    _expect(_fwd(L, scale=float("inf")), attn.ATTN_INVALID_ARGUMENT, "scale")
    _expect(_fwd(L, D=24), attn.ATTN_UNSUPPORTED, "D=24")
    _expect(_fwd(L, D=256), attn.ATTN_UNSUPPORTED, "D=256")
    _expect(_fwd(L, k=ctypes.c_void_p(0x200000008)), attn.ATTN_INVALID_ARGUMENT, "aligned")
    _expect(_fwd(L, T=1 << 30, D=64), attn.ATTN_INVALID_ARGUMENT, "too large")
    _expect(_fwd(L, B=1 << 20, Hq=256, Hkv=256, T=4096, D=64), attn.ATTN_INVALID_ARGUMENT, "row blocks")
    _expect(_bwd(L, B=1 << 16, Hq=256, Hkv=256, T=1 << 16, D=128, ws_bytes=1 << 40), attn.ATTN_INVALID_ARGUMENT,
            "row blocks")
    assert attn.attn_causal_bwd_workspace_bytes(1 << 16, 256, 256, 1 << 16, 128) == 0
    # o overlaps q; lse overlaps o
    _expect(_fwd(L, o=ctypes.c_void_p(0x100000000 + 64)), attn.ATTN_INVALID_ARGUMENT, "overlaps")
    _expect(_fwd(L, lse=ctypes.c_void_p(0x400000000 + 16)), attn.ATTN_INVALID_ARGUMENT, "overlap")


def test_bwd_invalid_arguments(L):
    _expect(_bwd(L, dv=None), attn.ATTN_INVALID_ARGUMENT, "'dv' is NULL")
    _expect(_bwd(L, ws=None), attn.ATTN_INVALID_ARGUMENT, "'workspace' is NULL")
    _expect(_bwd(L, Hq=4, Hkv=3), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_bwd(L, D=12), attn.ATTN_UNSUPPORTED, "D=12")
    _expect(_bwd(L, ws_bytes=16), attn.ATTN_WORKSPACE_TOO_SMALL, "needs 256")
    _expect(_bwd(L, dq=_p(0)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'q'")
    _expect(_bwd(L, dk=_p(6)), attn.ATTN_INVALID_ARGUMENT, "overlap")  # dk == dq
    _expect(_bwd(L, ws=_p(5)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'dout'")
    _expect(_bwd(L, scale=float("-inf")), attn.ATTN_INVALID_ARGUMENT, "scale")


def test_decode_invalid_arguments(L):
    _expect(_dec(L, bt=None), attn.ATTN_INVALID_ARGUMENT, "'block_table' is NULL")
    _expect(_dec(L, S=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_dec(L, npages=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_dec(L, Hq=6, Hkv=4), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_dec(L, page=8), attn.ATTN_UNSUPPORTED, "page_size=8")
    _expect(_dec(L, D=48), attn.ATTN_UNSUPPORTED, "D=48")
    _expect(_dec(L, Hq=34, Hkv=2), attn.ATTN_UNSUPPORTED, "Hq/Hkv=17")
    _expect(_dec(L, scale=float("nan")), attn.ATTN_INVALID_ARGUMENT, "scale")
    _expect(_dec(L, ws_bytes=1), attn.ATTN_WORKSPACE_TOO_SMALL, "needs")
    _expect(_dec(L, o=_p(1)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'k_pool'")
    _expect(_dec(L, bt=ctypes.c_void_p(0x400000002)), attn.ATTN_INVALID_ARGUMENT, "aligned")


def test_decode_noalloc_invalid_arguments(L):
    """The no-allocation decode validates exactly like attn_paged_decode (less the
    workspace) before any HIP call."""
    _expect(_decna(L, bt=None), attn.ATTN_INVALID_ARGUMENT, "'block_table' is NULL")
    _expect(_decna(L, o=None), attn.ATTN_INVALID_ARGUMENT, "'o' is NULL")
    _expect(_decna(L, S=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_decna(L, Hq=6, Hkv=4), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_decna(L, page=8), attn.ATTN_UNSUPPORTED, "page_size=8")
    _expect(_decna(L, D=48), attn.ATTN_UNSUPPORTED, "D=48")
    _expect(_decna(L, scale=float("nan")), attn.ATTN_INVALID_ARGUMENT, "scale")
    _expect(_decna(L, o=_p(1)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'k_pool'")
    _expect(_decna(L, lse=_p(5)), attn.ATTN_INVALID_ARGUMENT, "overlap")  # lse == o
    _expect(_decna(L, lse=ctypes.c_void_p(0x700000002)), attn.ATTN_INVALID_ARGUMENT, "aligned")


def test_decode_noalloc_scratch_constant():
    m = re.search(r"#define ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == attn.ATTN_PAGED_DECODE_NOALLOC_SCRATCH_BYTES


def test_materialized_invalid_arguments(L):
    _expect(_matf(L, p=None), attn.ATTN_INVALID_ARGUMENT, "'p' is NULL")
    _expect(_matf(L, D=20), attn.ATTN_UNSUPPORTED, "D=20")
    _expect(_matf(L, Hq=3, Hkv=2), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_matf(L, p=_p(3)), attn.ATTN_INVALID_ARGUMENT, "overlap")  # p == o
    _expect(_matf(L, B=1 << 10, Hq=1 << 10, T=1 << 10, D=8), attn.ATTN_INVALID_ARGUMENT, "2^40")
    _expect(_matb(L, p=None), attn.ATTN_INVALID_ARGUMENT, "'p' is NULL")
    _expect(_matb(L, ws_bytes=8), attn.ATTN_WORKSPACE_TOO_SMALL, "needs")
    _expect(_matb(L, dq=_p(4)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'p'")
    _expect(_matb(L, dv=_p(6)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'dp'")
    _expect(_matb(L, dp=ctypes.c_void_p(0x700000002)), attn.ATTN_INVALID_ARGUMENT, "aligned")
    _expect(_matb(L, scale=float("nan")), attn.ATTN_INVALID_ARGUMENT, "scale")


def test_prefill_invalid_arguments(L):
    _expect(_pre(L, q=None), attn.ATTN_INVALID_ARGUMENT, "'q' is NULL")
    _expect(_pre(L, ts=None), attn.ATTN_INVALID_ARGUMENT, "'token_start' is NULL")
    _expect(_pre(L, N=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_pre(L, Hq=3, Hkv=2), attn.ATTN_INVALID_ARGUMENT, "Hq % Hkv")
    _expect(_pre(L, D=24), attn.ATTN_UNSUPPORTED, "D=24")
    _expect(_pre(L, page=8), attn.ATTN_UNSUPPORTED, "page_size=8")
    _expect(_pre(L, scale=float("inf")), attn.ATTN_INVALID_ARGUMENT, "scale")
    _expect(_pre(L, o=_p(0)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'q'")
    _expect(_pre(L, lse=_p(6)), attn.ATTN_INVALID_ARGUMENT, "overlap")  # lse == o
    _expect(_pre(L, ts=ctypes.c_void_p(0x600000002)), attn.ATTN_INVALID_ARGUMENT, "aligned")
    _expect(_appt(L, ts=None), attn.ATTN_INVALID_ARGUMENT, "'token_start' is NULL")
    _expect(_appt(L, N=-1), attn.ATTN_INVALID_ARGUMENT, "N >= 0")
    _expect(_appt(L, page=48), attn.ATTN_UNSUPPORTED, "page_size")
    _expect(_appt(L, bt=_p(2)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'token_start'")
    _expect(_appt(L, kn=None), attn.ATTN_INVALID_ARGUMENT, "'k_new' is NULL")


def test_kv_invalid_arguments(L):
    _expect(_app(L, kn=None), attn.ATTN_INVALID_ARGUMENT, "'k_new' is NULL")
    _expect(_app(L, st=None), attn.ATTN_INVALID_ARGUMENT, "'kv_status' is NULL")
    _expect(_app(L, S=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_app(L, Hkv=0), attn.ATTN_INVALID_ARGUMENT, "positive")
    _expect(_app(L, page=24), attn.ATTN_UNSUPPORTED, "page_size 24")
    _expect(_app(L, D=40), attn.ATTN_UNSUPPORTED, "D=40")
    _expect(_app(L, kp=ctypes.c_void_p(0x300000004)), attn.ATTN_INVALID_ARGUMENT, "aligned")
    _expect(_app(L, kp=_p(0)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'k_new'")
    _expect(_app(L, fc=_p(6)), attn.ATTN_INVALID_ARGUMENT, "overlap")  # free_count inside free_pages
    _expect(_rel(L, ids=None), attn.ATTN_INVALID_ARGUMENT, "'seq_ids' is NULL")
    _expect(_rel(L, n=4), attn.ATTN_INVALID_ARGUMENT, "[0, S]")
    _expect(_rel(L, n=-1), attn.ATTN_INVALID_ARGUMENT, "[0, S]")
    _expect(_rel(L, page=128), attn.ATTN_UNSUPPORTED, "page_size 128")
    _expect(_rel(L, ctx=_p(0)), attn.ATTN_INVALID_ARGUMENT, "overlaps input 'seq_ids'")


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_lse_is_optional_for_decode_but_validated(L):
    _expect(_dec(L, lse=ctypes.c_void_p(0x700000002)), attn.ATTN_INVALID_ARGUMENT, "aligned")
    if _gpu_present():
        return  # a fully valid call would launch on the fake addresses
    assert _dec(L, lse=None) == attn.ATTN_DEVICE_ERROR  # valid without lse; no device here


def test_valid_call_without_device_reports_device_error(L):
    # Fully valid arguments reach the device check; never run this where a GPU
    # exists, since the fake addresses would then be launched on.
    if _gpu_present():
        pytest.skip("a GPU is present; this checks the no-device path")
    _expect(_fwd(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_bwd(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_dec(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_decna(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_decna(L, lse=None), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_matf(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_matb(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_matb(L, dp=None), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_app(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_appt(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_appt(L, N=0, kn=None, vn=None), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_pre(L), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_pre(L, lse=None), attn.ATTN_DEVICE_ERROR, "device")
    _expect(_rel(L), attn.ATTN_DEVICE_ERROR, "device")


def test_success_clears_nothing_spurious(L):
    # a failing call leaves a message; the binding raises AttnError with status + message
    with pytest.raises(attn.AttnError) as ei:
        attn._binding._check(_fwd(L, q=None))
    assert ei.value.status == attn.ATTN_INVALID_ARGUMENT and "'q' is NULL" in str(ei.value)
