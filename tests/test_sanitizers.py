"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/attn_oracle.c) is rebuilt with gcc -fsanitize=address,undefined
  and every pin of tests/oracle_pins.py, plus the oracle on the 256-token workload and a
  paged decode and prefill, runs against it in a child process.
* The library's host code (argument validation, error reporting, launch set-up; the
  device code is built as usual) is rebuilt with hipcc, each -fsanitize= behind
  -Xarch_host, and tests/test_abi.py -- every validation path and, with no GPU here,
  the no-device path -- runs against it in a child process.
Sanitizer runtimes are preloaded into the (uninstrumented) Python child; leak checking is
off (Python itself keeps memory until exit).  Each runtime is first shown to catch a
planted heap overflow, so a silent pass cannot come from a sanitizer that is not there.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")
CSRC = os.path.join(ROOT, "causal_self_attention_amd", "csrc")
LIB_SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_kv.hip",
               "attn_materialized.hip", "attn_prefill.hip", "attn_checks.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

PLANTED = r"""
#include <stdlib.h>
int planted_overflow(int n) {
    int* a = (int*)malloc(sizeof(int) * n);
    for (int i = 0; i < n; ++i) a[i] = i;
    int s = a[n];  /* one past the end */
    free(a);
    return s;
}
"""


def _gcc_runtimes():
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            pytest.skip(f"gcc's {name} is not installed")
        out.append(p)
    return ":".join(out)


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's ASan runtime is not installed")
    return found[-1]


def _child(code_or_args, preload, extra_env=None, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV, **(extra_env or {}))
    args = [sys.executable, "-c", code_or_args] if isinstance(code_or_args, str) else code_or_args
    return subprocess.run(args, env=env, capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def _planted_lib(tmp_path, compiler_cmd):
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    lib = tmp_path / "libplanted.so"
    subprocess.run(compiler_cmd + ["-o", str(lib), str(src)], check=True, capture_output=True)
    return lib


def _caught(r):
    return r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    preload = _gcc_runtimes()
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fPIC", "-shared"]
    planted = _planted_lib(tmp_path, ["gcc", "-std=c11"] + flags)
    r = _child(f"import ctypes; ctypes.CDLL({str(planted)!r}).planted_overflow(8)", preload)
    assert _caught(r), ("the gcc sanitizers did not catch a planted overflow", r.returncode, r.stderr[-2000:])

    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c11", "-fopenmp"] + flags + ["-o", str(lib), ORACLE_SRC, "-lm"], check=True)
    code = f"""
import sys
sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {TESTS!r})
import oracle_pins, synthetic_inputs as si
from oracle.oracle import Oracle
o = Oracle({str(lib)!r})
for pin in oracle_pins.ALL_PINS:
    pin(o)
h = si.causal_workload("mha_b8_h4_t256_d32")
o.causal_fwd(h["q"], h["k"], h["v"]); o.causal_bwd(h["q"], h["k"], h["v"], h["dout"])
d = si.paged_decode_inputs(S=8, Hq=16, Hkv=4, D=64, page_size=16, ctx_lo=1, ctx_hi=600, max_pages=40, seed=3)
o.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"])
p = si.paged_prefill_inputs(S=3, Hq=8, Hkv=2, D=32, page_size=16, cached_lo=0, cached_hi=90, new_lo=1, new_hi=60,
                            max_pages=12, seed=4)
o.paged_prefill(p["q"], p["k_pool"], p["v_pool"], p["block_table"], p["context_lens"], p["token_start"])
print("ORACLE CLEAN", flush=True)
"""
    r = _child(code, preload)
    assert r.returncode == 0 and "ORACLE CLEAN" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])


def test_library_host_code_under_asan_ubsan(tmp_path):
    preload = _clang_asan_runtime()
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", f]
    planted = _planted_lib(tmp_path, [HIPCC, "-x", "c", "-O1", "-g", "-fPIC", "-shared"] + san)
    r = _child(f"import ctypes; ctypes.CDLL({str(planted)!r}).planted_overflow(8)", preload)
    assert _caught(r), ("clang's sanitizers did not catch a planted overflow", r.returncode, r.stderr[-2000:])

    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")] + san

    def compile_one(src):
        obj = tmp_path / (src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        p = subprocess.run([HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", str(obj)],
                           capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-3000:]
        return str(obj)

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, LIB_SOURCES))
    lib = tmp_path / "libattn_san.so"
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", str(lib)] + objs, check=True,
                   capture_output=True)
    r = _child([sys.executable, "-m", "pytest", os.path.join(TESTS, "test_abi.py"), "-q", "-p", "no:cacheprovider"],
               preload, {"ATTN_LIBRARY": str(lib)})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-4000:])
    assert " passed" in r.stdout
