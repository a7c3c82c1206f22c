"""bench.py's contract on the host: the one-GPU refusal, the algorithmic work it divides
by, and the rule that counter-measured traffic is reported only for the kernel source it
was measured on.  No GPU is touched: these paths run before bench.py imports torch."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, (n, r.returncode, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def test_causal_flops_count_unmasked_pairs():
    # T = 3: pairs (0,0), (1,0), (1,1), (2,0), (2,1), (2,2) per head
    fwd, bwd = bench.causal_flops(2, 3, 3, 8)
    pairs = 2 * 3 * 6
    assert fwd == 4 * 8 * pairs  # QK^T and PV: 2 d each
    assert bwd == 10 * 8 * pairs  # QK^T recompute, dV, dP, dK, dQ: 2 d each
    # the 1024-token workload the headline is quoted on
    f, b = bench.causal_flops(4, 8, 1024, 64)
    assert f + b == 14 * 64 * 4 * 8 * 1024 * 1025 // 2 == 15_047_065_600


def test_decode_bytes_by_hand():
    # two sequences of 17 and 1 cached positions, 16-position pages, 2 query heads on
    # one KV head, d = 4: K and V rows 18 * 4 * 4 * 2 = 576 B, q in + o out 128 B,
    # LSE 16 B, 3 used table entries 12 B, 2 lengths 8 B
    d = {"context_lens": [17, 1], "page_size": 16}
    assert bench.decode_bytes(d, 2, 1, 4) == 576 + 128 + 16 + 12 + 8


def test_traffic_only_for_the_measured_kernel_source(monkeypatch):
    path = os.path.join(ROOT, "causal_self_attention_amd", "csrc", "attn_bwd.hip")
    digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    monkeypatch.setattr(bench, "BWD_TRAFFIC_SOURCE_SHA256_PREFIX", digest[:16])
    assert bench.bwd_traffic() == bench.BWD_TRAFFIC_BYTES
    other = "0" * 16 if not digest.startswith("0" * 16) else "f" * 16
    monkeypatch.setattr(bench, "BWD_TRAFFIC_SOURCE_SHA256_PREFIX", other)
    assert bench.bwd_traffic() is None
