"""ATTN_DEBUG_CHECKS=1: paged decode (both entry points) and prefill check their
device-side preconditions first and refuse a broken table, length or ragged offset
with ATTN_INVALID_ARGUMENT naming the sequence and page, launching nothing (the
outputs keep their contents).  The variable is read once per process, so the cases
run in a child process (tests/debug_checks_child.py); the broken tables are passed
only to checked calls."""
import os
import subprocess
import sys

import pytest

from gpu_common import announce, require_gpu

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_checks_refuse_broken_tables():
    require_gpu()
    announce("ATTN_DEBUG_CHECKS child process")
    env = dict(os.environ, ATTN_DEBUG_CHECKS="1")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_checks_child.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ALL DEBUG CHECKS OK" in r.stdout
