"""Test infrastructure only: the plain CPU reference for causal attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.
"""
