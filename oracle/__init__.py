"""CPU float64 oracle for exact attention forward — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP product path never does.
"""
