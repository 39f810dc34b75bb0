"""CPU oracle for rotated-scalar-codec KV decode attention (TEST INFRASTRUCTURE).

Plain, slow, float64 NumPy/Python definitions of what the decode path
computes: the Lloyd-Max codebooks, the sign-flip + Walsh-Hadamard rotation,
the per-group fp16 norm, nearest-centroid codes and their byte layout, and
full-dequant softmax attention.  It shares no code with the HIP library.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the library itself never does.

Parity status: every function here is pinned by a `-m "not gpu"` test
against closed forms, textbook values, brute force or hand-worked bytes
(tests/test_oracle_*.py).  Nothing is "parity unpinned".
"""
