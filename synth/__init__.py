"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds workload shapes and random-number generation only: no
step of the codec or of attention is computed here.  Both sides of every
parity check draw their inputs (K, V, q, sign vectors, context lengths) from
these generators, so a given (workload, seed) always produces the same bytes.
"""
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    rng_for,
    sign_vector,
    context_lengths,
    kv_slice,
    new_token_kv,
    queries,
    STREAMS,
)
