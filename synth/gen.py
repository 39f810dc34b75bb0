"""Seeded generators for the decode workloads.

Every draw comes from NumPy's PCG64 seeded with a SeedSequence of
(seed, stream, *indices), so any (sequence, KV head) slice can be regenerated on
its own, in any process, without producing the rest of the workload.

Streams:
  0 K prefill, 1 V prefill, 2 q, 3 K outlier channels, 4 K heavy-tail mask and
  values, 5 context lengths, 6 appended-token K, 7 appended-token V,
  8 K sign vector, 9 V sign vector.

The sign vectors are the Rademacher draws the codec makes from its seed; they
are generated here and handed to both the oracle and the library as inputs.
"""
import numpy as np

from .workloads import HEAD_DIM, Workload

STREAMS = {
    "k": 0, "v": 1, "q": 2, "k_outlier": 3, "k_tail": 4, "lengths": 5,
    "k_new": 6, "v_new": 7, "k_signs": 8, "v_signs": 9,
}
FP16_MAX = 65504.0


def rng_for(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, keys)])))


def sign_vector(seed: int, which: str) -> np.ndarray:
    """Rademacher vector in {+1,-1}^128 (float32) for the K ('k') or V ('v') codec."""
    bits = rng_for(seed, STREAMS[which + "_signs"]).integers(0, 2, HEAD_DIM)
    return (1 - 2 * bits).astype(np.float32)


def context_lengths(w: Workload, seed: int) -> np.ndarray:
    """Visible context per sequence after the step's append (int64 [B])."""
    if w.context is not None:
        return np.full(w.batch, w.context, dtype=np.int64)
    lo, hi = w.ragged_range
    return rng_for(seed, STREAMS["lengths"]).integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)


def _to_fp16(x: np.ndarray) -> np.ndarray:
    return np.clip(x, -FP16_MAX, FP16_MAX).astype(np.float16)


def _k_values(w: Workload, rng_main, rng_out, rng_tail, rows: int) -> np.ndarray:
    x = rng_main.standard_normal((rows, HEAD_DIM), dtype=np.float32)
    if w.k_outlier_channels:
        ch = rng_out.choice(HEAD_DIM, size=w.k_outlier_channels, replace=False)
        x[:, ch] *= np.float32(w.k_outlier_scale)
    if w.k_heavy_tail_frac > 0.0:
        mask = rng_tail.random((rows, HEAD_DIM)) < w.k_heavy_tail_frac
        n = int(mask.sum())
        x[mask] = rng_tail.standard_t(w.k_heavy_tail_nu, size=n).astype(np.float32)
    return _to_fp16(x)


def kv_slice(w: Workload, seed: int, which: str, b: int, h: int, length: int) -> np.ndarray:
    """Pre-encode fp16 K ('k') or V ('v') rows [length, 128] of sequence b, KV head h."""
    if which == "v":
        x = rng_for(seed, STREAMS["v"], b, h).standard_normal((length, HEAD_DIM), dtype=np.float32)
        return _to_fp16(x)
    return _k_values(w, rng_for(seed, STREAMS["k"], b, h), rng_for(seed, STREAMS["k_outlier"], b, h),
                     rng_for(seed, STREAMS["k_tail"], b, h), length)


def new_token_kv(w: Workload, seed: int, which: str, b: int, h: int, step: int, count: int = 1) -> np.ndarray:
    """fp16 rows [count, 128] appended to sequence b, KV head h at decode step `step`.

    K keeps the same outlier channels as the prefill of (b, h)."""
    if which == "v":
        x = rng_for(seed, STREAMS["v_new"], b, h, step).standard_normal((count, HEAD_DIM), dtype=np.float32)
        return _to_fp16(x)
    return _k_values(w, rng_for(seed, STREAMS["k_new"], b, h, step), rng_for(seed, STREAMS["k_outlier"], b, h),
                     rng_for(seed, STREAMS["k_tail"], b, h, step, 1), count)


def queries(w: Workload, seed: int, step: int = 0) -> np.ndarray:
    """Query rows [B, Hq, 128], float32 or float16 as the workload states."""
    x = rng_for(seed, STREAMS["q"], step).standard_normal((w.batch, w.num_q_heads, HEAD_DIM), dtype=np.float32)
    return x if w.q_dtype == "fp32" else x.astype(np.float16)
