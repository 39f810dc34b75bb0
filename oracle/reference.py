"""Whole-step reference: encode a cache into the library's byte layout, then attend.

Glue over codec.py and attention.py for the tests, the smoke check and the
benchmark's CPU-baseline leg.  Arrays are per (KV head, token) of ONE sequence
so that sampled checks at full size only touch the sequences they sample.
"""
import math

import numpy as np

from . import attention as att
from . import codec

SCALE = 1.0 / math.sqrt(128.0)


def encode_sequence(k16, v16, k_format, v_format, k_signs, v_signs, codebooks, capacity=None):
    """Encode one sequence [Hkv, L, 128] (fp16) into the library's layout.

    Returns dict with k_rec [Hkv, cap, 48|64] (or k_f16 [Hkv, cap, 128]), k_norms [Hkv, cap],
    v_tiles [Hkv, cap/32, 1536|2048], v_norms [Hkv, cap], plus the raw codes.
    Slots at or beyond L are zero."""
    hkv, L, _ = k16.shape
    cap = capacity or ((L + 31) // 32) * 32
    out = {}
    if k_format == "f16":
        kf = np.zeros((hkv, cap, 128), dtype=np.float16)
        kf[:, :L] = k16
        out["k_f16"] = kf
    else:
        kc, kn = codec.encode(k16, k_signs, codebooks[k_format])
        codes = np.zeros((hkv, cap, 128), dtype=np.uint8)
        codes[:, :L] = kc
        norms = np.zeros((hkv, cap), dtype=np.float16)
        norms[:, :L] = kn
        out["k_codes"], out["k_norms"] = codes, norms
        out["k_rec"] = codec.k_records_to_memory(codec.pack_k_record(codes, k_format), k_format)
    if v_format == "f16":   # the uncompressed comparison cache: values stored as they come
        vf = np.zeros((hkv, cap, 128), dtype=np.float16)
        vf[:, :L] = v16
        out["v_f16"] = vf
        out["v_tiles"] = codec.pack_v_tiles(vf, "f16")
        return out
    vc, vn = codec.encode(v16, v_signs, codebooks[v_format])
    codes = np.zeros((hkv, cap, 128), dtype=np.uint8)
    codes[:, :L] = vc
    norms = np.zeros((hkv, cap), dtype=np.float16)
    norms[:, :L] = vn
    out["v_codes"], out["v_norms"] = codes, norms
    out["v_tiles"] = codec.pack_v_tiles(codes, v_format)
    return out


def dequant_sequence(enc, k_format, v_format, k_signs, v_signs, codebooks, length):
    """Full-basis K and V [Hkv, L, 128] (float64) of an encoded sequence."""
    if k_format == "f16":
        k = enc["k_f16"][:, :length].astype(np.float64)
    else:
        k = codec.dequant(enc["k_codes"][:, :length], enc["k_norms"][:, :length], codebooks[k_format], k_signs)
    if v_format == "f16":
        return k, enc["v_f16"][:, :length].astype(np.float64)
    v = codec.dequant(enc["v_codes"][:, :length], enc["v_norms"][:, :length], codebooks[v_format], v_signs)
    return k, v


def decode_sequence(q, k_hat, v_hat, length, scale=SCALE):
    """Attention output [Hq, 128] (float64) of one sequence against its dequantised cache."""
    return att.attention(np.asarray(q)[None], [k_hat], [v_hat], [length], scale)[0]


def codes_from_library_layout(k_rec, v_tiles, k_format, v_format):
    """Unpack the library's byte layout back to codes [Hkv, cap, 128] (K may be None for f16;
    for f16 V the values come back, fp16)."""
    kc = None if k_rec is None else codec.unpack_k_record(codec.k_memory_to_records(k_rec, k_format), k_format)
    vc = codec.unpack_v_tiles(v_tiles, v_format)
    return kc, vc
