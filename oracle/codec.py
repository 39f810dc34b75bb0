"""Encode, byte layout and dequant of the rotated scalar codec (float64 / exact).

One 128-element head-dim group x (fp16) of one token and one KV head becomes
  * an fp16 L2 norm  n = RNE_fp16(||x||_2), and
  * 128 codebook indices idx_i = nearest entry of the codebook to y_i / n,
    where y = H (s * x) / sqrt(128) is the rotated group;
and is reconstructed as  x_hat = s * H (n * c[idx]) / sqrt(128).
(turboquant_plus "SMEM Pre-Dequant Experiment", "What Would Actually Work"
item 1: dequant is "index -> table[index] x norm"; mlxcel PR #369 "Change":
the codes live in the WHT-rotated basis.)

Readings where the pages are silent:
  * the norm is the exact real ||x||_2 rounded to nearest-even fp16, saturated
    at 65504; it is computed here with integers, so no summation order matters;
  * decisions compare y_i against n * beta_j, beta_j the midpoints of adjacent
    fp16 codebook entries, counting strict "greater than": ties and y = 0 go to
    the lower index, and n = 0 gives index 0 everywhere;
  * y_i = yhat_i / sqrt(128) in IEEE binary64, yhat = H (s * x) being exact.

Byte layouts (the pages print none; these are this library's):
  * turbo4 "octet word": 8 codes in one little-endian u32; code e (0..3) in
    bits 8e..8e+3, code e (4..7) in bits 8(e-4)+4..8(e-4)+7; each 4-bit field
    is sign-magnitude: bit 3 set for the 8 negative centroids, bits 0..2 the
    magnitude rank (0 = smallest |c|).
  * turbo3 "sub-block": 32 codes (3-bit ascending indices) in 3 u32 words
    A, B, C (12 bytes); for j = 0..3:
        A[8j..8j+2] = c[j],    A[8j+3..8j+5] = c[4+j],  A[8j+6..8j+7] = c[24+j] & 3
        B[8j..8j+2] = c[8+j],  B[8j+3..8j+5] = c[12+j], B[8j+6..8j+7] = c[28+j] & 3
        C[8j..8j+2] = c[16+j], C[8j+3..8j+5] = c[20+j], C[8j+6] = c[24+j] >> 2,
        C[8j+7] = c[28+j] >> 2
  * K record (one per token and KV head): turbo3 48 bytes = 4 sub-blocks for
    dims 32q..32q+31; turbo4 64 bytes = 16 octet words for dims 8w..8w+7.  In
    memory both are kept in blocks of 16 tokens, as pieces: turbo4 16-byte piece p
    (words 4p..4p+3) of the block's token i at byte 256 p + 16 i of the block's 1024
    bytes; turbo3 12-byte piece q (sub-block q) of token i at byte
    384 (q % 2) + 192 (q // 2) + 12 i of the block's 768 bytes.
  * V tile (32 tokens of one KV head, token-tiled): 64 chunks, chunk 16g + n
    holds the 8 tokens of slot group g and the 8 dims 8n..8n+7; element
    e = 8*nb + i of a chunk is dim 8n + nb of the token in tile slot
    r = 16*(i // 4) + 4*g + (i % 4).  turbo3 chunk = 2 sub-blocks (24 bytes,
    elements 0..31 then 32..63), sub-block p of chunk c at tile byte 768 p + 12 c;
    turbo4 chunk = 8 octet
    words (32 bytes), word nb holding elements 8nb..8nb+7, stored as two 16-byte
    pieces: piece p (words 4p..4p+3) of chunk c at tile byte 1024 p + 16 c.  Tile =
    1536 (turbo3) or 2048 (turbo4) bytes.
"""
import math

import numpy as np

from .hadamard import HEAD_DIM, inverse_rotate, rotate_unnormalised, SQRT_D
from .lloyd_max import decision_boundaries

BITS = {"turbo3": 3, "turbo4": 4}
K_RECORD_BYTES = {"turbo3": 48, "turbo4": 64}
V_TILE_TOKENS = 32
V_CHUNK_BYTES = {"turbo3": 24, "turbo4": 32, "f16": 128}
V_TILE_BYTES = {f: 64 * b for f, b in V_CHUNK_BYTES.items()}
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------- norm

def rne_fp16_of_sqrt(S: int) -> float:
    """Nearest-even fp16 value of sqrt(S) * 2**-24 for an integer S >= 0 (saturating).

    Exact: the candidate k*q is found with integer square roots and the
    rounding decision compares 4 S with q^2 (2k+1)^2."""
    if S < 0:
        raise ValueError("S must be non-negative")
    if S == 0:
        return 0.0
    r = math.isqrt(S)
    e = r.bit_length() - 1            # floor(log2 sqrt(S))
    q = 1 if e <= 10 else 1 << (e - 10)   # fp16 spacing at this magnitude, in units of 2**-24
    k = math.isqrt(S // (q * q))      # floor(sqrt(S) / q)
    lhs, rhs = 4 * S, q * q * (2 * k + 1) ** 2
    if lhs > rhs or (lhs == rhs and k & 1):
        k += 1
    return min(k * q * 2.0 ** -24, FP16_MAX)


def exact_sum_of_squares(x16) -> list:
    """sum(x_i^2) * 2**48 as Python ints, one per 128-group (x16: fp16 [..., 128]).

    Each fp16 value is an integer multiple of 2**-24 below 2**40 of them; the
    squares are split in 20-bit halves so every partial sum fits in int64."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    m = np.abs(x * 2.0 ** 24).astype(np.int64)
    hi, lo = m >> 20, m & ((1 << 20) - 1)
    a = (hi * hi).sum(axis=-1).reshape(-1)
    b = (hi * lo).sum(axis=-1).reshape(-1)
    c = (lo * lo).sum(axis=-1).reshape(-1)
    return [(int(ai) << 40) + (int(bi) << 21) + int(ci) for ai, bi, ci in zip(a, b, c)]


def group_norm_fp16(x16) -> np.ndarray:
    """fp16 L2 norm of each 128-group: RNE_fp16(sqrt(sum x_i^2)), exact, saturating at 65504."""
    x16 = np.asarray(x16, dtype=np.float16)
    sums = exact_sum_of_squares(x16)
    vals = np.array([rne_fp16_of_sqrt(s) for s in sums], dtype=np.float64)
    return vals.astype(np.float16).reshape(x16.shape[:-1])


# ----------------------------------------------------------------------------- codes

def rotated_coordinates(x16, signs) -> np.ndarray:
    """y = H (s * x) / sqrt(128) in float64, H (s * x) itself being exact."""
    return rotate_unnormalised(np.asarray(x16, dtype=np.float16), signs) / SQRT_D


def encode(x16, signs, codebook16):
    """(codes, norms) for fp16 groups x16 [..., 128].

    codes: uint8 ascending codebook indices, idx_i = #{j : y_i > n * beta_j}.
    norms: fp16 group norms."""
    n16 = group_norm_fp16(x16)
    y = rotated_coordinates(x16, signs)
    beta = decision_boundaries(codebook16)
    thr = n16.astype(np.float64)[..., None] * beta          # [..., K-1], exact products
    codes = (y[..., :, None] > thr[..., None, :]).sum(axis=-1)
    return codes.astype(np.uint8), n16


def boundary_margin(x16, signs, codebook16, eps: float = 1e-5) -> np.ndarray:
    """True where a rotated coordinate lies within eps (input units) of a decision threshold."""
    n16 = group_norm_fp16(x16)
    y = rotated_coordinates(x16, signs)
    thr = n16.astype(np.float64)[..., None] * decision_boundaries(codebook16)
    return (np.abs(y[..., :, None] - thr[..., None, :]) < eps).any(axis=-1)


# ----------------------------------------------------------------------------- bit layouts

def turbo4_nibble(idx):
    """Ascending index 0..15 -> sign-magnitude nibble (bit 3 = negative, bits 0..2 = |c| rank)."""
    idx = np.asarray(idx, dtype=np.int64)
    return np.where(idx >= 8, idx - 8, 8 | (7 - idx)).astype(np.uint8)


def turbo4_index(nib):
    """Inverse of turbo4_nibble."""
    nib = np.asarray(nib, dtype=np.int64)
    mag = nib & 7
    return np.where(nib & 8, 7 - mag, 8 + mag).astype(np.uint8)


def _sub3_fields():
    """For each of the 32 codes of a turbo3 sub-block: [(word, bit, width, code_shift), ...]."""
    f = []
    for e in range(32):
        j = e % 4
        if e < 4:
            f.append([(0, 8 * j, 3, 0)])
        elif e < 8:
            f.append([(0, 8 * j + 3, 3, 0)])
        elif e < 12:
            f.append([(1, 8 * j, 3, 0)])
        elif e < 16:
            f.append([(1, 8 * j + 3, 3, 0)])
        elif e < 20:
            f.append([(2, 8 * j, 3, 0)])
        elif e < 24:
            f.append([(2, 8 * j + 3, 3, 0)])
        elif e < 28:
            f.append([(0, 8 * j + 6, 2, 0), (2, 8 * j + 6, 1, 2)])
        else:
            f.append([(1, 8 * j + 6, 2, 0), (2, 8 * j + 7, 1, 2)])
    return f


SUB3_FIELDS = _sub3_fields()


def _words_to_bytes(words):
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(words.shape[:-1] + (-1,))


def _bytes_to_words(b):
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    return b.view("<u4").reshape(b.shape[:-1] + (-1,)).astype(np.int64)


def pack_sub3(codes32) -> np.ndarray:
    """32 three-bit codes [..., 32] -> 12 bytes [..., 12]."""
    c = np.asarray(codes32, dtype=np.int64)
    words = np.zeros(c.shape[:-1] + (3,), dtype=np.int64)
    for e, fields in enumerate(SUB3_FIELDS):
        for word, bit, width, shift in fields:
            words[..., word] |= ((c[..., e] >> shift) & ((1 << width) - 1)) << bit
    return _words_to_bytes(words)


def unpack_sub3(b12) -> np.ndarray:
    w = _bytes_to_words(b12)
    out = np.zeros(w.shape[:-1] + (32,), dtype=np.int64)
    for e, fields in enumerate(SUB3_FIELDS):
        for word, bit, width, shift in fields:
            out[..., e] |= ((w[..., word] >> bit) & ((1 << width) - 1)) << shift
    return out.astype(np.uint8)


def pack_oct4(codes8) -> np.ndarray:
    """8 four-bit ascending indices [..., 8] -> 4 bytes [..., 4] (sign-magnitude nibbles)."""
    nib = turbo4_nibble(codes8).astype(np.int64)
    word = np.zeros(nib.shape[:-1], dtype=np.int64)
    for e in range(8):
        bit = 8 * e if e < 4 else 8 * (e - 4) + 4
        word |= nib[..., e] << bit
    return _words_to_bytes(word[..., None])


def unpack_oct4(b4) -> np.ndarray:
    w = _bytes_to_words(b4)[..., 0]
    nib = np.zeros(w.shape + (8,), dtype=np.int64)
    for e in range(8):
        bit = 8 * e if e < 4 else 8 * (e - 4) + 4
        nib[..., e] = (w >> bit) & 15
    return turbo4_index(nib)


def pack_k_record(codes, fmt: str) -> np.ndarray:
    """Token-major K record: codes [..., 128] -> bytes [..., 48 | 64]."""
    c = np.asarray(codes)
    if fmt == "turbo3":
        return np.concatenate([pack_sub3(c[..., 32 * q:32 * q + 32]) for q in range(4)], axis=-1)
    if fmt == "turbo4":
        return np.concatenate([pack_oct4(c[..., 8 * w:8 * w + 8]) for w in range(16)], axis=-1)
    raise ValueError(fmt)


def unpack_k_record(rec, fmt: str) -> np.ndarray:
    r = np.asarray(rec, dtype=np.uint8)
    if fmt == "turbo3":
        return np.concatenate([unpack_sub3(r[..., 12 * q:12 * q + 12]) for q in range(4)], axis=-1)
    if fmt == "turbo4":
        return np.concatenate([unpack_oct4(r[..., 4 * w:4 * w + 4]) for w in range(16)], axis=-1)
    raise ValueError(fmt)


K_BLOCK_TOKENS = 16   # quantised K records are interleaved in pieces over blocks of this many tokens


def k_records_to_memory(records, fmt: str) -> np.ndarray:
    """Records [..., T, bytes] (T a multiple of 16) -> the bytes in memory order, same shape.

    turbo4: piece p (record bytes 16p..16p+15) of token 16 b + i at byte 1024 b + 256 p + 16 i.
    turbo3: piece q (sub-block q, record bytes 12q..12q+11) of token 16 b + i at byte
    768 b + 384 (q % 2) + 192 (q // 2) + 12 i."""
    r = np.asarray(records, dtype=np.uint8)
    if fmt not in ("turbo3", "turbo4"):
        return r.copy()
    T = r.shape[-2]
    if T % K_BLOCK_TOKENS:
        raise ValueError("token count must be a multiple of 16")
    nb = T // K_BLOCK_TOKENS
    if fmt == "turbo4":
        blk = r.reshape(r.shape[:-2] + (nb, K_BLOCK_TOKENS, 4, 16))               # [.., blocks, i, p, 16]
        return np.ascontiguousarray(np.swapaxes(blk, -3, -2)).reshape(r.shape)    # [.., blocks, p, i, 16]
    blk = r.reshape(r.shape[:-2] + (nb, K_BLOCK_TOKENS, 2, 2, 12))                # [.., blocks, i, q//2, q%2, 12]
    mem = np.moveaxis(blk, (-4, -3, -2), (-2, -3, -4))                            # [.., blocks, q%2, q//2, i, 12]
    return np.ascontiguousarray(mem).reshape(r.shape)


def k_memory_to_records(mem, fmt: str) -> np.ndarray:
    """Inverse of k_records_to_memory."""
    m = np.asarray(mem, dtype=np.uint8)
    if fmt not in ("turbo3", "turbo4"):
        return m.copy()
    T = m.shape[-2]
    nb = T // K_BLOCK_TOKENS
    if fmt == "turbo4":
        blk = m.reshape(m.shape[:-2] + (nb, 4, K_BLOCK_TOKENS, 16))               # [.., blocks, p, i, 16]
        return np.ascontiguousarray(np.swapaxes(blk, -3, -2)).reshape(m.shape)
    blk = m.reshape(m.shape[:-2] + (nb, 2, 2, K_BLOCK_TOKENS, 12))                # [.., blocks, q%2, q//2, i, 12]
    rec = np.moveaxis(blk, (-4, -3, -2), (-2, -3, -4))                            # [.., blocks, i, q//2, q%2, 12]
    return np.ascontiguousarray(rec).reshape(m.shape)


def v_tile_slot(g: int, i: int) -> int:
    """Tile slot (0..31) of element-token i (0..7) in slot group g (0..3)."""
    return 16 * (i // 4) + 4 * g + (i % 4)


def _v_chunk_elements(codes_tile):
    """codes_tile [..., 32, 128] -> chunk elements [..., 64 chunks, 64 elements] (same dtype)."""
    c = np.asarray(codes_tile)
    out = np.zeros(c.shape[:-2] + (64, 64), dtype=c.dtype)
    for g in range(4):
        for n in range(16):
            for nb in range(8):
                for i in range(8):
                    out[..., 16 * g + n, 8 * nb + i] = c[..., v_tile_slot(g, i), 8 * n + nb]
    return out


def _v_chunk_elements_inverse(elems):
    e = np.asarray(elems)
    out = np.zeros(e.shape[:-2] + (32, 128), dtype=e.dtype)
    for g in range(4):
        for n in range(16):
            for nb in range(8):
                for i in range(8):
                    out[..., v_tile_slot(g, i), 8 * n + nb] = e[..., 16 * g + n, 8 * nb + i]
    return out


def pack_v_tiles(codes, fmt: str) -> np.ndarray:
    """Token-tiled V: codes [T, 128] (T a multiple of 32) -> bytes [T/32, 1536 | 2048].

    fmt "f16": the uncompressed comparison layout -- the same chunk element order
    with fp16 values for codes (128-byte chunks, 8192-byte tiles)."""
    c = np.asarray(codes)
    if c.shape[-2] % V_TILE_TOKENS:
        raise ValueError("token count must be a multiple of 32")
    tiles = c.reshape(c.shape[:-2] + (c.shape[-2] // V_TILE_TOKENS, V_TILE_TOKENS, HEAD_DIM))
    el = _v_chunk_elements(tiles)                                  # [..., nt, 64, 64]
    if fmt == "turbo3":
        chunk = np.concatenate([pack_sub3(el[..., :32]), pack_sub3(el[..., 32:])], axis=-1)
        # two 12-byte pieces (sub-blocks) per chunk: piece p of chunk c at tile byte 768 p + 12 c
        pieces = np.swapaxes(chunk.reshape(chunk.shape[:-1] + (2, 12)), -3, -2)  # [.., nt, p, c, 12]
        return np.ascontiguousarray(pieces).reshape(chunk.shape[:-2] + (-1,))
    elif fmt == "turbo4":
        chunk = np.concatenate([pack_oct4(el[..., 8 * nb:8 * nb + 8]) for nb in range(8)], axis=-1)
        # two 16-byte pieces per chunk: piece p of chunk c at tile byte 1024 p + 16 c
        pieces = np.swapaxes(chunk.reshape(chunk.shape[:-1] + (2, 16)), -3, -2)  # [.., nt, p, c, 16]
        return np.ascontiguousarray(pieces).reshape(chunk.shape[:-2] + (-1,))
    elif fmt == "f16":
        chunk = np.ascontiguousarray(el).view(np.uint8)                # 64 little-endian fp16 values
    else:
        raise ValueError(fmt)
    return chunk.reshape(chunk.shape[:-2] + (-1,))


def unpack_v_tiles(tiles, fmt: str) -> np.ndarray:
    """Inverse of pack_v_tiles: bytes [nt, tile bytes] -> codes [nt*32, 128]."""
    t = np.asarray(tiles, dtype=np.uint8)
    cb = V_CHUNK_BYTES[fmt]
    if fmt in ("turbo3", "turbo4"):   # pieces back into chunks
        pb = cb // 2
        ch = np.swapaxes(t.reshape(t.shape[:-1] + (2, 64, pb)), -3, -2).reshape(t.shape[:-1] + (64, cb))
    else:
        ch = t.reshape(t.shape[:-1] + (64, cb))
    if fmt == "turbo3":
        el = np.concatenate([unpack_sub3(ch[..., :12]), unpack_sub3(ch[..., 12:])], axis=-1)
    elif fmt == "f16":
        el = np.ascontiguousarray(ch).view(np.float16)                  # [..., 64, 64]
    else:
        el = np.concatenate([unpack_oct4(ch[..., 4 * nb:4 * nb + 4]) for nb in range(8)], axis=-1)
    codes = _v_chunk_elements_inverse(el)                            # [..., nt, 32, 128]
    return codes.reshape(codes.shape[:-3] + (-1, HEAD_DIM))


# ----------------------------------------------------------------------------- dequant

def dequant_rotated(codes, norms16, codebook16) -> np.ndarray:
    """Rotated-basis reconstruction n * c[idx] (float64), as used by the rotated attention path."""
    cb = np.asarray(codebook16, dtype=np.float16).astype(np.float64)
    return np.asarray(norms16, dtype=np.float16).astype(np.float64)[..., None] * cb[np.asarray(codes, dtype=np.int64)]


def dequant(codes, norms16, codebook16, signs) -> np.ndarray:
    """Full reconstruction in the original basis: s * H (n * c[idx]) / sqrt(128) (float64)."""
    return inverse_rotate(dequant_rotated(codes, norms16, codebook16), signs)
