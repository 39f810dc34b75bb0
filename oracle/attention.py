"""Single-token decode attention over the dequantised cache (float64).

The result the decode path must reach is plain softmax attention of each
query head over every visible token of its KV head, with K and V fully
dequantised in the original basis: mlxcel PR #369 compares its rotated route
against exactly this ("Result": the full-dequant reference, update_and_fetch +
SDPA, GQA 4 query heads over 2 KV heads).  Query head h reads KV head
h // (Hq / Hkv) (contiguous GQA groups, as SDPA's head broadcast).

The rotated route of the same PR ("Change"; identity
rotate(SDPA(q,k,v)) == SDPA(q,k,rotate(v))) and the split/log-sum-exp merge
are written out too, as self-checks of that identity, not as the definition.
"""
import numpy as np

from .codec import dequant_rotated
from .hadamard import inverse_rotate, rotate


def attention(q, k_hat, v_hat, lengths, scale: float) -> np.ndarray:
    """o[b, h] = sum_t softmax_t(scale * q[b,h] . k_hat[b,g,t]) v_hat[b,g,t], t < lengths[b].

    q [B, Hq, D]; k_hat, v_hat: per-sequence arrays [Hkv, L_b, D] (a list of B)
    or one array [B, Hkv, Lmax, D].  float64 throughout; returns [B, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        kb = np.asarray(k_hat[b], dtype=np.float64)
        vb = np.asarray(v_hat[b], dtype=np.float64)
        hkv = kb.shape[0]
        group = Hq // hkv
        L = int(lengths[b])
        for h in range(Hq):
            g = h // group
            z = scale * (kb[g, :L] @ q[b, h])
            p = np.exp(z - z.max())
            p /= p.sum()
            out[b, h] = p @ vb[g, :L]
    return out


def attention_naive(q, k_hat, v_hat, lengths, scale: float) -> np.ndarray:
    """The same definition with explicit Python loops (for tiny inputs only)."""
    import math
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        hkv = len(k_hat[b])
        group = Hq // hkv
        L = int(lengths[b])
        for h in range(Hq):
            g = h // group
            z = [scale * sum(float(q[b][h][i]) * float(k_hat[b][g][t][i]) for i in range(D)) for t in range(L)]
            mx = max(z)
            w = [math.exp(v - mx) for v in z]
            s = sum(w)
            for i in range(D):
                out[b][h][i] = sum(w[t] * float(v_hat[b][g][t][i]) for t in range(L)) / s
    return np.array(out)


def partial(q_rows, k_rows, v_rows, scale: float):
    """Unnormalised partial over one token range: (m, l, o) with
    m = max z, l = sum exp(z - m), o = sum exp(z - m) v (o not divided by l)."""
    z = scale * (np.asarray(k_rows, dtype=np.float64) @ np.asarray(q_rows, dtype=np.float64).T)  # [T, G]
    if z.shape[0] == 0:
        g = np.asarray(q_rows).shape[0]
        return np.full(g, -np.inf), np.zeros(g), np.zeros((g, np.asarray(v_rows).shape[-1]))
    m = z.max(axis=0)
    w = np.exp(z - m)
    return m, w.sum(axis=0), w.T @ np.asarray(v_rows, dtype=np.float64)


def combine(partials):
    """Log-sum-exp merge of (m, l, o) partials of disjoint token ranges -> normalised output."""
    ms = np.stack([p[0] for p in partials])        # [S, G]
    M = ms.max(axis=0)
    scale = np.where(np.isfinite(ms), np.exp(ms - M), 0.0)
    L = sum(s * p[1] for s, p in zip(scale, partials))
    O = sum(s[:, None] * p[2] for s, p in zip(scale, partials))
    return O / L[:, None]


def attention_rotated(q, k_codes, k_norms, v_codes, v_norms, lengths, scale, k_codebook, v_codebook,
                      k_signs, v_signs, k_f16=None) -> np.ndarray:
    """Rotated route: scores against n_K * c[idx_K] with q rotated into K's basis
    (or against raw fp16 K when k_f16 is given), values accumulated as
    n_V * c[idx_V] in V's rotated basis, then only the output is inverse-rotated.

    Codes/norms: per-sequence arrays [Hkv, L_b, 128] / [Hkv, L_b] (lists of B)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    out_rot = np.zeros((B, Hq, D))
    for b in range(B):
        if k_f16 is None:
            kb = dequant_rotated(k_codes[b], k_norms[b], k_codebook)
            qb = rotate(q[b], k_signs)
        else:
            kb = np.asarray(k_f16[b], dtype=np.float64)
            qb = q[b]
        vb = dequant_rotated(v_codes[b], v_norms[b], v_codebook)
        hkv = vb.shape[0]
        group = Hq // hkv
        L = int(lengths[b])
        for h in range(Hq):
            g = h // group
            z = scale * (kb[g, :L] @ qb[h])
            p = np.exp(z - z.max())
            out_rot[b, h] = (p / p.sum()) @ vb[g, :L]
    return inverse_rotate(out_rot, v_signs)


def sparse_v_bound(q, k_hat, v_hat, length, scale: float, tau: float):
    """What sparse V may drop from one sequence's attention (float64).

    The V-side skip (turboquant_plus "SMEM Pre-Dequant Experiment", idea 2 "Sparse K
    attention", which names the existing SPARSE_V skip of V work for negligible
    weights; mlxcel PR #369, commit "docs(cache): add ADR 0002 ... (sparse-V study)":
    exact below fp16 round-off at tau = 1e-6) leaves the scores and the softmax sum
    alone and drops only p_t v_t terms.  A decoder may drop token t of KV head g only
    when every query head of g gives it a weight below tau relative to that head's
    largest weight.  Returns (o, bound): o [Hq, D] the exact attention, and bound
    [Hq, D] = sum over such tokens t of w_{h,t} |v_{g,t}| (w the normalised weights),
    the most any choice of dropped tokens can move o.

    q [Hq, D]; k_hat, v_hat [Hkv, L, D]."""
    q = np.asarray(q, dtype=np.float64)
    kb = np.asarray(k_hat, dtype=np.float64)
    vb = np.asarray(v_hat, dtype=np.float64)
    Hq, D = q.shape
    hkv = kb.shape[0]
    group = Hq // hkv
    L = int(length)
    o = np.zeros((Hq, D))
    bound = np.zeros((Hq, D))
    for g in range(hkv):
        heads = range(g * group, (g + 1) * group)
        rel = np.stack([np.exp(scale * (kb[g, :L] @ q[h]) - (scale * (kb[g, :L] @ q[h])).max()) for h in heads])
        droppable = np.all(rel < tau, axis=0)          # [L]
        for i, h in enumerate(heads):
            w = rel[i] / rel[i].sum()
            o[h] = w @ vb[g, :L]
            bound[h] = (w * droppable) @ np.abs(vb[g, :L])
    return o, bound


def sparse_k_bound(q, k_hat, v_hat, length, scale: float, tau: float):
    """What a K-side skip may drop from one sequence's attention (float64).

    turboquant_plus "SMEM Pre-Dequant Experiment", idea 2 "Sparse K attention": skip
    the K work of positions whose attention contribution is negligible, decided from
    a cheap estimate such as the stored norm (here: score_upper_bound, an upper
    bound, so the estimate never lets a significant token go).  Unlike sparse V a
    skipped token leaves the scores, the softmax sum and the p.v sum alike.  A decoder
    may drop token t of KV head g only when every query head of g gives it a weight
    below tau relative to that head's largest weight (the same tokens sparse_v_bound
    calls droppable).  With w the weights normalised over all tokens, D = sum of w over
    the dropped tokens and o the exact output, the output of the kept tokens is
    o' = (o - sum_drop w v) / (1 - D), so |o' - o| <= (D |o| + sum_drop w |v|) / (1 - D),
    which only grows with the dropped set.  Returns (o, bound): o [Hq, D] the exact
    attention, bound [Hq, D] that expression with every droppable token dropped.

    q [Hq, D]; k_hat, v_hat [Hkv, L, D]."""
    q = np.asarray(q, dtype=np.float64)
    kb = np.asarray(k_hat, dtype=np.float64)
    vb = np.asarray(v_hat, dtype=np.float64)
    Hq, D = q.shape
    hkv = kb.shape[0]
    group = Hq // hkv
    L = int(length)
    o = np.zeros((Hq, D))
    bound = np.zeros((Hq, D))
    for g in range(hkv):
        heads = range(g * group, (g + 1) * group)
        rel = np.stack([np.exp(scale * (kb[g, :L] @ q[h]) - (scale * (kb[g, :L] @ q[h])).max()) for h in heads])
        droppable = np.all(rel < tau, axis=0)          # [L]
        for i, h in enumerate(heads):
            w = rel[i] / rel[i].sum()
            o[h] = w @ vb[g, :L]
            d = float(w[droppable].sum())
            bound[h] = (d * np.abs(o[h]) + (w * droppable) @ np.abs(vb[g, :L])) / (1.0 - d)
    return o, bound


def score_upper_bound(q_row, k_norm, codebook, scale: float) -> float:
    """An upper bound on the score of one query row against any token whose stored
    norm is k_norm, whatever its codes: the token's dequantised K row in the rotated
    basis is k_norm * c[idx], every entry at most max|c| in magnitude, so by
    Cauchy-Schwarz (the rotation keeps q's length)
    scale * q . k_hat <= scale * |q| * k_norm * sqrt(D) * max|c|.
    This is the norm-only estimate turboquant_plus "SMEM Pre-Dequant Experiment",
    idea 2, asks for, made one-sided: a token whose bound is already below
    (running max + ln tau) for every head of its KV head has a weight below tau."""
    q = np.asarray(q_row, dtype=np.float64)
    c = np.asarray(codebook, dtype=np.float64)
    return float(scale * np.sqrt(q @ q) * float(k_norm) * np.sqrt(q.shape[0]) * np.abs(c).max())


def attention_chunk(q, k_hat, v_hat, lengths, scale: float) -> np.ndarray:
    """Decode attention of a chunk of Tq query positions per sequence (float64).

    Decode with Tq > 1 query positions (speculative verification, chunked decode;
    mlxcel PR #369 "Change" shapes the decode output [B, Hq, Tq, D]; the chunk's own
    tokens are the last Tq of the cache and are causal among themselves): query position tau of sequence b
    (0 <= tau < Tq) sits at absolute position L_b - Tq + tau and attends to tokens
    t <= L_b - Tq + tau, i.e. to the first L_b - Tq + 1 + tau tokens.

    q [B, Hq, Tq, D]; k_hat, v_hat as for `attention`; lengths[b] >= Tq.
    Returns [B, Hq, Tq, D]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Tq, D = q.shape
    out = np.zeros((B, Hq, Tq, D))
    for b in range(B):
        L = int(lengths[b])
        assert L >= Tq, "the chunk's tokens must be in the cache"
        for tau in range(Tq):
            out[b, :, tau] = attention(q[b:b + 1, :, tau], [k_hat[b]], [v_hat[b]], [L - Tq + 1 + tau], scale)[0]
    return out
