"""Pins for the oracle's decode attention (full-dequant definition, rotated identity, LSE merge)."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import codec
from synth import sign_vector
from tests.conftest import load_codebook

SCALE = 1 / np.sqrt(128)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_vectorised_equals_naive_loops():
    rng = np.random.default_rng(0)
    q = _rand(rng, 2, 4, 128)
    k = _rand(rng, 2, 2, 9, 128)
    v = _rand(rng, 2, 2, 9, 128)
    lengths = [9, 5]
    np.testing.assert_allclose(att.attention(q, k, v, lengths, SCALE),
                               att.attention_naive(q.tolist(), k.tolist(), v.tolist(), lengths, SCALE),
                               rtol=0, atol=1e-13)


def test_matches_torch_sdpa_float64_gqa():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, L = 2, 8, 2, 33
    q = _rand(rng, B, Hq, 128)
    k = _rand(rng, B, Hkv, L, 128)
    v = _rand(rng, B, Hkv, L, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, :, None, :],
        torch.tensor(k).repeat_interleave(Hq // Hkv, dim=1),
        torch.tensor(v).repeat_interleave(Hq // Hkv, dim=1), scale=SCALE)[:, :, 0, :].numpy()
    np.testing.assert_allclose(att.attention(q, k, v, [L, L], SCALE), ref, rtol=0, atol=1e-13)


def test_special_cases():
    rng = np.random.default_rng(2)
    q = _rand(rng, 1, 2, 128)
    k = _rand(rng, 1, 1, 6, 128)
    v = _rand(rng, 1, 1, 6, 128)
    # one visible token -> that token's value
    np.testing.assert_allclose(att.attention(q, k, v, [1], SCALE)[0, 0], v[0, 0, 0], atol=1e-15, rtol=0)
    # identical keys -> mean of the values
    kk = np.repeat(k[:, :, :1], 6, axis=2)
    np.testing.assert_allclose(att.attention(q, kk, v, [6], SCALE)[0, 1], v[0, 0].mean(0), atol=1e-14, rtol=0)
    # zero query -> uniform mean
    np.testing.assert_allclose(att.attention(np.zeros_like(q), k, v, [6], SCALE)[0, 0], v[0, 0].mean(0),
                               atol=1e-14, rtol=0)
    # one dominant score -> that value
    kd = k.copy()
    kd[0, 0, 3] = q[0, 0] * 1e3
    np.testing.assert_allclose(att.attention(q, kd, v, [6], SCALE)[0, 0], v[0, 0, 3], atol=1e-12, rtol=0)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(3)
    q = _rand(rng, 1, 6, 128)
    k = _rand(rng, 1, 3, 7, 128)
    v = _rand(rng, 1, 3, 7, 128)
    a = att.attention(q, k, v, [7], SCALE)
    b = att.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), [7], SCALE)
    np.testing.assert_allclose(a, b, atol=1e-15, rtol=0)


@pytest.mark.parametrize("parts", [[0, 40], [0, 1, 40], [0, 7, 8, 31, 40], [0, 20, 20, 40]])
def test_split_lse_merge_equals_unsplit(parts):
    rng = np.random.default_rng(4)
    q = _rand(rng, 3, 128) * 3
    k = _rand(rng, 40, 128)
    v = _rand(rng, 40, 128)
    ref = att.attention(q[None], k[None, None].repeat(3, 1), v[None, None].repeat(3, 1), [40], SCALE)[0]
    ps = [att.partial(q, k[a:b], v[a:b], SCALE) for a, b in zip(parts[:-1], parts[1:])]
    np.testing.assert_allclose(att.combine(ps), ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kfmt,vfmt", [("turbo3", "turbo3"), ("turbo4", "turbo4"), ("f16", "turbo4")])
def test_rotated_route_equals_full_dequant(kfmt, vfmt, codebooks):
    """rotate(SDPA(q,k,v)) == SDPA(q,k,rotate(v)) on dequantised caches, GQA 4 query over 2 KV heads."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, L = 2, 4, 2, 50
    sk, sv = sign_vector(0, "k"), sign_vector(0, "v")
    k16 = rng.standard_normal((B, Hkv, L, 128)).astype(np.float16)
    v16 = rng.standard_normal((B, Hkv, L, 128)).astype(np.float16)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float16)
    vc, vn = codec.encode(v16, sv, codebooks[vfmt])
    v_hat = codec.dequant(vc, vn, codebooks[vfmt], sv)
    lengths = [L, 31]
    if kfmt == "f16":
        kc = kn = None
        k_hat = k16.astype(np.float64)
        k_f16 = k16
    else:
        kc, kn = codec.encode(k16, sk, codebooks[kfmt])
        k_hat = codec.dequant(kc, kn, codebooks[kfmt], sk)
        k_f16 = None
    full = att.attention(q, k_hat, v_hat, lengths, SCALE)
    rot = att.attention_rotated(q, kc, kn, vc, vn, lengths, SCALE,
                                codebooks.get(kfmt), codebooks[vfmt], sk, sv, k_f16=k_f16)
    np.testing.assert_allclose(rot, full, rtol=0, atol=1e-12 * np.abs(full).max())


def test_reference_glue_round_trips_through_the_layout(codebooks):
    from oracle import reference as ref
    from synth import get_workload, kv_slice, queries
    w = get_workload(0)
    sk, sv = sign_vector(0, "k"), sign_vector(0, "v")
    k16 = np.stack([kv_slice(w, 0, "k", 0, h, 256) for h in range(2)])
    v16 = np.stack([kv_slice(w, 0, "v", 0, h, 256) for h in range(2)])
    enc = ref.encode_sequence(k16, v16, "turbo3", "turbo3", sk, sv, codebooks)
    kc, vc = ref.codes_from_library_layout(enc["k_rec"], enc["v_tiles"], "turbo3", "turbo3")
    np.testing.assert_array_equal(kc, enc["k_codes"])
    np.testing.assert_array_equal(vc, enc["v_codes"])
    k_hat, v_hat = ref.dequant_sequence(enc, "turbo3", "turbo3", sk, sv, codebooks, 256)
    q = queries(w, 0)[0]
    o = ref.decode_sequence(q, k_hat, v_hat, 256)
    o_exact = att.attention(q[None], [k16.astype(np.float64)], [v16.astype(np.float64)], [256], SCALE)[0]
    # 3-bit codes: the quantised attention stays close to the unquantised one
    assert np.linalg.norm(o - o_exact) / np.linalg.norm(o_exact) < 0.5


def test_sparse_v_bound_hand_example():
    """Three tokens, one KV head, two query heads, D = 1: scores (scale 1) of head 0 are
    0, -20, -1 and of head 1 are 0, -30, -40.  Relative weights: head 0 [1, e^-20, e^-1],
    head 1 [1, e^-30, e^-40].  At tau = 1e-6 only token 1 is below tau for both heads
    (token 2 is not, for head 0), so the bound is w_{h,1} |v_1| per head."""
    from oracle.attention import sparse_v_bound
    # scores are q.k: with q = 1, K holds the wanted scores, one head at a time
    k0 = np.array([[[0.0], [-20.0], [-1.0]]])         # [Hkv=1, L=3, D=1]
    k1 = np.array([[[0.0], [-30.0], [-40.0]]])
    v = np.array([[[2.0], [-3.0], [5.0]]])
    for kk, rel in ((k0, [1.0, np.exp(-20.0), np.exp(-1.0)]), (k1, [1.0, np.exp(-30.0), np.exp(-40.0)])):
        o, b = sparse_v_bound(np.array([[1.0]]), kk, v, 3, 1.0, 1e-6)
        w = np.array(rel) / sum(rel)
        np.testing.assert_allclose(o[0, 0], w @ v[0, :, 0], rtol=1e-15)
    # both heads together: head 0 on k0-scores and head 1 on k1-scores need one K per head,
    # so use two-dimensional K with q selecting the coordinate
    k = np.concatenate([k0, k1], axis=2)              # [1, 3, 2]
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    vv = np.repeat(v, 2, axis=2)
    o, b = sparse_v_bound(q, k, vv, 3, 1.0, 1e-6)
    w0 = np.array([1.0, np.exp(-20.0), np.exp(-1.0)])
    w0 /= w0.sum()
    w1 = np.array([1.0, np.exp(-30.0), np.exp(-40.0)])
    w1 /= w1.sum()
    np.testing.assert_allclose(b[0], [w0[1] * 3.0] * 2, rtol=1e-12)
    np.testing.assert_allclose(b[1], [w1[1] * 3.0] * 2, rtol=1e-12)
    # tau = 0 drops nothing; tau = 1 drops every token that is nobody's maximum
    _, b0 = sparse_v_bound(q, k, vv, 3, 1.0, 0.0)
    assert np.all(b0 == 0)
    _, b1 = sparse_v_bound(q, k, vv, 3, 1.0, 1.0)
    np.testing.assert_allclose(b1[0], [w0[1] * 3.0 + w0[2] * 5.0] * 2, rtol=1e-12)


def test_sparse_v_bound_covers_any_dropped_subset():
    """Dropping any subset of the droppable tokens from the p.v sum (the softmax sum
    unchanged) moves o by at most the bound; o is the exact attention."""
    from oracle.attention import attention, sparse_v_bound
    rng = np.random.default_rng(3)
    hkv, G, L, D = 2, 3, 200, 16
    k = rng.standard_normal((hkv, L, D)) * 3.0
    v = rng.standard_normal((hkv, L, D))
    q = rng.standard_normal((hkv * G, D)) * 3.0
    tau = 1e-3
    o, bound = sparse_v_bound(q, k, v, L, 0.5, tau)
    np.testing.assert_allclose(o, attention(q[None], [k], [v], [L], 0.5)[0], rtol=1e-12, atol=1e-14)
    for h in range(hkv * G):
        g = h // G
        z = np.stack([0.5 * (k[g] @ q[hh]) for hh in range(g * G, (g + 1) * G)])
        rel = np.exp(z - z.max(axis=1, keepdims=True))
        droppable = np.all(rel < tau, axis=0)
        assert droppable.any()
        w = rel[h - g * G] / rel[h - g * G].sum()
        for trial in range(5):
            drop = droppable & (rng.random(L) < 0.5)
            o_drop = (w * ~drop) @ v[g]
            assert np.all(np.abs(o_drop - o[h]) <= bound[h] + 1e-15)


def test_sparse_k_bound_hand_example():
    """Three tokens, one KV head, one query head, D = 1, scale 1: scores 0, -20, -1,
    values 2, -3, 5.  At tau = 1e-6 token 1 is droppable (weight ratio e^-20) and token 2
    is not.  Dropping token 1 gives o' = (2 + 5 e^-1) / (1 + e^-1) exactly; the bound is
    (D |o| + w_1 |v_1|) / (1 - D) with D = w_1, and it is attained up to rounding by that
    drop when o and -v_1 have the same sign (here o > 0, v_1 = -3)."""
    from oracle.attention import sparse_k_bound
    k = np.array([[[0.0], [-20.0], [-1.0]]])
    v = np.array([[[2.0], [-3.0], [5.0]]])
    o, b = sparse_k_bound(np.array([[1.0]]), k, v, 3, 1.0, 1e-6)
    rel = np.array([1.0, np.exp(-20.0), np.exp(-1.0)])
    w = rel / rel.sum()
    np.testing.assert_allclose(o[0, 0], w @ v[0, :, 0], rtol=1e-15)
    d = w[1]
    np.testing.assert_allclose(b[0, 0], (d * abs(o[0, 0]) + d * 3.0) / (1 - d), rtol=1e-12)
    o_drop = (2.0 + 5.0 * np.exp(-1.0)) / (1.0 + np.exp(-1.0))
    np.testing.assert_allclose(abs(o_drop - o[0, 0]), b[0, 0], rtol=1e-6)
    # tau = 0: nothing droppable; tau = 1: everything but the maximum
    _, b0 = sparse_k_bound(np.array([[1.0]]), k, v, 3, 1.0, 0.0)
    assert np.all(b0 == 0)
    _, b1 = sparse_k_bound(np.array([[1.0]]), k, v, 3, 1.0, 1.0)
    d1 = w[1] + w[2]
    np.testing.assert_allclose(b1[0, 0], (d1 * abs(o[0, 0]) + w[1] * 3.0 + w[2] * 5.0) / (1 - d1), rtol=1e-12)
    assert abs(2.0 - o[0, 0]) <= b1[0, 0]   # o' = v_0 (not attained: v_2 has o's sign)


def test_sparse_k_bound_covers_any_dropped_subset():
    """Removing any subset of the droppable tokens from the whole softmax (scores, sum and
    p.v) moves o by at most the bound."""
    from oracle.attention import attention, sparse_k_bound
    rng = np.random.default_rng(5)
    hkv, G, L, D = 2, 3, 200, 16
    k = rng.standard_normal((hkv, L, D)) * 3.0
    v = rng.standard_normal((hkv, L, D))
    q = rng.standard_normal((hkv * G, D)) * 3.0
    tau = 1e-3
    o, bound = sparse_k_bound(q, k, v, L, 0.5, tau)
    np.testing.assert_allclose(o, attention(q[None], [k], [v], [L], 0.5)[0], rtol=1e-12, atol=1e-14)
    for h in range(hkv * G):
        g = h // G
        z = np.stack([0.5 * (k[g] @ q[hh]) for hh in range(g * G, (g + 1) * G)])
        rel = np.exp(z - z.max(axis=1, keepdims=True))
        droppable = np.all(rel < tau, axis=0)
        assert droppable.any()
        zh = z[h - g * G]
        for trial in range(5):
            keep = ~(droppable & (rng.random(L) < 0.5))
            wk = np.exp(zh[keep] - zh.max())
            o_drop = (wk / wk.sum()) @ v[g][keep]
            assert np.all(np.abs(o_drop - o[h]) <= bound[h] * (1 + 1e-12) + 1e-15)


def test_score_upper_bound_holds_and_is_attained():
    """Cauchy-Schwarz: every score over random codes stays below the norm-only bound, and
    the bound is reached by the code that puts the largest-magnitude entry, with q's sign,
    on every coordinate of a q whose entries all have one magnitude."""
    from oracle.attention import score_upper_bound
    from oracle.hadamard import rotate
    rng = np.random.default_rng(6)
    for name in ("turbo3", "turbo4"):
        cb = load_codebook(name).astype(np.float64)
        for trial in range(50):
            q = rng.standard_normal(128) * rng.uniform(0.1, 10.0)
            n = rng.uniform(0.0, 50.0)
            idx = rng.integers(0, len(cb), 128)
            qr = rotate(q, sign_vector(0, "k"))
            z = SCALE * n * (qr @ cb[idx])
            assert z <= score_upper_bound(q, n, cb, SCALE) * (1 + 1e-12)
        qe = np.where(rng.random(128) < 0.5, -2.5, 2.5)
        best = np.where(qe > 0, np.argmax(cb), np.argmin(cb))
        np.testing.assert_allclose(SCALE * 3.0 * (qe @ cb[best]), score_upper_bound(qe, 3.0, cb, SCALE), rtol=1e-12)


def test_chunk_attention_is_causal_and_reduces_to_single_token():
    """Tq = 1 is the single-token decode; position tau of a chunk depends on exactly the first
    L - Tq + 1 + tau tokens (changing a later token leaves it unchanged, changing that token
    does not); brute force with Python loops on a tiny chunk."""
    from oracle.attention import attention, attention_chunk, attention_naive
    rng = np.random.default_rng(11)
    B, hkv, G, L, D, Tq = 2, 2, 3, 9, 8, 4
    k = [rng.standard_normal((hkv, L, D)) for _ in range(B)]
    v = [rng.standard_normal((hkv, L, D)) for _ in range(B)]
    q = rng.standard_normal((B, hkv * G, Tq, D))
    lens = [L, L - 2]
    o = attention_chunk(q, k, v, lens, 0.3)
    np.testing.assert_allclose(attention_chunk(q[:, :, :1], k, v, lens, 0.3)[:, :, 0],
                               attention(q[:, :, 0], k, v, lens, 0.3), rtol=0, atol=0)
    for b in range(B):
        for tau in range(Tq):
            n = lens[b] - Tq + 1 + tau
            ref = attention_naive(q[b:b + 1, :, tau].tolist(), [k[b].tolist()], [v[b].tolist()], [n], 0.3)[0]
            np.testing.assert_allclose(o[b, :, tau], ref, rtol=1e-12, atol=1e-14)
            k2 = [x.copy() for x in k]
            v2 = [x.copy() for x in v]
            if n < L:
                k2[b][:, n:] += 5.0
                v2[b][:, n:] -= 3.0
                np.testing.assert_allclose(attention_chunk(q, k2, v2, lens, 0.3)[b, :, tau], o[b, :, tau],
                                           rtol=0, atol=0)
            v2[b][:, n - 1] += 1.0
            assert np.all(np.abs(attention_chunk(q, k2, v2, lens, 0.3)[b, :, tau] - o[b, :, tau]) > 0)
