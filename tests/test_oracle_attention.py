"""Pins for the oracle's decode attention (full-dequant definition, rotated identity, LSE merge)."""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import codec
from synth import sign_vector

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
