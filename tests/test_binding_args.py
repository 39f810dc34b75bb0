"""The Python binding rejects mis-shaped, mistyped, strided or host tensors with ValueError
before the library is called (the C ABI takes bare device pointers, so such a tensor would
otherwise become an out-of-bounds device access).  CPU only: the cache is built on the host
and the library loader is replaced by one that fails the test if it is reached."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_decode_amd as tq
from quantized_kv_cache_decode_amd import binding
from synth import sign_vector

B, HKV, HQ, CAP = 2, 2, 8, 64


@pytest.fixture
def cache(monkeypatch):
    def unreachable(*a, **k):
        raise AssertionError("the library was called with arguments the binding should have rejected")
    monkeypatch.setattr(binding, "load_library", unreachable)
    return tq.Cache(B, HKV, CAP, "turbo3", "turbo4", sign_vector(0, "k"), sign_vector(0, "v"), device="cpu")


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


WS = torch.zeros(1 << 16, dtype=torch.uint8)


@pytest.mark.parametrize("k_new,v_new,match", [
    (f16(B, HKV, 3, 128), f16(B, HKV, 2, 128), "v_new has shape"),
    (f16(B + 1, HKV, 3, 128), f16(B + 1, HKV, 3, 128), "k_new has shape"),
    (f16(B, HKV, 3, 64), f16(B, HKV, 3, 64), "k_new has shape"),
    (f32(B, HKV, 3, 128), f32(B, HKV, 3, 128), "dtype"),
    (f16(B, HKV, 128, 3).transpose(2, 3), f16(B, HKV, 3, 128), "contiguous"),
    (f16(B, HKV, 128), f16(B, HKV, 128), r"\[B, Hkv, t_new, 128\]"),
    (f16(B, HKV, 3, 128), f16(B, HKV, 3, 128), "not on a GPU"),
])
def test_encode_append_rejects(cache, k_new, v_new, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_encode_append(cache, k_new, v_new)


def test_host_lengths_must_cover_every_sequence(cache):
    with pytest.raises(ValueError, match="one entry per sequence"):
        tq.tq_encode_append(cache, f16(B, HKV, 3, 128), f16(B, HKV, 3, 128), seq_lens_host=[0])
    with pytest.raises(ValueError, match="counts has shape"):
        tq.tq_encode_append(cache, f16(B, HKV, 3, 128), f16(B, HKV, 3, 128), counts=[1, 2, 3])
    with pytest.raises(ValueError, match="one entry per sequence"):
        tq.tq_decode_workspace_size(cache, HQ, [5, 5, 5])


@pytest.mark.parametrize("q,out,match", [
    (f16(B, HQ, 128), f16(B, HQ, 128), "q_rot has dtype"),
    (f16(B, HQ + 1, 128), f32(B, HQ + 1, 128), "multiple of"),
    (f16(B + 1, HQ, 128), f32(B + 1, HQ, 128), "q has shape"),
    (f16(B, HQ, 128), f32(B, HQ, 64), "q_rot has shape"),
    (f16(B, HQ, 128), f32(B, HQ, 128), "not on a GPU"),
])
def test_rotate_q_rejects(cache, q, out, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_rotate_q(cache, q, out)


@pytest.mark.parametrize("q_rot,out_rot,match", [
    (f16(B, HQ, 128), f32(B, HQ, 128), "dtype"),
    (f32(B, HQ, 128), f32(B, HQ - 1, 128), "out_rot has shape"),
    (f32(B, HQ, 2, 128), f32(B, HQ, 2, 128), r"\[B, Hq, 128\]"),
    (f32(B, HQ, 128), f32(B, HQ, 128), "not on a GPU"),
])
def test_decode_attention_rejects(cache, q_rot, out_rot, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_decode_attention(cache, q_rot, 0.1, out_rot, WS)


def test_workspace_must_be_a_contiguous_tensor(cache):
    with pytest.raises(ValueError, match="workspace"):
        tq.tq_decode_attention_fused(cache, f16(B, HQ, 128), 0.1, f16(B, HQ, 128), np.zeros(10, np.uint8))
    with pytest.raises(ValueError, match="workspace"):
        tq.tq_decode_attention_fused(cache, f16(B, HQ, 128), 0.1, f16(B, HQ, 128), WS[::2])


@pytest.mark.parametrize("q,out,match", [
    (f16(B, HQ, 128), f32(B, HQ, 128), "out has dtype"),
    (f16(B, HQ, 128), f16(B, HQ, 1, 128), "out has shape"),
    (torch.zeros((B, HQ, 128), dtype=torch.bfloat16), f16(B, HQ, 128), "q has dtype"),
    (f16(B, HQ, 128), f16(B, HQ, 128), "not on a GPU"),
])
def test_decode_attention_fused_rejects(cache, q, out, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_decode_attention_fused(cache, q, 0.1, out, WS)


@pytest.mark.parametrize("q,out,match", [
    (f16(B, HQ, 128), f16(B, HQ, 128), r"\[B, Hq, Tq, 128\]"),
    (f16(B, HQ, 3, 128), f16(B, HQ, 2, 128), "out has shape"),
    (f16(B, HQ, 3, 128), f16(B, HQ, 3, 128), "not on a GPU"),
])
def test_decode_chunk_rejects(cache, q, out, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_decode_chunk_fused(cache, q, 0.1, out, WS)


@pytest.mark.parametrize("k_new,q,out,match", [
    (f16(B, HKV, 2, 128), f16(B, HQ, 128), f16(B, HQ, 128), "k_new has shape"),
    (f16(B, HKV, 1, 128), f16(B, HQ, 2, 128), f16(B, HQ, 2, 128), r"\[B, Hq, 128\]"),
    (f16(B, HKV, 1, 128), f16(B, HQ, 128), f16(B, 2 * HQ, 128), "out has shape"),
    (f16(B, HKV, 1, 128), f16(B, HQ, 128), f16(B, HQ, 128), "not on a GPU"),
])
def test_decode_step_rejects(cache, k_new, q, out, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_decode_step(cache, k_new, f16(B, HKV, 1, 128), q, 0.1, out, WS)


@pytest.mark.parametrize("out_rot,out,match", [
    (f16(B, HQ, 128), f16(B, HQ, 128), "out_rot has dtype"),
    (f32(B, HQ, 128), f32(B, HQ, 128), "out has dtype"),
    (f32(B, HQ, 128), f16(B, HQ + 2, 128), "out has shape"),
    (f32(B, HQ, 128), f16(B, HQ, 128), "not on a GPU"),
])
def test_inverse_rotate_rejects(cache, out_rot, out, match):
    with pytest.raises(ValueError, match=match):
        tq.tq_inverse_rotate_out(cache, out_rot, out)


def test_decode_step_noalloc_rejects(cache):
    with pytest.raises(ValueError, match="v_new has shape"):
        tq.tq_decode_step_noalloc(cache, f16(B, HKV, 1, 128), f16(B, HKV, 2, 128), f16(B, HQ, 128), 0.1,
                                  f16(B, HQ, 128))
    with pytest.raises(ValueError, match="not on a GPU"):
        tq.tq_decode_step_noalloc(cache, f16(B, HKV, 1, 128), f16(B, HKV, 1, 128), f16(B, HQ, 128), 0.1,
                                  f16(B, HQ, 128))
