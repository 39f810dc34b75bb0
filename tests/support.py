"""Helpers shared by the GPU parity tests: seeded inputs, GPU encode/decode through
the C ABI, download of the library's bytes, and the oracle on the same inputs.

The oracle is imported only inside the helpers that run it (oracle_*, compare_codes),
so importing this module -- as bench.py does for its GPU set-up -- loads no oracle code."""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np

from synth import context_lengths, kv_slice, new_token_kv, queries, sign_vector

SCALE = 1.0 / np.sqrt(128.0)
REL_L2_TOL = 1e-3
MAX_ABS_TOL = 5e-3


def scaled(w, **kw):
    return replace(w, **kw)


def gen_kv(w, seed, lengths, which):
    """[Hkv, L_b, 128] fp16 per sequence b (threaded over (b, h) slices)."""
    jobs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    with ThreadPoolExecutor(16) as ex:
        sl = list(ex.map(lambda bh: kv_slice(w, seed, which, bh[0], bh[1], int(lengths[bh[0]])), jobs))
    H = w.num_kv_heads
    return [np.stack(sl[b * H:(b + 1) * H]) for b in range(w.batch)]


def padded_tensor(arrs, t_max):
    import torch
    B, H = len(arrs), arrs[0].shape[0]
    out = torch.zeros((B, H, max(t_max, 1), 128), dtype=torch.float16, device="cuda")
    for b, a in enumerate(arrs):
        if a.shape[1]:
            out[b, :, :a.shape[1]] = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return out


def make_cache(w, capacity, seed=0):
    import quantized_kv_cache_decode_amd as tq
    return tq.Cache(w.batch, w.num_kv_heads, capacity, w.k_format, w.v_format,
                    sign_vector(seed, "k"), sign_vector(seed, "v"))


def encode_on_gpu(w, k_list, v_list, lengths, capacity, seed=0):
    """Prefill a fresh cache through tq_encode_append with per-sequence counts."""
    import quantized_kv_cache_decode_amd as tq
    cache = make_cache(w, capacity, seed)
    t_max = int(max(lengths)) if len(lengths) else 0
    if t_max:
        tq.tq_encode_append(cache, padded_tensor(k_list, t_max), padded_tensor(v_list, t_max),
                            counts=np.asarray(lengths, dtype=np.int32))
    return cache


def download_sequence(cache, b):
    """The library's bytes of sequence b as numpy (K records or fp16 K, norms, V tiles)."""
    out = {}
    if cache.k_format == "f16":
        out["k_f16"] = cache.k_data[b].cpu().numpy()
    else:
        out["k_rec"] = cache.k_data[b].cpu().numpy()
        out["k_norms"] = cache.k_norms[b].cpu().numpy().view(np.float16)
    out["v_tiles"] = cache.v_data[b].cpu().numpy()
    if cache.v_norms is not None:
        out["v_norms"] = cache.v_norms[b].cpu().numpy().view(np.float16)
    return out


def oracle_on_bytes(cache, b, L, q_b, codebooks, seed=0):
    """Oracle attention [Hq, 128] over the GPU-written bytes of sequence b (unpacked by the oracle)."""
    from oracle import reference
    k_hat, v_hat = oracle_dequant_bytes(cache, b, L, codebooks, seed)
    return reference.decode_sequence(q_b, k_hat, v_hat, L)


def oracle_dequant_bytes(cache, b, L, codebooks, seed=0):
    """K and V [Hkv, L, 128] (float64, original basis) of sequence b from the GPU-written bytes."""
    return oracle_dequant_download(download_sequence(cache, b), cache.k_format, cache.v_format, L, codebooks, seed)


def oracle_dequant_download(d, k_format, v_format, L, codebooks, seed=0):
    """K and V [Hkv, L, 128] (float64, original basis) from bytes already downloaded by
    download_sequence (no GPU access: safe to run in worker threads)."""
    from oracle import reference
    kc, vc = reference.codes_from_library_layout(d.get("k_rec"), d["v_tiles"], k_format, v_format)
    enc = {"v_f16": vc} if v_format == "f16" else {"v_codes": vc, "v_norms": d["v_norms"]}
    if k_format == "f16":
        enc["k_f16"] = d["k_f16"]
    else:
        enc["k_codes"], enc["k_norms"] = kc, d["k_norms"]
    return reference.dequant_sequence(enc, k_format, v_format, sign_vector(seed, "k"),
                                      sign_vector(seed, "v"), codebooks, L)


def oracle_errors_all_sequences(cache, L, q, got, codebooks, seed=0, workers=8):
    """(rel-L2, max-abs) of every sequence's GPU output against the oracle on the GPU-written
    bytes; the bytes are downloaded first, the oracle runs in worker threads."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import reference
    downloads = [download_sequence(cache, b) for b in range(cache.batch)]

    def one(b):
        k_hat, v_hat = oracle_dequant_download(downloads[b], cache.k_format, cache.v_format, int(L[b]), codebooks,
                                               seed)
        return errors(got[b], reference.decode_sequence(q[b], k_hat, v_hat, int(L[b])))

    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, range(cache.batch)))


def oracle_end_to_end(w, k16, v16, L, q_b, codebooks, seed=0):
    """Oracle encode + full-dequant attention [Hq, 128] of one sequence from its fp16 inputs."""
    from oracle import reference
    sk, sv = sign_vector(seed, "k"), sign_vector(seed, "v")
    enc = reference.encode_sequence(k16[:, :L], v16[:, :L], w.k_format, w.v_format, sk, sv, codebooks)
    k_hat, v_hat = reference.dequant_sequence(enc, w.k_format, w.v_format, sk, sv, codebooks, L)
    return reference.decode_sequence(q_b, k_hat, v_hat, L)


def gpu_decode(cache, q_np, variant=0):
    """Decode of q [B, Hq, 128] through the C ABI; returns fp16 [B, Hq, 128] as numpy.

    variant 0 (MFMA) / 1 (VALU reference): tq_rotate_q -> tq_decode_attention(variant) ->
    tq_inverse_rotate_out;
    "fused": tq_decode_attention_fused (rotations inside the decode and merge kernels)."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to("cuda")
    B, Hq, _ = q.shape
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.zeros(tq.tq_decode_workspace_size(cache, Hq), dtype=torch.uint8, device="cuda")
    if variant == "fused":
        tq.tq_decode_attention_fused(cache, q, SCALE, out, ws)
    else:
        q_rot = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        out_rot = torch.empty_like(q_rot)
        tq.tq_rotate_q(cache, q, q_rot)
        tq.tq_decode_attention(cache, q_rot, SCALE, out_rot, ws, variant=variant)
        tq.tq_inverse_rotate_out(cache, out_rot, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def errors(got_fp16, want):
    g = np.asarray(got_fp16, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    rel = np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300)
    return float(rel), float(np.abs(g - w).max())


def assert_close(got_fp16, want, what=""):
    rel, mx = errors(got_fp16, want)
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, f"{what}: rel-L2 {rel:.3e} (<= {REL_L2_TOL}), max-abs {mx:.3e} (<= {MAX_ABS_TOL})"
    return rel, mx


def compare_codes(cache, b, k16, v16, L, w, codebooks, seed=0):
    """Codes and norms of sequence b: GPU bytes vs oracle encode of the same fp16 rows.

    Returns (mismatching codes, codes within 1e-5 of a decision threshold, total codes);
    asserts norms bit-exact and every mismatch inside the boundary margin."""
    from oracle import codec, reference
    sk, sv = sign_vector(seed, "k"), sign_vector(seed, "v")
    d = download_sequence(cache, b)
    kc, vc = reference.codes_from_library_layout(d.get("k_rec"), d["v_tiles"], w.k_format, w.v_format)
    mism = margin = total = 0
    parts = []
    if w.v_format != "f16":
        parts.append(("v", v16, vc, d["v_norms"], sv, w.v_format))
    else:   # the uncompressed comparison cache holds the rows bit for bit; slots past L stay zero
        np.testing.assert_array_equal(vc[:, :L].view(np.uint16), v16[:, :L].view(np.uint16))
        assert np.all(vc[:, L:].view(np.uint16) == 0)
    if w.k_format != "f16":
        parts.append(("k", k16, kc, d["k_norms"], sk, w.k_format))
    else:
        np.testing.assert_array_equal(d["k_f16"][:, :L].view(np.uint16), k16[:, :L].view(np.uint16))
    for name, x16, codes_gpu, norms_gpu, signs, fmt in parts:
        for t0 in range(0, L, 4096):
            t1 = min(L, t0 + 4096)
            oc, on = codec.encode(x16[:, t0:t1], signs, codebooks[fmt])
            np.testing.assert_array_equal(norms_gpu[:, t0:t1].view(np.uint16), on.view(np.uint16),
                                          err_msg=f"{name} norms of sequence {b}")
            bad = codes_gpu[:, t0:t1] != oc
            near = codec.boundary_margin(x16[:, t0:t1], signs, codebooks[fmt])
            assert not np.any(bad & ~near), f"{name} codes differ outside the boundary margin (sequence {b})"
            mism += int(bad.sum())
            margin += int(near.sum())
            total += bad.size
    return mism, margin, total


def new_token_rows(w, seed, step=0):
    """The step's new K and V rows as fp16 [B, Hkv, 1, 128] numpy arrays."""
    kn = np.stack([np.stack([new_token_kv(w, seed, "k", b, h, step) for h in range(w.num_kv_heads)])
                   for b in range(w.batch)])
    vn = np.stack([np.stack([new_token_kv(w, seed, "v", b, h, step) for h in range(w.num_kv_heads)])
                   for b in range(w.batch)])
    return kn, vn


def gpu_decode_step(cache, kn, vn, q_np):
    """tq_decode_step: append kn, vn [B, Hkv, 1, 128] and decode q; returns fp16 [B, Hq, 128]."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to("cuda")
    B, Hq, _ = q.shape
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    ws = torch.zeros(tq.tq_decode_workspace_size(cache, Hq), dtype=torch.uint8, device="cuda")
    tq.tq_decode_step(cache, torch.from_numpy(np.ascontiguousarray(kn)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(vn)).cuda(), q, SCALE, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def prefill_then_decode_step(w, seed=0, lengths=None, capacity=None):
    """A workload through tq_decode_step: prefill L_b - 1 rows, then one step that appends the
    L_b-th row and decodes (sequences with L_b = 0 get their first row).

    Returns (cache, k_list, v_list (full rows incl. the appended one), lengths after the step,
    q, out fp16)."""
    L = context_lengths(w, seed) if lengths is None else np.asarray(lengths)
    pre = np.maximum(L - 1, 0)
    L = pre + 1
    k_list = gen_kv(w, seed, pre, "k")
    v_list = gen_kv(w, seed, pre, "v")
    cap = capacity or int(((L.max() + 31) // 32) * 32)
    cache = encode_on_gpu(w, k_list, v_list, pre, cap, seed)
    kn, vn = new_token_rows(w, seed)
    q = queries(w, seed)
    out = gpu_decode_step(cache, kn, vn, q)
    k_list = [np.concatenate([k, kk], axis=1) for k, kk in zip(k_list, kn)]
    v_list = [np.concatenate([v, vv], axis=1) for v, vv in zip(v_list, vn)]
    return cache, k_list, v_list, L, q, out


def prefill_and_step(w, seed=0, lengths=None, capacity=None):
    """Inputs and GPU cache of a workload: prefill L_b - appends rows, then one append step.

    Returns (cache, k_list, v_list (full rows incl. the appended one), lengths, q)."""
    import torch
    L = context_lengths(w, seed) if lengths is None else np.asarray(lengths)
    n_app = w.appends_per_step
    pre = np.maximum(L - n_app, 0)
    k_list = gen_kv(w, seed, pre, "k")
    v_list = gen_kv(w, seed, pre, "v")
    cap = capacity or int(((L.max() + 31) // 32) * 32)
    cache = encode_on_gpu(w, k_list, v_list, pre, cap, seed)
    if n_app:
        kn = [np.stack([new_token_kv(w, seed, "k", b, h, 0, n_app) for h in range(w.num_kv_heads)])
              for b in range(w.batch)]
        vn = [np.stack([new_token_kv(w, seed, "v", b, h, 0, n_app) for h in range(w.num_kv_heads)])
              for b in range(w.batch)]
        import quantized_kv_cache_decode_amd as tq
        counts = (L - pre).astype(np.int32)
        tq.tq_encode_append(cache, padded_tensor(kn, n_app), padded_tensor(vn, n_app), counts=counts)
        k_list = [np.concatenate([k, kk[:, :c]], axis=1) for k, kk, c in zip(k_list, kn, counts)]
        v_list = [np.concatenate([v, vv[:, :c]], axis=1) for v, vv, c in zip(v_list, vn, counts)]
    torch.cuda.synchronize()
    return cache, k_list, v_list, L, queries(w, seed)
