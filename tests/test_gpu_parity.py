"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: packed codes and fp16 norms bit-exact (codes within 1e-5 of a decision
threshold excluded and counted, at most 1e-4 of all codes); decode outputs
(fp16) within relative-L2 1e-3 and max-abs 5e-3 of the oracle's unrounded
float64 output.  Decode parity is checked twice: (i) on the GPU-written bytes
(unpacked by the oracle), (ii) end to end from the same fp16 inputs.
"""
import hashlib
import sys

import numpy as np
import pytest

from oracle import codec, reference
from oracle.hadamard import inverse_rotate, rotate
from synth import get_workload, queries, sign_vector
from tests import support as S

pytestmark = pytest.mark.gpu

VARIANTS = [0, 1, "fused"]


def _say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_kv_cache_decode_amd as tq
    tq.load_library()     # raises if the library is missing: no silent fallback


# ----------------------------------------------------------------------------- rotations

@pytest.mark.parametrize("q_fp32", [False, True])
@pytest.mark.parametrize("k_format", ["turbo3", "f16"])
def test_rotate_q(q_fp32, k_format):
    import torch

    import quantized_kv_cache_decode_amd as tq
    w = S.scaled(get_workload(1), k_format=k_format, v_format="turbo4" if k_format == "f16" else "turbo3")
    cache = S.make_cache(w, 32)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 28, 128)).astype(np.float32 if q_fp32 else np.float16)
    qt = torch.from_numpy(q).cuda()
    q_rot = torch.empty((1, 28, 128), dtype=torch.float32, device="cuda")
    tq.tq_rotate_q(cache, qt, q_rot)
    got = q_rot.cpu().numpy().astype(np.float64)
    want = rotate(q.astype(np.float64), sign_vector(0, "k")) if k_format != "f16" else q.astype(np.float64)
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


def test_inverse_rotate_out():
    import torch

    import quantized_kv_cache_decode_amd as tq
    cache = S.make_cache(S.scaled(get_workload(0), batch=3), 32)
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, 4, 128)).astype(np.float32)
    out = torch.empty((3, 4, 128), dtype=torch.float16, device="cuda")
    tq.tq_inverse_rotate_out(cache, torch.from_numpy(o).cuda(), out)
    got = out.cpu().numpy().astype(np.float64)
    want = inverse_rotate(o.astype(np.float64), sign_vector(0, "v"))
    # fp32 butterflies then one rounding to fp16: within one fp16 ulp of the exact value
    ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want.astype(np.float16).astype(np.float64)) > 0.99


# ----------------------------------------------------------------------------- workloads

def _small_workloads():
    return {
        "c0": (get_workload(0), None),
        "c1": (get_workload(1), None),
        "c2": (get_workload(2), None),
        # fp16 K + turbo3 V (turbo3-asym, the low-memory mix of mlxcel commit #376)
        "c2t3": (S.scaled(get_workload(2), v_format="turbo3"), None),
        "c3s": (S.scaled(get_workload(3), batch=3, context=2048), None),
        "c4s": (S.scaled(get_workload(4), batch=6, context=None, ragged_range=(1, 3000)),
                np.array([1, 31, 33, 2049, 700, 2999])),
    }


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c2t3", "c3s", "c4s"])
def test_encode_bit_exact(name, codebooks):
    w, lens = _small_workloads()[name]
    cache, k_list, v_list, L, _ = S.prefill_and_step(w, lengths=lens)
    np.testing.assert_array_equal(cache.seq_lens.cpu().numpy(), L)
    mism = margin = total = 0
    for b in range(w.batch):
        m, g, t = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        mism, margin, total = mism + m, margin + g, total + t
    _say(f"[{name}] code mismatches {mism} / {total}; within 1e-5 of a threshold {margin}")
    assert margin <= 1e-4 * total
    assert mism <= margin


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c2t3", "c3s", "c4s"])
def test_decode_parity(name, variant, codebooks):
    w, lens = _small_workloads()[name]
    cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
    got = S.gpu_decode(cache, q, variant=variant)
    worst = (0.0, 0.0)
    for b in range(w.batch):
        on_bytes = S.oracle_on_bytes(cache, b, int(L[b]), q[b], codebooks)
        e2e = S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks)
        r1 = S.assert_close(got[b], on_bytes, f"{name} b={b} on GPU bytes")
        r2 = S.assert_close(got[b], e2e, f"{name} b={b} end to end")
        worst = tuple(max(x) for x in zip(worst, r1, r2))
    _say(f"[{name} v{variant}] worst rel-L2 {worst[0]:.2e} max-abs {worst[1]:.2e}")


@pytest.mark.parametrize("k_format,v_format", [("turbo3", "turbo3"), ("turbo4", "turbo4"), ("turbo4", "turbo3"),
                                               ("f16", "turbo3"), ("f16", "f16")])
def test_one_token_appends_bit_exact(k_format, v_format, codebooks):
    """tq_encode_append of one token per sequence (the one-row kernel, each row encoded over
    a whole wave) into every kind of V-tile slot -- a fresh tile, mid-tile, its last slot --
    after prefills of 0 to 100 tokens: codes and norms against the oracle's encode of the same
    rows, the earlier tokens' codes kept."""
    import quantized_kv_cache_decode_amd as tq
    from synth import kv_slice, new_token_kv
    pre = [0, 1, 5, 31, 32, 33, 63, 64, 100]
    w = S.scaled(get_workload(0), batch=len(pre), num_q_heads=4, num_kv_heads=2, k_format=k_format,
                 v_format=v_format)
    k = [np.stack([kv_slice(w, 0, "k", b, h, n) for h in range(2)]) for b, n in enumerate(pre)]
    v = [np.stack([kv_slice(w, 0, "v", b, h, n) for h in range(2)]) for b, n in enumerate(pre)]
    cache = S.encode_on_gpu(w, k, v, pre, 128)
    kn = [np.stack([new_token_kv(w, 0, "k", b, h, 0) for h in range(2)]) for b in range(len(pre))]
    vn = [np.stack([new_token_kv(w, 0, "v", b, h, 0) for h in range(2)]) for b in range(len(pre))]
    tq.tq_encode_append(cache, S.padded_tensor(kn, 1), S.padded_tensor(vn, 1))
    np.testing.assert_array_equal(cache.seq_lens.cpu().numpy(), np.array(pre) + 1)
    for b, n in enumerate(pre):
        k_all = np.concatenate([k[b], kn[b]], axis=1)
        v_all = np.concatenate([v[b], vn[b]], axis=1)
        S.compare_codes(cache, b, k_all, v_all, n + 1, w, codebooks)


@pytest.mark.parametrize("variant", VARIANTS)
def test_sixteen_decode_steps_gqa_4_over_2(variant, codebooks):
    """The parity shape of mlxcel PR #369 ("Result"): GQA 4 query heads over 2 KV heads,
    16 successive decode steps, each compared with the full-dequant reference, and the
    visible offset advancing by exactly one token per append."""
    import quantized_kv_cache_decode_amd as tq
    from synth import kv_slice, new_token_kv
    w = get_workload(0)
    pre = 240
    k = [np.stack([kv_slice(w, 0, "k", 0, h, pre) for h in range(2)])]
    v = [np.stack([kv_slice(w, 0, "v", 0, h, pre) for h in range(2)])]
    cache = S.encode_on_gpu(w, k, v, [pre], 256)
    for step in range(16):
        kn = np.stack([new_token_kv(w, 0, "k", 0, h, step) for h in range(2)])
        vn = np.stack([new_token_kv(w, 0, "v", 0, h, step) for h in range(2)])
        tq.tq_encode_append(cache, S.padded_tensor([kn], 1), S.padded_tensor([vn], 1))
        k[0] = np.concatenate([k[0], kn], axis=1)
        v[0] = np.concatenate([v[0], vn], axis=1)
        L = pre + step + 1
        assert int(cache.seq_lens.cpu()[0]) == L and int(cache.lengths[0]) == L
        q = queries(w, 0, step)
        got = S.gpu_decode(cache, q, variant=variant)
        S.assert_close(got[0], S.oracle_end_to_end(w, k[0], v[0], L, q[0], codebooks), f"step {step}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_workspace_reused_across_calls(variant, codebooks):
    """One workspace (filled with garbage first) serves successive decode calls with growing,
    multi-split lengths."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    from synth import kv_slice, new_token_kv
    w = S.scaled(get_workload(1), context=None)
    L0 = 3000
    k = [np.stack([kv_slice(w, 2, "k", 0, h, L0) for h in range(4)])]
    v = [np.stack([kv_slice(w, 2, "v", 0, h, L0) for h in range(4)])]
    cache = S.encode_on_gpu(w, k, v, [L0], 4864, seed=2)
    ws = torch.full((tq.tq_decode_workspace_size(cache, 28, [4800]),), 0x7f, dtype=torch.uint8, device="cuda")
    q_rot = torch.empty((1, 28, 128), dtype=torch.float32, device="cuda")
    out_rot = torch.empty_like(q_rot)
    out = torch.empty((1, 28, 128), dtype=torch.float16, device="cuda")
    for step in range(3):
        n = 300 * (step + 1)
        kn = np.stack([new_token_kv(w, 2, "k", 0, h, step, n) for h in range(4)])
        vn = np.stack([new_token_kv(w, 2, "v", 0, h, step, n) for h in range(4)])
        tq.tq_encode_append(cache, S.padded_tensor([kn], n), S.padded_tensor([vn], n))
        k[0] = np.concatenate([k[0], kn], axis=1)
        v[0] = np.concatenate([v[0], vn], axis=1)
        L = int(cache.lengths[0])
        q = queries(w, 2, step)
        if variant == "fused":
            tq.tq_decode_attention_fused(cache, torch.from_numpy(q).cuda(), S.SCALE, out, ws)
        else:
            tq.tq_rotate_q(cache, torch.from_numpy(q).cuda(), q_rot)
            tq.tq_decode_attention(cache, q_rot, S.SCALE, out_rot, ws, variant=variant)
            tq.tq_inverse_rotate_out(cache, out_rot, out)
        torch.cuda.synchronize()
        S.assert_close(out.cpu().numpy()[0], S.oracle_end_to_end(w, k[0], v[0], L, q[0], codebooks, seed=2),
                       f"step {step} L={L}")


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c2t3", "c3s", "c4s"])
def test_fused_call_matches_separate_calls_bitwise(name):
    """tq_decode_attention_fused == tq_rotate_q + tq_decode_attention + tq_inverse_rotate_out,
    bit for bit (the same rotation routine and merge arithmetic run inside the fused kernels);
    the workloads cover fp32 q (c0) and fp16 q, and the unrotated fp16-K mode (c2)."""
    w, lens = _small_workloads()[name]
    cache, _, _, _, q = S.prefill_and_step(w, lengths=lens)
    sep = S.gpu_decode(cache, q, variant=0)
    fused = S.gpu_decode(cache, q, variant="fused")
    np.testing.assert_array_equal(fused.view(np.uint16), sep.view(np.uint16))


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c2t3", "c3s", "c4s"])
def test_decode_step_parity(name, codebooks):
    """tq_decode_step (append + attend in one call): the appended token's codes and norms are
    bit-exact, the lengths advance by one, and the output matches the oracle end to end and
    the two-call route (tq_encode_append, then the fused decode) up to rounding."""
    w, lens = _small_workloads()[name]
    cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
    np.testing.assert_array_equal(cache.seq_lens.cpu().numpy(), L)
    np.testing.assert_array_equal(cache.lengths, L)
    mism = margin = total = 0
    for b in range(w.batch):
        m, g, t = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        mism, margin, total = mism + m, margin + g, total + t
        S.assert_close(got[b], S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks),
                       f"{name} b={b}")
    assert mism <= margin <= 1e-4 * total
    two_call = S.gpu_decode(cache, q, variant="fused")
    rel, mx = S.errors(got, two_call.astype(np.float64))
    _say(f"[{name} step] vs two-call route: rel-L2 {rel:.2e} max-abs {mx:.2e}")
    assert rel <= 2e-4 and mx <= 2e-3


def test_decode_step_sixteen_steps_gqa_4_over_2(codebooks):
    """Sixteen successive tq_decode_step calls (GQA 4 over 2), across a 32-token tile boundary
    and a split boundary, each checked against the full-dequant oracle."""
    w = get_workload(0)
    pre = 250
    from synth import kv_slice, new_token_kv
    k = [np.stack([kv_slice(w, 0, "k", 0, h, pre) for h in range(2)])]
    v = [np.stack([kv_slice(w, 0, "v", 0, h, pre) for h in range(2)])]
    cache = S.encode_on_gpu(w, k, v, [pre], 288)
    for step in range(16):
        kn = np.stack([new_token_kv(w, 0, "k", 0, h, step) for h in range(2)])[None]
        vn = np.stack([new_token_kv(w, 0, "v", 0, h, step) for h in range(2)])[None]
        q = queries(w, 0, step)
        got = S.gpu_decode_step(cache, kn, vn, q)
        k[0] = np.concatenate([k[0], kn[0]], axis=1)
        v[0] = np.concatenate([v[0], vn[0]], axis=1)
        L = pre + step + 1
        assert int(cache.seq_lens.cpu()[0]) == L and int(cache.lengths[0]) == L
        S.assert_close(got[0], S.oracle_end_to_end(w, k[0], v[0], L, q[0], codebooks), f"step {step}")
    m, _, _ = S.compare_codes(cache, 0, k[0], v[0], pre + 16, w, codebooks)
    assert m == 0


@pytest.mark.parametrize("group,k_format,v_format", [(1, "turbo4", "turbo3"), (16, "turbo3", "turbo4"),
                                                     (7, "f16", "turbo4"), (1, "f16", "turbo3"),
                                                     (4, "f16", "turbo3"), (7, "f16", "turbo3"),
                                                     (16, "f16", "turbo3")])
def test_decode_step_groups_formats_and_empty(group, k_format, v_format, codebooks):
    """The step at group sizes 1, 7 and 16, mixed formats and fp16 K, with a sequence whose
    first token the step appends (length 0 before it) and one ending on a tile boundary."""
    w = S.scaled(get_workload(0), batch=3, num_q_heads=2 * group, num_kv_heads=2, k_format=k_format,
                 v_format=v_format)
    cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=np.array([1, 300, 64]))
    for b in range(3):
        S.assert_close(got[b], S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks),
                       f"G={group} b={b} L={int(L[b])}")
        m, _, _ = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        assert m == 0


def test_decode_does_not_mutate_cache():
    w = get_workload(0)
    cache, _, _, _, q = S.prefill_and_step(w)

    def digest():
        h = hashlib.sha256()
        for t in (cache.k_data, cache.k_norms, cache.v_data, cache.v_norms, cache.seq_lens):
            h.update(t.cpu().numpy().tobytes())
        return h.hexdigest()

    before = digest()
    for variant in VARIANTS:
        S.gpu_decode(cache, q, variant=variant)
    assert digest() == before


@pytest.mark.parametrize("variant", VARIANTS)
def test_empty_and_single_token_sequences(variant, codebooks):
    w = S.scaled(get_workload(0), batch=3)
    cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=np.array([1, 0, 65]))
    got = S.gpu_decode(cache, q, variant=variant)
    assert np.all(got[1] == 0)
    for b in (0, 2):
        S.assert_close(got[b], S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks))
    # one visible token: the output is that token's reconstructed value for every query head
    d = S.download_sequence(cache, 0)
    _, vc = reference.codes_from_library_layout(d.get("k_rec"), d["v_tiles"], w.k_format, w.v_format)
    v0 = codec.dequant(vc[:, :1], d["v_norms"][:, :1], codebooks["turbo3"], sign_vector(0, "v"))[:, 0]
    np.testing.assert_allclose(got[0].astype(np.float64), np.repeat(v0, 2, axis=0), atol=2e-3, rtol=0)


@pytest.mark.parametrize("k_format", ["turbo4", "f16"])
@pytest.mark.parametrize("group", [1, 4, 16])
@pytest.mark.parametrize("variant", VARIANTS)
def test_group_size_extremes(group, variant, k_format, codebooks):
    w = S.scaled(get_workload(0), num_q_heads=2 * group, num_kv_heads=2, k_format=k_format, v_format="turbo3")
    cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=np.array([300]))
    got = S.gpu_decode(cache, q, variant=variant)
    S.assert_close(got[0], S.oracle_end_to_end(w, k_list[0], v_list[0], 300, q[0], codebooks), f"G={group}")


def test_appends_merge_into_partial_tiles(codebooks):
    """Appends of 5, 1, 37 and 100 rows land mid-tile and across tiles; earlier tokens of
    a shared V tile keep their codes."""
    import quantized_kv_cache_decode_amd as tq
    from synth import kv_slice
    for fmt in ("turbo3", "turbo4"):
        w = S.scaled(get_workload(0), batch=2, k_format=fmt, v_format=fmt)
        total = 3 + 5 + 1 + 37 + 100
        full_k = [np.stack([kv_slice(w, 1, "k", b, h, total) for h in range(2)]) for b in range(2)]
        full_v = [np.stack([kv_slice(w, 1, "v", b, h, total) for h in range(2)]) for b in range(2)]
        cache = S.make_cache(w, 160, seed=1)
        pos = 0
        for n in (3, 5, 1, 37, 100):
            tq.tq_encode_append(cache, S.padded_tensor([x[:, pos:pos + n] for x in full_k], n),
                                S.padded_tensor([x[:, pos:pos + n] for x in full_v], n))
            pos += n
        for b in range(2):
            m, _, _ = S.compare_codes(cache, b, full_k[b], full_v[b], total, w, codebooks, seed=1)
            assert m == 0


# ----------------------------------------------------------------------------- full size

@pytest.mark.timeout(900)
@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_full_size_sampled(index, codebooks):
    """Full-size workloads in the launch configuration the benchmark times (prefill, then one
    tq_decode_step): the outputs of every sequence against the oracle on the GPU-written bytes;
    codes and norms of the sampled sequences (the shortest and longest, or the first and last)
    in full against the oracle's encode of the same rows, which makes the sampled outputs end
    to end as well."""
    w = get_workload(index)
    _say(f"[full {w.name}] generating + encoding")
    cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w)
    sample = [int(np.argmin(L)), int(np.argmax(L))] if index == 4 else sorted({0, w.batch - 1})
    for b in sample:
        m, g, t = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        _say(f"[full {w.name}] b={b} L={int(L[b])} code mismatches {m}/{t}, margin {g}")
        assert m <= g <= 1e-4 * t
    errs = S.oracle_errors_all_sequences(cache, L, q, got, codebooks)
    worst_rel, worst_abs = max(e[0] for e in errs), max(e[1] for e in errs)
    _say(f"[full {w.name}] all {w.batch} sequences: worst rel-L2 {worst_rel:.2e} max-abs {worst_abs:.2e}")
    for b, (rel, mx) in enumerate(errs):
        assert rel <= S.REL_L2_TOL and mx <= S.MAX_ABS_TOL, f"b={b}: rel-L2 {rel:.3e} max-abs {mx:.3e}"


@pytest.mark.parametrize("variant", [0, "fused"])
def test_one_row_of_many_splits(variant, codebooks):
    """One (sequence, KV head) row of 262144 turbo4 tokens (35 MB: past the small-call plan,
    short of the bandwidth-bound one) is cut into 2048 splits of 128 tokens: the merge gives the
    row four waves (few rows) and each lane group folds 2048 / 16 = 128 partials over eight load
    rounds of 17."""
    w = S.scaled(get_workload(3), batch=1, num_kv_heads=1, num_q_heads=4)
    lens = np.array([262144])
    _say("[one row of many splits] generating + encoding")
    cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
    got = S.gpu_decode(cache, q, variant=variant)
    rel, mx = S.assert_close(got[0], S.oracle_on_bytes(cache, 0, int(L[0]), q[0], codebooks), "on GPU bytes")
    _say(f"[one row of many splits v{variant}] rel-L2 {rel:.2e} max-abs {mx:.2e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt,tokens", [("turbo4", 262144), ("turbo3", 393216)])
def test_middle_sized_decode_step(fmt, tokens, codebooks):
    """A decode step past the small-call plan (32 MB of packed K and V) and short of the
    bandwidth-bound one (4M token-heads): one row of 35 / 39 MB, one wave per split, and the
    token appended by two extra one-wave work groups whose K side stages q itself.  Codes and
    norms bit-exact, the output against the oracle on the GPU-written bytes."""
    w = S.scaled(get_workload(3), batch=1, num_kv_heads=1, num_q_heads=4, k_format=fmt, v_format=fmt)
    _say(f"[middle-sized step {fmt}] generating + encoding")
    cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=np.array([tokens]))
    m, g, t = S.compare_codes(cache, 0, k_list[0], v_list[0], int(L[0]), w, codebooks)
    assert g <= 1e-4 * t
    rel, mx = S.assert_close(got[0], S.oracle_on_bytes(cache, 0, int(L[0]), q[0], codebooks), "on GPU bytes")
    _say(f"[middle-sized step {fmt}] rel-L2 {rel:.2e} max-abs {mx:.2e}; codes {m} / {t} mismatched, {g} in the margin")


@pytest.mark.parametrize("variant", [0, "fused"])
@pytest.mark.parametrize("fmt,hq", [("turbo4", 4), ("turbo3", 8)])
def test_row_at_maximum_capacity(fmt, hq, variant, codebooks):
    """A (sequence, KV head) row at the largest capacity the library accepts (2^24 tokens; the
    decode kernel addresses a row's K records, V tiles and norms with 32-bit byte offsets, here
    up to 2^30).  A 256-token block is encoded once and its bytes copied over the whole row on
    the device, with the V norms of every odd copy doubled (exact in fp16).  The copies' keys
    are identical, so are their softmax weights, and attention over all 2^24 tokens is 1.5
    times the oracle's attention over the one block; a read that lands on the wrong copy, or
    past the row (zeros), shows in that factor."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    cap, blk = tq.binding.MAX_CAPACITY, 256
    w = S.scaled(get_workload(0), batch=1, num_kv_heads=1, num_q_heads=hq, k_format=fmt, v_format=fmt)
    k_list, v_list = S.gen_kv(w, 0, [blk], "k"), S.gen_kv(w, 0, [blk], "v")
    _say(f"[maximum capacity {fmt}] encoding {blk} tokens, copying them over {cap}")
    cache = S.encode_on_gpu(w, k_list, v_list, [blk], cap)
    reps = cap // blk
    k, kn = cache.k_data[0, 0], cache.k_norms[0, 0]
    v, vn = cache.v_data[0, 0], cache.v_norms[0, 0]
    k.view(reps, blk, -1)[1:] = k[:blk]
    kn.view(reps, blk)[1:] = kn[:blk]
    v.view(reps, blk // 32, -1)[1:] = v[:blk // 32]
    vn.view(reps, blk)[1:] = vn[:blk]
    vn.view(torch.float16).view(reps, blk)[1::2] *= 2
    cache.seq_lens.fill_(cap)
    cache.lengths[:] = cap
    q = queries(w, 0)
    got = S.gpu_decode(cache, q, variant=variant)
    d = {"k_rec": cache.k_data[0][:, :blk].cpu().numpy(),
         "k_norms": cache.k_norms[0][:, :blk].cpu().numpy().view(np.float16),
         "v_tiles": cache.v_data[0][:, :blk // 32].cpu().numpy(),
         "v_norms": cache.v_norms[0][:, :blk].cpu().numpy().view(np.float16)}
    k_hat, v_hat = S.oracle_dequant_download(d, fmt, fmt, blk, codebooks)
    want = 1.5 * reference.decode_sequence(q[0], k_hat, v_hat, blk)
    rel, mx = S.assert_close(got[0], want, "copies of one block")
    _say(f"[maximum capacity {fmt} v{variant}] rel-L2 {rel:.2e} max-abs {mx:.2e}")


@pytest.mark.timeout(600)
def test_bandwidth_bound_step_edge_rows(codebooks):
    """A step large enough (>= 4M token-heads) that the row's first two splits append the token,
    with rows whose step appends their first token, whose only split is the one appending K,
    and rows whose earlier tokens end one short of and exactly on a split boundary (splits of
    1600 tokens here)."""
    w = get_workload(4)
    lens = np.array([1, 2, 33, 1600, 1601, 131072, 131072, 131072, 131072])
    w = S.scaled(w, batch=len(lens))
    assert int((lens - 1).sum()) * w.num_kv_heads >= 4 << 20
    _say("[bandwidth-bound step] generating + encoding")
    cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
    np.testing.assert_array_equal(cache.seq_lens.cpu().numpy(), L)
    for b in (0, 1, 2, 3, 4, 5):
        m, g, t = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        assert m <= g <= 1e-4 * t
        rel, mx = S.assert_close(got[b], S.oracle_on_bytes(cache, b, int(L[b]), q[b], codebooks), f"b={b}")
        _say(f"[bandwidth-bound step] b={b} L={int(L[b])} rel-L2 {rel:.2e} max-abs {mx:.2e}")
    assert np.all(np.isfinite(got.astype(np.float32)))


# ----------------------------------------------------------------------------- sparse V

@pytest.mark.parametrize("variant", [0, "fused"])
def test_sparse_v_skips_nothing_on_gaussian_scores(variant, codebooks):
    """At tau = 1e-6 the benchmark-like inputs (Gaussian keys and queries) leave no V tile
    below the threshold, so the output is bit-identical to exact attention's."""
    w, lens = _small_workloads()["c1"]
    cache, _, _, _, q = S.prefill_and_step(w, lengths=lens)
    exact = S.gpu_decode(cache, q, variant=variant)
    cache.v_skip_threshold = 1e-6
    np.testing.assert_array_equal(S.gpu_decode(cache, q, variant=variant), exact)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tau", [1e-6, 1e-2])
@pytest.mark.parametrize("variant", [0, "fused", "step"])
def test_sparse_v_drops_only_droppable_tokens(tau, variant, codebooks):
    """Peaked scores (queries x16, G = 4) on a call large enough (>= 4M token-heads) that the
    splits run 16 iterations: the output with sparse V moves from the exact route's by at
    most the oracle's bound for what may be dropped (tokens whose weight is below tau for
    every head of the group; tau widened by 10% for the scores' fp16 rounding), and at
    tau = 1e-2 it does drop.  (A split's first tile per token set sets its running max and
    is never skipped, so short splits skip little.)"""
    import torch

    import quantized_kv_cache_decode_amd as tq
    from oracle import attention as att
    from synth import kv_slice
    B, L = 64, 8200
    w = S.scaled(get_workload(0), batch=B, num_q_heads=32, num_kv_heads=8)
    pre = L - (1 if variant == "step" else 0)
    assert pre * B * 8 >= 4 << 20
    # every sequence holds the same keys and values (one generated sequence, copied on the GPU)
    k0 = np.stack([kv_slice(w, 0, "k", 0, h, pre) for h in range(8)])
    v0 = np.stack([kv_slice(w, 0, "v", 0, h, pre) for h in range(8)])
    cache = S.make_cache(w, 8224)
    tq.tq_encode_append(cache, torch.from_numpy(k0).cuda()[None].expand(B, -1, -1, -1).contiguous(),
                        torch.from_numpy(v0).cuda()[None].expand(B, -1, -1, -1).contiguous())
    q = (queries(w, 0) * 16).astype(np.float32)
    kn, vn = S.new_token_rows(w, 0)

    def run(threshold):
        cache.v_skip_threshold = threshold
        if variant == "step":
            cache.set_lengths(np.full(B, pre, dtype=np.int32))   # the step rewrites the same slot
            return S.gpu_decode_step(cache, kn, vn, q).astype(np.float64)
        return S.gpu_decode(cache, q, variant=variant).astype(np.float64)

    exact = run(0.0)
    got = run(tau)
    moved = 0.0
    for b in (0, B - 1):
        k_hat, v_hat = S.oracle_dequant_bytes(cache, b, L, codebooks)
        _, bound = att.sparse_v_bound(q[b], k_hat, v_hat, L, S.SCALE, 1.1 * tau)
        diff = np.abs(got[b] - exact[b])
        slack = np.abs(exact[b]) * 2.0 ** -9 + 1e-5   # the two routes' fp16 output rounding
        assert np.all(diff <= bound + slack), f"b={b}: {np.max(diff - bound - slack)}"
        moved = max(moved, float(diff.max()))
        _say(f"[sparse V {variant} tau={tau}] b={b} max move {diff.max():.2e}, max bound {bound.max():.2e}")
    if tau >= 1e-2:
        assert moved > 0.0


# ----------------------------------------------------------------------------- sparse K

@pytest.mark.parametrize("variant", [0, "fused"])
def test_sparse_k_skips_nothing_on_gaussian_scores(variant, codebooks):
    """At tau = 1e-6 the norm bound of Gaussian keys (about 24 above the scores' scale)
    never falls below the running max + ln tau, so the output is bit-identical to exact
    attention's."""
    w, lens = _small_workloads()["c1"]
    cache, _, _, _, q = S.prefill_and_step(w, lengths=lens)
    exact = S.gpu_decode(cache, q, variant=variant)
    cache.k_skip_threshold = 1e-6
    np.testing.assert_array_equal(S.gpu_decode(cache, q, variant=variant), exact)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("variant", [0, "fused", "step"])
def test_sparse_k_drops_only_droppable_tokens(variant, codebooks):
    """Keys with small norms outside every 512-token block's first 128 tokens (K x 0.01,
    their V x 1000 so that their weight shows), queries x 3, G = 4, a call of >= 4M
    token-heads (splits of many 128-token iterations).  The iterations of small-norm keys
    qualify at tau = 1e-2 once a split has seen a block start (the norm bound, about 0.7,
    is below a running max of about 7.8 + ln 1e-2) and never at 1e-6.  With the skip the
    output moves from the exact route's by at most the oracle's bound for dropping tokens
    from the whole softmax (tau widened by 10% for the scores' fp16 rounding) -- and it
    does move; at 1e-6 it is bit-identical."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    from oracle import attention as att
    from synth import kv_slice
    B, L = 64, 8200
    w = S.scaled(get_workload(0), batch=B, num_q_heads=32, num_kv_heads=8)
    pre = L - (1 if variant == "step" else 0)
    assert pre * B * 8 >= 4 << 20
    small = (np.arange(pre) % 512) >= 128
    k0 = np.stack([kv_slice(w, 0, "k", 0, h, pre) for h in range(8)]).astype(np.float32)
    v0 = np.stack([kv_slice(w, 0, "v", 0, h, pre) for h in range(8)]).astype(np.float32)
    k0[:, small] *= 0.01
    v0[:, small] *= 1000.0
    k0, v0 = k0.astype(np.float16), v0.astype(np.float16)
    cache = S.make_cache(w, 8224)
    tq.tq_encode_append(cache, torch.from_numpy(k0).cuda()[None].expand(B, -1, -1, -1).contiguous(),
                        torch.from_numpy(v0).cuda()[None].expand(B, -1, -1, -1).contiguous())
    q = (queries(w, 0) * 3).astype(np.float32)
    kn, vn = S.new_token_rows(w, 0)

    def run(threshold):
        cache.k_skip_threshold = threshold
        if variant == "step":
            cache.set_lengths(np.full(B, pre, dtype=np.int32))   # the step rewrites the same slot
            return S.gpu_decode_step(cache, kn, vn, q).astype(np.float64)
        return S.gpu_decode(cache, q, variant=variant).astype(np.float64)

    exact = run(0.0)
    np.testing.assert_array_equal(run(1e-6), exact)
    got = run(1e-2)
    moved = 0.0
    for b in (0, B - 1):
        k_hat, v_hat = S.oracle_dequant_bytes(cache, b, L, codebooks)
        _, bound = att.sparse_k_bound(q[b], k_hat, v_hat, L, S.SCALE, 1.1e-2)
        diff = np.abs(got[b] - exact[b])
        slack = np.abs(exact[b]) * 2.0 ** -9 + 1e-5   # the two routes' fp16 output rounding
        assert np.all(diff <= bound + slack), f"b={b}: {np.max(diff - bound - slack)}"
        moved = max(moved, float(diff.max()))
        _say(f"[sparse K {variant}] b={b} max move {diff.max():.2e}, max bound {bound.max():.2e}")
    assert moved > 0.0


# ----------------------------------------------------------------------------- chunk (Tq > 1)

def _gpu_chunk(cache, q_np):
    import torch

    import quantized_kv_cache_decode_amd as tq
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    B, Hq, Tq, _ = q.shape
    out = torch.empty((B, Hq, Tq, 128), dtype=torch.float16, device="cuda")
    ws = torch.zeros(tq.tq_decode_workspace_size(cache, Hq * Tq), dtype=torch.uint8, device="cuda")
    tq.tq_decode_chunk_fused(cache, q, S.SCALE, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("group,q_len,k_format,v_format", [
    (2, 3, "turbo3", "turbo3"), (4, 4, "turbo4", "turbo4"), (7, 2, "f16", "turbo4"), (1, 16, "turbo3", "turbo4"),
    (8, 2, "turbo3", "turbo3"), (1, 5, "f16", "turbo3"), (4, 3, "f16", "turbo3"), (7, 2, "f16", "turbo3"),
    (16, 1, "f16", "turbo3")])
def test_chunk_decode_parity(group, q_len, k_format, v_format, codebooks):
    """Causal decode of a chunk of q_len positions per sequence against the oracle, with a
    sequence exactly q_len long, one whose chunk straddles a split boundary (129 tokens,
    128-token splits), a tile-aligned and a ragged one."""
    from oracle import attention as att
    w = S.scaled(get_workload(0), batch=4, num_q_heads=2 * group, num_kv_heads=2, k_format=k_format,
                 v_format=v_format)
    lens = np.array([q_len, 129, 256, 1000])
    cache, _, _, L, _ = S.prefill_and_step(w, lengths=lens)
    q = np.stack([queries(w, 0, step=t) for t in range(q_len)], axis=2)     # [B, Hq, Tq, 128]
    got = _gpu_chunk(cache, q)
    for b in range(4):
        k_hat, v_hat = S.oracle_dequant_bytes(cache, b, int(L[b]), codebooks)
        ref = att.attention_chunk(q[b:b + 1], [k_hat], [v_hat], [int(L[b])], S.SCALE)[0]
        S.assert_close(got[b], ref, f"G={group} q_len={q_len} b={b} L={int(L[b])}")


def test_chunk_of_one_is_the_fused_decode():
    w, lens = _small_workloads()["c1"]
    cache, _, _, _, q = S.prefill_and_step(w, lengths=lens)
    np.testing.assert_array_equal(_gpu_chunk(cache, q[:, :, None])[:, :, 0], S.gpu_decode(cache, q, "fused"))


# ----------------------------------------------------------------------------- fp16 comparison cache

@pytest.mark.parametrize("group", [1, 7, 16])
@pytest.mark.parametrize("variant", [0, "fused", "step", "chunk"])
def test_f16_cache_parity(group, variant, codebooks):
    """The uncompressed fp16 K and V cache (the pages' '× fp16' comparison point) through the
    same MFMA decode: rows stored bit for bit, outputs against the oracle's plain attention on
    them, through the separate, fused, step and chunk calls."""
    from oracle import attention as att
    w = S.scaled(get_workload(0), batch=3, num_q_heads=2 * group, num_kv_heads=2, k_format="f16",
                 v_format="f16")
    lens = np.array([2, 300, 64])
    if variant == "step":
        cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
    else:
        cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
    if variant == "chunk":
        q_len = 2 if group <= 8 else 1
        qc = np.stack([queries(w, 0, step=t) for t in range(q_len)], axis=2)
        got = _gpu_chunk(cache, qc)
    elif variant != "step":
        got = S.gpu_decode(cache, q, variant=variant)
    for b in range(3):
        m, _, _ = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        assert m == 0
        if variant == "chunk":
            k_hat, v_hat = S.oracle_dequant_bytes(cache, b, int(L[b]), codebooks)
            want = att.attention_chunk(qc[b:b + 1], [k_hat], [v_hat], [int(L[b])], S.SCALE)[0]
        else:
            want = S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks)
        S.assert_close(got[b], want, f"fp16 cache {variant} G={group} b={b} L={int(L[b])}")


@pytest.mark.parametrize("group,k_format,v_format", [(7, "turbo3", "turbo3"), (7, "f16", "turbo4"),
                                                     (16, "turbo4", "turbo3"), (16, "f16", "f16")])
@pytest.mark.parametrize("variant", [0, "fused", "step"])
def test_split_waves_with_few_or_no_tokens(group, k_format, v_format, variant, codebooks):
    """Small calls run four waves per 128-token split, each streaming a quarter of its tokens
    in 32-token iterations: lengths that leave one, two, three or all four waves with tokens
    (and splits of one token) give the same outputs as the oracle."""
    lens = np.array([1, 31, 32, 33, 64, 96, 97, 128, 129, 200, 255, 257, 383])
    w = S.scaled(get_workload(0), batch=len(lens), num_q_heads=2 * group, num_kv_heads=2, k_format=k_format,
                 v_format=v_format)
    if variant == "step":
        cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
    else:
        cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
        got = S.gpu_decode(cache, q, variant=variant)
    for b in range(len(lens)):
        want = S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks)
        S.assert_close(got[b], want, f"{variant} G={group} {k_format}/{v_format} L={int(L[b])}")


@pytest.mark.parametrize("k_format,v_format", [("turbo3", "turbo3"), ("turbo4", "turbo3")])
@pytest.mark.parametrize("variant", [0, "fused", "step"])
def test_uneven_split_waves(k_format, v_format, variant, codebooks):
    """A small call whose plan cuts 320-token splits (4 rows of 18000 tokens): the four waves of
    a split take 3, 3, 3 and 1 of its 32-token iterations, and the last split's short tail
    leaves two of them without tokens."""
    lens = np.array([18000])
    w = S.scaled(get_workload(1), batch=1, k_format=k_format, v_format=v_format)
    if variant == "step":
        cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
    else:
        cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
        got = S.gpu_decode(cache, q, variant=variant)
    want = S.oracle_end_to_end(w, k_list[0], v_list[0], int(L[0]), q[0], codebooks)
    S.assert_close(got[0], want, f"{variant} {k_format}/{v_format} L={int(L[0])}")


# ----------------------------------------------------------------------------- many sequences

@pytest.mark.parametrize("variant", ["fused", "step"])
def test_more_sequences_than_one_launch(variant, codebooks):
    """300 sequences: the calls split them into launches of 256 (host lengths ride in the
    kernel arguments); sequences on both sides of the seam, and the last, are checked."""
    w = S.scaled(get_workload(0), batch=300)
    lens = 1 + np.random.default_rng(7).integers(0, 80, 300)
    if variant == "step":
        cache, k_list, v_list, L, q, got = S.prefill_then_decode_step(w, lengths=lens)
        np.testing.assert_array_equal(cache.seq_lens.cpu().numpy(), L)
    else:
        cache, k_list, v_list, L, q = S.prefill_and_step(w, lengths=lens)
        got = S.gpu_decode(cache, q, variant="fused")
    for b in (0, 255, 256, 299):
        m, _, _ = S.compare_codes(cache, b, k_list[b], v_list[b], int(L[b]), w, codebooks)
        assert m == 0
        S.assert_close(got[b], S.oracle_end_to_end(w, k_list[b], v_list[b], int(L[b]), q[b], codebooks),
                       f"{variant} b={b} L={int(L[b])}")


# ----------------------------------------------------------------------------- measurement aid

@pytest.mark.parametrize("n_bytes,blocks", [(16, 1), (4096, 3), ((1 << 24) + 48, 1024)])
def test_stream_read_reads_every_word(n_bytes, blocks):
    """The streaming-read kernel behind the HBM read ceiling reads every 16-byte word once:
    the XOR of its per-work-group checksums equals the XOR of the buffer's 32-bit words."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    words = np.random.default_rng(3).integers(0, 2 ** 32, n_bytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sums = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    tq.tq_stream_read(src, sums)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sums.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


# ----------------------------------------------------------------------------- encoder edge rows

def _adversarial_rows():
    """fp16 rows whose norms sit on or next to fp16 rounding midpoints (exact ties both
    ways, a hair above a tie), in the subnormal range, at saturation, and all-zero or
    single-element rows, plus Gaussian rows scaled across the fp16 range."""
    rows = []
    def row(vals):
        x = np.zeros(128, dtype=np.float16)
        x[:len(vals)] = np.array(vals, dtype=np.float64).astype(np.float16)
        return x
    rows += [row([2048, 64, 1]),                       # sqrt = 2049: tie, even wins (2048)
             row([2048, 110, 14, 1]),                  # sqrt = 2051: tie, even wins (2052)
             row([2048, 64, 1, 2.0 ** -24]),           # a hair above the tie: 2050
             row([3 * 2.0 ** -24, 4 * 2.0 ** -24]),    # subnormal, exact
             row([-7.5]), row([0.0]), row([65504.0]), row([65504.0, 65504.0]),
             row([60000.0, 20000.0]), row([2.0 ** -14, -2.0 ** -14, 2.0 ** -24]),
             row([1.0] * 128), row([-1.0] * 64 + [1.0] * 64), row([0.5] * 4)]
    rng = np.random.default_rng(11)
    for scale in (2.0 ** -20, 2.0 ** -12, 1.0, 64.0, 2048.0):
        g = rng.standard_normal((24, 128)) * scale
        rows += list(np.clip(g, -65504, 65504).astype(np.float16))
    return np.stack(rows)


@pytest.mark.parametrize("fmt", ["turbo3", "turbo4"])
def test_encode_adversarial_norms_and_codes(fmt, codebooks):
    """Rows whose norm rounding is decided by the encoder's exact fallback (ties and near-ties),
    subnormal and saturating norms, zero rows: norms bit for bit and codes equal to the oracle's
    outside the 1e-5 boundary margin, through the bulk append, the decode step and the one-row
    append kernel."""
    import torch

    import quantized_kv_cache_decode_amd as tq
    x = _adversarial_rows()
    n = len(x)
    w = S.scaled(get_workload(0), batch=1, num_q_heads=2, num_kv_heads=1, k_format=fmt, v_format=fmt)
    cap = ((n + 31) // 32) * 32
    cache = S.make_cache(w, cap)
    kx = torch.from_numpy(x[None, None]).cuda()
    tq.tq_encode_append(cache, kx, kx.clone())
    m, g, t = S.compare_codes(cache, 0, x[None], x[None], n, w, codebooks)
    assert m <= g
    _say(f"[adversarial {fmt}] {n} rows: codes {m} mismatches / {t}, {g} within the margin")
    # the decode step's in-kernel append: each row in turn as the step's new token
    cache2 = S.make_cache(w, cap)
    q = np.zeros((1, 2, 128), dtype=np.float16)
    for i in range(n):
        S.gpu_decode_step(cache2, x[None, None, i:i + 1], x[None, None, i:i + 1], q)
    m2, g2, t2 = S.compare_codes(cache2, 0, x[None], x[None], n, w, codebooks)
    assert m2 <= g2
    # the one-row append kernel: each row in turn through tq_encode_append of one token
    cache3 = S.make_cache(w, cap)
    for i in range(n):
        xi = torch.from_numpy(np.ascontiguousarray(x[None, None, i:i + 1])).cuda()
        tq.tq_encode_append(cache3, xi, xi.clone())
    m3, g3, t3 = S.compare_codes(cache3, 0, x[None], x[None], n, w, codebooks)
    assert m3 <= g3
