"""The no-allocation decode step (tq_decode_step_noalloc, for callers that cannot allocate)
against tq_decode_step with a workspace: two calls in a row, the second on a smaller input,
each on identical cache copies -- outputs bit for bit, and the appended token's bytes and
the lengths equal; the first call's output also within the parity bars of the oracle."""
import sys

import numpy as np
import pytest

from synth import get_workload
from tests import support as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_kv_cache_decode_amd as tq
    tq.load_library()


def _copy(cache):
    import copy

    import quantized_kv_cache_decode_amd as tq
    c = copy.copy(cache)
    for name in ("k_data", "k_norms", "v_data", "v_norms", "seq_lens"):
        t = getattr(cache, name)
        setattr(c, name, None if t is None else t.clone())
    c.lengths = cache.lengths.copy()
    c._desc = tq.binding.tq_cache(
        cache.batch, cache.num_kv_heads, 128, cache.capacity, cache._desc.k_format, cache._desc.v_format,
        c.k_data.data_ptr(), 0 if c.k_norms is None else c.k_norms.data_ptr(), c.v_data.data_ptr(),
        0 if c.v_norms is None else c.v_norms.data_ptr(), c.seq_lens.data_ptr(), cache.k_signs.data_ptr(),
        cache.v_signs.data_ptr(), cache.k_codebook.data_ptr(), cache.v_codebook.data_ptr(), 0.0, 0.0)
    return c


def _bytes(cache):
    return [t.cpu().numpy().tobytes() for t in (cache.k_data, cache.k_norms, cache.v_data, cache.v_norms,
                                                 cache.seq_lens) if t is not None]


def _run(w, lens, codebooks, check_oracle):
    import torch

    import quantized_kv_cache_decode_amd as tq
    L = np.asarray(lens)
    pre = L - 1
    k_list = S.gen_kv(w, 0, pre, "k")
    v_list = S.gen_kv(w, 0, pre, "v")
    cap = int(((L.max() + 31) // 32) * 32)
    a = S.encode_on_gpu(w, k_list, v_list, pre, cap)
    b = _copy(a)
    kn, vn = S.new_token_rows(w, 0)
    kn_t, vn_t = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
    from synth import queries
    q_np = queries(w, 0)
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    out_a = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float16, device="cuda")
    out_b = torch.full_like(out_a, 7.0)
    ws = torch.full((tq.tq_decode_workspace_size(a, w.num_q_heads),), 0x7f, dtype=torch.uint8, device="cuda")
    tq.tq_decode_step(a, kn_t, vn_t, q, S.SCALE, out_a, ws)
    tq.tq_decode_step_noalloc(b, kn_t, vn_t, q, S.SCALE, out_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_b.cpu().numpy().view(np.uint16), out_a.cpu().numpy().view(np.uint16))
    assert _bytes(a) == _bytes(b)
    np.testing.assert_array_equal(b.lengths, L)
    if check_oracle:
        kf = [np.concatenate([k, kk], axis=1) for k, kk in zip(k_list, kn)]
        vf = [np.concatenate([v, vv], axis=1) for v, vv in zip(v_list, vn)]
        for bb in (0, w.batch - 1):
            S.assert_close(out_b.cpu().numpy()[bb],
                           S.oracle_end_to_end(w, kf[bb], vf[bb], int(L[bb]), q_np[bb], codebooks), f"b={bb}")
    print(f"[no-alloc] {w.name} B={w.batch} lengths {L.min()}..{L.max()}: bit-identical", file=sys.stderr,
          flush=True)


def test_noalloc_step_matches_the_workspace_step_twice(codebooks):
    """First a bandwidth-bound call (the row's first splits append; many partials), then a
    smaller latency-bound one (extra append work groups): the second call reuses the array
    the first left its partials in."""
    big = S.scaled(get_workload(4), batch=8, context=None)
    lens = np.array([131072, 131072, 131072, 131072, 99000, 4096, 1, 33])
    assert int((lens - 1).sum()) * big.num_kv_heads >= 4 << 20      # the bandwidth-bound plan
    _run(big, lens, codebooks, check_oracle=False)
    small = S.scaled(get_workload(1), context=None)
    _run(small, np.array([3000]), codebooks, check_oracle=True)


def test_noalloc_step_other_formats(codebooks):
    """fp16 K + turbo4 V at group 7 and turbo4 at group 4, both smaller again."""
    _run(S.scaled(get_workload(2), context=None), np.array([5000]), codebooks, check_oracle=True)
    _run(S.scaled(get_workload(3), batch=3, context=None), np.array([2048, 77, 513]), codebooks, check_oracle=True)
