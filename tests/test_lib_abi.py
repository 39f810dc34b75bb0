"""CPU-side checks of libtqattn: it loads, exports every declared entry point, and
validates arguments on the host (no kernel is launched by these calls)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_kv_cache_decode_amd as tq
from quantized_kv_cache_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tqattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from quantized_kv_cache_decode_amd import build
        build.build(verbose=False)
    return tq.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "tq_decode_attention" in names and "tq_encode_append" in names
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (tq_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(binding.EXPORTED) == set(names)


def test_library_is_built_for_gfx950(lib):
    data = open(binding.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def _desc(**over):
    fake = 0x10000
    d = dict(batch=2, num_kv_heads=2, head_dim=128, capacity=64, k_format=3, v_format=3,
             k_data=fake, k_norms=fake, v_data=fake, v_norms=fake, seq_lens=fake, k_signs=fake,
             v_signs=fake, k_codebook=fake, v_codebook=fake)
    d.update(over)
    return binding.tq_cache(**d)


def _lens(*v):
    a = np.array(v, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _err(lib):
    return lib.tq_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), binding.TQ_EUNSUPPORTED),
    (dict(capacity=48), binding.TQ_EINVAL),
    (dict(capacity=0), binding.TQ_EINVAL),
    (dict(capacity=(1 << 24) + 32), binding.TQ_EINVAL),
    (dict(v_format=0), binding.TQ_EUNSUPPORTED),
    (dict(k_format=7), binding.TQ_EUNSUPPORTED),
    (dict(v_data=0), binding.TQ_EINVAL),
    (dict(k_norms=0), binding.TQ_EINVAL),
    (dict(batch=0), binding.TQ_EINVAL),
])
def test_bad_cache_descriptors(lib, over, status):
    d = _desc(**over)
    a, p = _lens(0, 0)
    q = ctypes.c_void_p(0x20000)
    assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 4, q, None) == status
    assert _err(lib)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 1, None, None) == status


def test_f16_k_needs_no_norms(lib):
    d = _desc(k_format=0, k_norms=0, k_signs=0, k_codebook=0)
    a, p = _lens(0, 0)
    # valid descriptor; the error comes from the heads check, proving the descriptor passed
    assert lib.tq_rotate_q(ctypes.byref(d), ctypes.c_void_p(1), 0, 3, ctypes.c_void_p(1), None) == binding.TQ_EINVAL
    assert "num_q_heads" in _err(lib)


def test_heads_checks(lib):
    d = _desc()
    q = ctypes.c_void_p(0x20000)
    assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 3, q, None) == binding.TQ_EINVAL        # 3 % 2
    assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 34, q, None) == binding.TQ_EUNSUPPORTED  # group 17
    assert lib.tq_rotate_q(ctypes.byref(d), ctypes.c_void_p(0), 0, 4, q, None) == binding.TQ_EINVAL


def test_append_capacity_and_counts(lib):
    d = _desc()
    q = ctypes.c_void_p(0x20000)
    a, p = _lens(60, 10)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 5, None, None) == binding.TQ_ECAPACITY
    assert "capacity" in _err(lib)
    c, pc = _lens(6, 0)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 5, pc, None) == binding.TQ_EINVAL      # count > t_new
    c, pc = _lens(-1, 0)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 5, pc, None) == binding.TQ_EINVAL
    a, p = _lens(-3, 0)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 0, None, None) == binding.TQ_EINVAL
    a, p = _lens(10, 10)
    assert lib.tq_encode_append(ctypes.byref(d), p, q, q, 0, None, None) == binding.TQ_OK          # no-op
    assert lib.tq_encode_append(ctypes.byref(d), ctypes.c_void_p(0), q, q, 1, None, None) == binding.TQ_EINVAL


def test_workspace_size_and_check(lib):
    d = _desc()
    a, p = _lens(64, 17)
    n = lib.tq_decode_workspace_size(ctypes.byref(d), 4, p)
    assert n > 0 and n % 4 == 0
    # one split per (sequence, KV head) at these lengths, plus the decode step's slot:
    # 2*2*(1+1) slots x group 2 x 130 floats
    assert n == 2 * 2 * 2 * 2 * 130 * 4
    q = ctypes.c_void_p(0x20000)
    st = lib.tq_decode_attention(ctypes.byref(d), p, q, 4, ctypes.c_float(0.1), q, q, n - 4, None)
    assert st == binding.TQ_EWORKSPACE
    st = lib.tq_decode_attention_variant(ctypes.byref(d), p, q, 4, ctypes.c_float(0.1), q, q, n, 9, None)
    assert st == binding.TQ_EINVAL
    a, p = _lens(65, 0)
    assert lib.tq_decode_workspace_size(ctypes.byref(d), 4, p) == 0
    assert lib.tq_decode_attention(ctypes.byref(d), p, q, 4, ctypes.c_float(0.1), q, q, 10 ** 9, None) == \
        binding.TQ_ECAPACITY


def test_workspace_grows_with_context(lib):
    d = _desc(batch=1, num_kv_heads=8, capacity=131072)
    sizes = []
    for L in (256, 4096, 131072):
        a, p = _lens(L)
        sizes.append(lib.tq_decode_workspace_size(ctypes.byref(d), 64, p))
    assert sizes[0] <= sizes[1] <= sizes[2]


@pytest.mark.parametrize("batch,hkv,hq,lens,bytes_per_token", [
    (32, 8, 32, [32768] * 32, 132),                                 # batched turbo4
    (16, 8, 64, list(np.linspace(1024, 131072, 16).astype(int)), 100),  # ragged turbo3
])
def test_partials_are_small_next_to_the_cache(lib, batch, hkv, hq, lens, bytes_per_token):
    """In the bandwidth-bound regime the split partials (written once, read once) stay
    under 5% of the packed K+V bytes a decode call streams.  The workspace holds
    max_splits partials per (sequence, KV head); the splits actually written are
    bounded through the smallest chunk consistent with that max_splits."""
    d = _desc(batch=batch, num_kv_heads=hkv, capacity=131072)
    a, p = _lens(*lens)
    ws = lib.tq_decode_workspace_size(ctypes.byref(d), hq, p)
    group = hq // hkv
    per_item = group * 130 * 4
    assert ws % (batch * hkv * per_item) == 0
    max_splits = ws // (batch * hkv * per_item) - 1   # one slot per row is the decode step's
    chunk_min = -(-max(lens) // max_splits)
    items = sum(hkv * -(-int(L) // chunk_min) for L in lens)
    kv = sum(lens) * hkv * bytes_per_token
    assert 2 * items * per_item < 0.05 * kv


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_LIB", None)
    with pytest.raises(FileNotFoundError):
        binding.load_library(str(tmp_path / "missing.so"))


def test_no_kernel_spills_to_scratch():
    """Every kernel of the last build keeps its state in registers/LDS: a spill to scratch
    memory (or a private array the compiler could not promote) would put per-lane memory
    traffic on the hot path.  Reads the compiler's resource remarks that build.py records."""
    from quantized_kv_cache_decode_amd import build
    if not os.path.exists(build.RESOURCE_REPORT):
        pytest.skip("no build in this tree (build.py writes the resource report)")
    lines = [l.split() for l in open(build.RESOURCE_REPORT).read().splitlines() if l.strip()]
    assert lines, "empty resource report"
    spills = [l for l in lines if l[-1] != "scratch=0"]
    assert not spills, spills


def test_chunk_decode_checks(lib):
    """tq_decode_chunk_fused: q_len >= 1, group * q_len <= 16 columns, every sequence holds the
    chunk, and the workspace is sized for group * q_len columns."""
    d = _desc()                       # 2 KV heads
    q = ctypes.c_void_p(0x20000)
    a, p = _lens(40, 9)
    big = 10 ** 9

    def call(heads, q_len, ws=big):
        return lib.tq_decode_chunk_fused(ctypes.byref(d), p, q, 0, heads, q_len, ctypes.c_float(0.1), q, q, ws, None)

    assert call(4, 0) == binding.TQ_EINVAL
    assert call(4, 9) == binding.TQ_EUNSUPPORTED and "q_len" in _err(lib)     # group 2 x 9 > 16
    assert call(4, 10) == binding.TQ_EUNSUPPORTED
    assert call(2, 10) == binding.TQ_EINVAL and "fewer" in _err(lib)          # sequence 1 holds 9 < 10
    n = lib.tq_decode_workspace_size(ctypes.byref(d), 4 * 8, p)
    assert n > 0
    assert call(4, 8, n - 4) == binding.TQ_EWORKSPACE


def test_sparse_v_threshold_range(lib):
    q = ctypes.c_void_p(0x20000)
    for tau, status in ((-0.5, binding.TQ_EINVAL), (1.5, binding.TQ_EINVAL), (float("nan"), binding.TQ_EINVAL)):
        d = _desc(v_skip_threshold=tau)
        assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 4, q, None) == status
        assert "v_skip_threshold" in _err(lib)


def test_sparse_k_threshold_range(lib):
    q = ctypes.c_void_p(0x20000)
    for tau, status in ((-0.5, binding.TQ_EINVAL), (1.5, binding.TQ_EINVAL), (float("nan"), binding.TQ_EINVAL)):
        d = _desc(k_skip_threshold=tau)
        assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 4, q, None) == status
        assert "k_skip_threshold" in _err(lib)
    d = _desc(k_skip_threshold=1e-6)   # valid: the heads check fails next
    assert lib.tq_rotate_q(ctypes.byref(d), q, 0, 3, q, None) == binding.TQ_EINVAL
    assert "num_q_heads" in _err(lib)


def test_f16_v_only_with_f16_k(lib):
    q = ctypes.c_void_p(0x20000)
    ok = _desc(k_format=0, v_format=0, k_norms=0, k_signs=0, k_codebook=0, v_norms=0, v_signs=0, v_codebook=0)
    # valid descriptor (the heads check fails next, proving it passed)
    assert lib.tq_rotate_q(ctypes.byref(ok), q, 0, 3, q, None) == binding.TQ_EINVAL
    assert "num_q_heads" in _err(lib)
    bad = _desc(k_format=3, v_format=0, v_norms=0)
    assert lib.tq_rotate_q(ctypes.byref(bad), q, 0, 4, q, None) == binding.TQ_EUNSUPPORTED
    a, p = _lens(10, 10)
    st = lib.tq_decode_attention_variant(ctypes.byref(ok), p, q, 4, ctypes.c_float(0.1), q, q, 10 ** 9, 1, None)
    assert st == binding.TQ_EUNSUPPORTED and "reference" in _err(lib)


def test_stream_read_checks(lib):
    """The streaming-read measurement aid validates before launching (no GPU needed)."""
    p = ctypes.c_void_p(0x10000)
    assert lib.tq_stream_read(None, 1024, p, 4, None) == binding.TQ_EINVAL
    assert lib.tq_stream_read(p, 1024, None, 4, None) == binding.TQ_EINVAL
    assert lib.tq_stream_read(p, 0, p, 4, None) == binding.TQ_EINVAL
    assert lib.tq_stream_read(p, 1000, p, 4, None) == binding.TQ_EINVAL
    assert lib.tq_stream_read(p, 1024, p, 0, None) == binding.TQ_EINVAL
    assert lib.tq_stream_read(p, 1024, p, (1 << 20) + 1, None) == binding.TQ_EINVAL


def test_noalloc_step_checks_before_touching_the_device(lib):
    """The no-allocation step rejects, on the host, calls whose partials exceed its per-GPU
    array (1024 x 8 rows of 2 slots x 16 heads x 520 bytes = 136 MB > 64 MiB), full caches
    and NULL pointers -- no device call is made on these paths."""
    q = ctypes.c_void_p(0x20000)
    d = _desc(batch=1024, num_kv_heads=8, capacity=32)
    a, p = _lens(*([10] * 1024))
    n = lib.tq_decode_workspace_size(ctypes.byref(d), 128, p)
    assert n > binding.NOALLOC_SCRATCH_BYTES
    st = lib.tq_decode_step_noalloc(ctypes.byref(d), p, q, q, q, 0, 128, ctypes.c_float(0.1), q, None)
    assert st == binding.TQ_EWORKSPACE and "scratch" in _err(lib)
    d = _desc()
    a, p = _lens(64, 3)
    assert lib.tq_decode_step_noalloc(ctypes.byref(d), p, q, q, q, 0, 4, ctypes.c_float(0.1), q, None) == \
        binding.TQ_ECAPACITY
    a, p = _lens(5, 3)
    assert lib.tq_decode_step_noalloc(ctypes.byref(d), p, q, ctypes.c_void_p(0), q, 0, 4, ctypes.c_float(0.1), q,
                                      None) == binding.TQ_EINVAL
    assert lib.tq_decode_step_noalloc(ctypes.byref(d), p, q, q, q, 0, 3, ctypes.c_float(0.1), q, None) == \
        binding.TQ_EINVAL


@pytest.mark.parametrize("k_format,v_format,L,slots", [
    # turbo3 8K layer: 32768 token-heads over 256 work items -> 128-token splits (12.8 KB of
    # packed K+V each), 64 per row, plus the step's slot
    (3, 3, 8192, 65),
    # fp16-K 16K layer: 256-token splits would stream 82 KB each, so the decode step's two
    # append groups per row are counted in: 248 items -> ceil(65536 / 248) = 265 tokens,
    # rounded up to 320 -> 52 splits per row, plus the step's slot
    (0, 4, 16384, 53),
])
def test_latency_plan_split_counts(lib, k_format, v_format, L, slots):
    """The small-call split plan, read off the workspace size (B*Hkv*slots*G partials of
    130 floats): one work group per compute unit, the append groups included when a split
    streams more than 32 KB."""
    fake = 0x10000
    d = _desc(batch=1, num_kv_heads=4, capacity=16384, k_format=k_format, v_format=v_format,
              k_norms=fake if k_format else 0)
    a, p = _lens(L)
    assert lib.tq_decode_workspace_size(ctypes.byref(d), 28, p) == 1 * 4 * slots * 7 * 130 * 4


def test_latency_plan_keeps_its_items_when_rows_are_many(lib):
    """With 2 append groups per row taking half the units or more, the plan does not shrink:
    64 sequences x 2 KV heads of 512 fp16-K tokens (65536 token-heads, 21 MB) -> 256 items of
    256 tokens (82 KB each), 2 per row, plus the step's slot."""
    d = _desc(batch=64, num_kv_heads=2, capacity=512, k_format=0, v_format=4, k_norms=0)
    a, p = _lens(*([512] * 64))
    assert lib.tq_decode_workspace_size(ctypes.byref(d), 4, p) == 64 * 2 * 3 * 2 * 130 * 4


def test_binding_constants_match_the_header():
    """The binding's copies of the header's size limits are the header's values."""
    import os
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "tqattn.h")).read()
    defs = {k: eval(v.replace("(size_t)", "")) for k, v in re.findall(r"^#define (TQ_\w+) (.+)$", text, re.M)}
    assert defs["TQ_MAX_CAPACITY"] == binding.MAX_CAPACITY
    assert defs["TQ_NOALLOC_SCRATCH_BYTES"] == binding.NOALLOC_SCRATCH_BYTES


def test_cache_capacity_checked_in_the_binding():
    with pytest.raises(ValueError):
        binding.Cache(1, 1, binding.MAX_CAPACITY + 32, "turbo4", "turbo4", None, None, device="cpu")
    with pytest.raises(ValueError):
        binding.Cache(1, 1, 48, "turbo4", "turbo4", None, None, device="cpu")
