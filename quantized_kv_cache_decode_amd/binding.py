"""Thin ctypes binding of libtqattn: argument marshalling only.

Every function has the C ABI's name and forwards device pointers
(torch tensors' data_ptr()) and the current HIP stream.  All arithmetic of the
decode path runs in the library's kernels; torch provides device memory and
streams.  Importing works without a GPU; calling a compute entry point needs
the built library and a GPU, and fails loudly otherwise.
"""
import ctypes
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtqattn.so")
TABLE_PATH = os.path.join(HERE, "tables", "codebooks.json")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ECAPACITY, TQ_EWORKSPACE, TQ_EHIP = range(6)
TQ_FMT = {"f16": 0, "turbo3": 3, "turbo4": 4}
K_RECORD_BYTES = {"turbo3": 48, "turbo4": 64}
V_TILE_BYTES = {"turbo3": 1536, "turbo4": 2048, "f16": 8192}
NOALLOC_SCRATCH_BYTES = 64 << 20   # TQ_NOALLOC_SCRATCH_BYTES: the no-allocation step's partials, per GPU
MAX_CAPACITY = 1 << 24             # TQ_MAX_CAPACITY: tokens per (sequence, KV head) row
EXPORTED = (
    "tq_encode_append", "tq_rotate_q", "tq_decode_workspace_size", "tq_decode_attention",
    "tq_decode_attention_variant", "tq_decode_attention_fused", "tq_decode_chunk_fused", "tq_decode_step",
    "tq_decode_step_noalloc",
    "tq_inverse_rotate_out", "tq_stream_read",
    "tq_last_error", "tq_version",
)


class TqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libtqattn status {status}: {message}")
        self.status = status


class tq_cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32), ("k_format", ctypes.c_int32), ("v_format", ctypes.c_int32),
        ("k_data", ctypes.c_void_p), ("k_norms", ctypes.c_void_p), ("v_data", ctypes.c_void_p),
        ("v_norms", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("k_signs", ctypes.c_void_p),
        ("v_signs", ctypes.c_void_p), ("k_codebook", ctypes.c_void_p), ("v_codebook", ctypes.c_void_p),
        ("v_skip_threshold", ctypes.c_float), ("k_skip_threshold", ctypes.c_float),
    ]


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtqattn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with `python -m quantized_kv_cache_decode_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    cp = ctypes.POINTER(tq_cache)
    lib.tq_encode_append.argtypes = [cp, P, P, P, I32, P, P]
    lib.tq_rotate_q.argtypes = [cp, P, I32, I32, P, P]
    lib.tq_decode_workspace_size.argtypes = [cp, I32, P]
    lib.tq_decode_workspace_size.restype = SZ
    lib.tq_decode_attention.argtypes = [cp, P, P, I32, F32, P, P, SZ, P]
    lib.tq_decode_attention_variant.argtypes = [cp, P, P, I32, F32, P, P, SZ, I32, P]
    lib.tq_decode_attention_fused.argtypes = [cp, P, P, I32, I32, F32, P, P, SZ, P]
    lib.tq_decode_step.argtypes = [cp, P, P, P, P, I32, I32, F32, P, P, SZ, P]
    lib.tq_decode_step_noalloc.argtypes = [cp, P, P, P, P, I32, I32, F32, P, P]
    lib.tq_decode_chunk_fused.argtypes = [cp, P, P, I32, I32, I32, F32, P, P, SZ, P]
    lib.tq_inverse_rotate_out.argtypes = [cp, P, I32, P, P]
    lib.tq_stream_read.argtypes = [P, SZ, P, I32, P]
    lib.tq_last_error.restype = ctypes.c_char_p
    lib.tq_version.restype = ctypes.c_char_p
    for name in ("tq_encode_append", "tq_rotate_q", "tq_decode_attention", "tq_decode_attention_variant",
                 "tq_decode_attention_fused", "tq_decode_chunk_fused", "tq_decode_step", "tq_decode_step_noalloc",
                 "tq_inverse_rotate_out", "tq_stream_read"):
        getattr(lib, name).restype = ctypes.c_int
    _LIB = lib
    return lib


def codebook_bits(fmt: str) -> np.ndarray:
    """Frozen fp16 codebook (uint16 bit patterns, ascending) of a quantised format."""
    with open(TABLE_PATH) as f:
        t = json.load(f)
    return np.array([int(h, 16) for h in t[fmt]["codebook_fp16_hex"]], dtype=np.uint16)


def _check(status):
    if status != TQ_OK:
        raise TqError(status, load_library().tq_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _host_i32(lengths, n=None, what="seq_lens_host"):
    arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    if n is not None and arr.shape != (n,):
        raise ValueError(f"{what} has shape {arr.shape}; one entry per sequence ({n}) is needed")
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


# Argument checks, all made before the library is called: the C ABI takes bare device
# pointers, so a tensor of the wrong shape, dtype, layout or device would otherwise become
# an out-of-bounds device access instead of a Python error.
def _tensor(t, name, shape, dtypes):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(cache, *named):
    """Every tensor (and the cache's own buffers) on the cache's GPU."""
    dev = cache.k_data.device
    if dev.type != "cuda":
        raise ValueError("the cache's buffers are not on a GPU")
    for name, t in named:
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the cache on {dev}")


def _workspace(workspace):
    import torch
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous torch tensor")
    return workspace


def _q_shape(cache, q, name="q"):
    """[B, Hq, 128] (or [B, Hq, Tq, 128] for a chunk) with Hq a multiple of Hkv."""
    if q.dim() < 3 or q.shape[0] != cache.batch or q.shape[-1] != 128 or q.shape[1] % cache.num_kv_heads:
        raise ValueError(f"{name} has shape {tuple(q.shape)}; expected [{cache.batch}, Hq, ..., 128] with Hq a "
                         f"multiple of {cache.num_kv_heads}")
    return tuple(q.shape)


class Cache:
    """Device buffers of one layer's KV cache (torch tensors) and their C descriptor.

    k_format: "turbo3" | "turbo4" | "f16"; v_format: "turbo3" | "turbo4", or "f16" with
    k_format "f16" (the uncompressed comparison cache).
    `lengths` is the host copy of the visible length per sequence; it is advanced
    by tq_encode_append together with the device copy."""

    def __init__(self, batch, num_kv_heads, capacity, k_format, v_format, k_signs, v_signs, device="cuda"):
        import torch
        if capacity <= 0 or capacity % 32 or capacity > MAX_CAPACITY:
            raise ValueError(f"capacity {capacity} must be a positive multiple of 32, at most {MAX_CAPACITY}")
        self.batch, self.num_kv_heads, self.capacity = batch, num_kv_heads, capacity
        self.k_format, self.v_format = k_format, v_format
        dev = torch.device(device)
        slots = (batch, num_kv_heads, capacity)
        if k_format == "f16":
            self.k_data = torch.zeros(slots + (128,), dtype=torch.float16, device=dev)
            self.k_norms = None
        else:
            self.k_data = torch.zeros(slots + (K_RECORD_BYTES[k_format],), dtype=torch.uint8, device=dev)
            self.k_norms = torch.zeros(slots, dtype=torch.int16, device=dev)
        self.v_data = torch.zeros((batch, num_kv_heads, capacity // 32, V_TILE_BYTES[v_format]),
                                  dtype=torch.uint8, device=dev)
        self.v_norms = None if v_format == "f16" else torch.zeros(slots, dtype=torch.int16, device=dev)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.k_signs = torch.as_tensor(np.asarray(k_signs, dtype=np.float32)).to(dev)
        self.v_signs = torch.as_tensor(np.asarray(v_signs, dtype=np.float32)).to(dev)
        cbk = codebook_bits(k_format) if k_format != "f16" else np.zeros(16, np.uint16)
        self.k_codebook = torch.as_tensor(cbk.view(np.int16).copy()).to(dev)
        cbv = codebook_bits(v_format) if v_format != "f16" else np.zeros(16, np.uint16)
        self.v_codebook = torch.as_tensor(cbv.view(np.int16).copy()).to(dev)
        self.lengths = np.zeros(batch, dtype=np.int32)
        self._desc = tq_cache(
            batch, num_kv_heads, 128, capacity, TQ_FMT[k_format], TQ_FMT[v_format],
            self.k_data.data_ptr(), 0 if self.k_norms is None else self.k_norms.data_ptr(),
            self.v_data.data_ptr(), 0 if self.v_norms is None else self.v_norms.data_ptr(), self.seq_lens.data_ptr(),
            self.k_signs.data_ptr(), self.v_signs.data_ptr(), self.k_codebook.data_ptr(),
            self.v_codebook.data_ptr(), 0.0, 0.0)

    @property
    def v_skip_threshold(self) -> float:
        """Sparse-V weight threshold of the decode calls (0 = exact attention)."""
        return float(self._desc.v_skip_threshold)

    @v_skip_threshold.setter
    def v_skip_threshold(self, tau: float):
        self._desc.v_skip_threshold = float(tau)

    @property
    def k_skip_threshold(self) -> float:
        """Sparse-K weight threshold of the decode calls (0 = exact attention)."""
        return float(self._desc.k_skip_threshold)

    @k_skip_threshold.setter
    def k_skip_threshold(self, tau: float):
        self._desc.k_skip_threshold = float(tau)

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def set_lengths(self, lengths):
        """Set the visible length of every sequence (host and device copies)."""
        import torch
        self.lengths = np.asarray(lengths, dtype=np.int32).copy()
        self.seq_lens.copy_(torch.as_tensor(self.lengths))


def tq_encode_append(cache: Cache, k_new, v_new, seq_lens_host=None, counts=None, stream=None):
    """Append fp16 rows k_new, v_new [B, Hkv, t_new, 128] at each sequence's current length.

    counts: optional per-sequence number of rows to take (ragged prefill)."""
    import torch
    if getattr(k_new, "dim", lambda: 0)() != 4:
        raise ValueError("k_new must be [B, Hkv, t_new, 128]")
    t_new = int(k_new.shape[2])
    shape = (cache.batch, cache.num_kv_heads, t_new, 128)
    _tensor(k_new, "k_new", shape, (torch.float16,))
    _tensor(v_new, "v_new", shape, (torch.float16,))
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    if counts is None:
        cnt, pc = np.full(cache.batch, t_new, dtype=np.int32), ctypes.c_void_p(0)
    else:
        cnt, pc = _host_i32(counts, cache.batch, "counts")
    _on_gpu(cache, ("k_new", k_new), ("v_new", v_new))
    _check(load_library().tq_encode_append(cache.desc, p, _ptr(k_new), _ptr(v_new), t_new, pc, _stream(stream)))
    cache.lengths = arr + cnt


def tq_rotate_q(cache: Cache, q, q_rot, stream=None):
    """q [B, Hq, 128] (fp16 or fp32) -> q_rot fp32 in K's codec basis."""
    import torch
    shape = _q_shape(cache, q)
    if len(shape) != 3:
        raise ValueError("q must be [B, Hq, 128]")
    _tensor(q, "q", shape, (torch.float16, torch.float32))
    _tensor(q_rot, "q_rot", shape, (torch.float32,))
    _on_gpu(cache, ("q", q), ("q_rot", q_rot))
    _check(load_library().tq_rotate_q(cache.desc, _ptr(q), int(q.dtype == torch.float32), int(q.shape[1]),
                                      _ptr(q_rot), _stream(stream)))


def tq_decode_workspace_size(cache: Cache, num_q_heads: int, seq_lens_host=None) -> int:
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    n = load_library().tq_decode_workspace_size(cache.desc, num_q_heads, p)
    if n == 0:
        raise TqError(TQ_EINVAL, load_library().tq_last_error().decode())
    return int(n)


def tq_decode_attention(cache: Cache, q_rot, scale, out_rot, workspace, seq_lens_host=None, variant=0,
                        stream=None):
    """out_rot [B, Hq, 128] fp32 = decode attention in V's rotated basis (workspace: device memory).

    variant 0 (default): the MFMA kernel; 1: the plain VALU reference kernel."""
    import torch
    shape = _q_shape(cache, q_rot, "q_rot")
    if len(shape) != 3:
        raise ValueError("q_rot must be [B, Hq, 128]")
    _tensor(q_rot, "q_rot", shape, (torch.float32,))
    _tensor(out_rot, "out_rot", shape, (torch.float32,))
    _workspace(workspace)
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    _on_gpu(cache, ("q_rot", q_rot), ("out_rot", out_rot), ("workspace", workspace))
    _check(load_library().tq_decode_attention_variant(
        cache.desc, p, _ptr(q_rot), int(q_rot.shape[1]), float(scale), _ptr(out_rot), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), int(variant), _stream(stream)))


def tq_decode_attention_fused(cache: Cache, q, scale, out, workspace, seq_lens_host=None, stream=None):
    """out fp16 [B, Hq, 128] = decode attention of q [B, Hq, 128] (fp16 or fp32, unrotated), with the
    q rotation and the output's inverse rotation done inside the decode and merge kernels."""
    import torch
    shape = _q_shape(cache, q)
    if len(shape) != 3:
        raise ValueError("q must be [B, Hq, 128]")
    _tensor(q, "q", shape, (torch.float16, torch.float32))
    _tensor(out, "out", shape, (torch.float16,))
    _workspace(workspace)
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    _on_gpu(cache, ("q", q), ("out", out), ("workspace", workspace))
    _check(load_library().tq_decode_attention_fused(
        cache.desc, p, _ptr(q), int(q.dtype == torch.float32), int(q.shape[1]), float(scale), _ptr(out),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def tq_decode_chunk_fused(cache: Cache, q, scale, out, workspace, seq_lens_host=None, stream=None):
    """out fp16 [B, Hq, Tq, 128] = causal decode attention of a chunk of Tq query positions
    q [B, Hq, Tq, 128] (fp16 or fp32, unrotated) over each sequence's visible tokens, the
    chunk's own Tq tokens last.  Workspace: tq_decode_workspace_size(cache, Hq * Tq)."""
    import torch
    shape = _q_shape(cache, q)
    if len(shape) != 4:
        raise ValueError("q must be [B, Hq, Tq, 128]")
    _tensor(q, "q", shape, (torch.float16, torch.float32))
    _tensor(out, "out", shape, (torch.float16,))
    _workspace(workspace)
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    _on_gpu(cache, ("q", q), ("out", out), ("workspace", workspace))
    _check(load_library().tq_decode_chunk_fused(
        cache.desc, p, _ptr(q), int(q.dtype == torch.float32), int(q.shape[1]), int(q.shape[2]), float(scale),
        _ptr(out), _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def tq_decode_step(cache: Cache, k_new, v_new, q, scale, out, workspace, seq_lens_host=None, stream=None):
    """Append one token (k_new, v_new fp16 [B, Hkv, 1, 128]) to every sequence and attend q
    [B, Hq, 128] over all visible tokens including it; out fp16 [B, Hq, 128].  The workspace is
    sized with the lengths before the append."""
    import torch
    kv_shape = (cache.batch, cache.num_kv_heads, 1, 128)
    _tensor(k_new, "k_new", kv_shape, (torch.float16,))
    _tensor(v_new, "v_new", kv_shape, (torch.float16,))
    shape = _q_shape(cache, q)
    if len(shape) != 3:
        raise ValueError("q must be [B, Hq, 128]")
    _tensor(q, "q", shape, (torch.float16, torch.float32))
    _tensor(out, "out", shape, (torch.float16,))
    _workspace(workspace)
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    _on_gpu(cache, ("k_new", k_new), ("v_new", v_new), ("q", q), ("out", out), ("workspace", workspace))
    _check(load_library().tq_decode_step(
        cache.desc, p, _ptr(k_new), _ptr(v_new), _ptr(q), int(q.dtype == torch.float32), int(q.shape[1]),
        float(scale), _ptr(out), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _stream(stream)))
    cache.lengths = arr + 1


def tq_decode_step_noalloc(cache: Cache, k_new, v_new, q, scale, out, seq_lens_host=None, stream=None):
    """tq_decode_step without a workspace, for callers that cannot allocate: the split partials
    live in the library's own per-GPU array (NOALLOC_SCRATCH_BYTES); calls that overlap on one
    GPU race on it."""
    import torch
    kv_shape = (cache.batch, cache.num_kv_heads, 1, 128)
    _tensor(k_new, "k_new", kv_shape, (torch.float16,))
    _tensor(v_new, "v_new", kv_shape, (torch.float16,))
    shape = _q_shape(cache, q)
    if len(shape) != 3:
        raise ValueError("q must be [B, Hq, 128]")
    _tensor(q, "q", shape, (torch.float16, torch.float32))
    _tensor(out, "out", shape, (torch.float16,))
    arr, p = _host_i32(cache.lengths if seq_lens_host is None else seq_lens_host, cache.batch)
    _on_gpu(cache, ("k_new", k_new), ("v_new", v_new), ("q", q), ("out", out))
    _check(load_library().tq_decode_step_noalloc(
        cache.desc, p, _ptr(k_new), _ptr(v_new), _ptr(q), int(q.dtype == torch.float32), int(q.shape[1]),
        float(scale), _ptr(out), _stream(stream)))
    cache.lengths = arr + 1


def tq_inverse_rotate_out(cache: Cache, out_rot, out, stream=None):
    """out_rot fp32 [B, Hq, 128] -> out fp16 [B, Hq, 128] in the original basis."""
    import torch
    shape = _q_shape(cache, out_rot, "out_rot")
    if len(shape) != 3:
        raise ValueError("out_rot must be [B, Hq, 128]")
    _tensor(out_rot, "out_rot", shape, (torch.float32,))
    _tensor(out, "out", shape, (torch.float16,))
    _on_gpu(cache, ("out_rot", out_rot), ("out", out))
    _check(load_library().tq_inverse_rotate_out(cache.desc, _ptr(out_rot), int(out_rot.shape[1]), _ptr(out),
                                                _stream(stream)))


def tq_stream_read(src, sums, stream=None):
    """Measurement aid: stream-read every byte of the contiguous device tensor `src`; work
    group i writes the XOR of the 32-bit words it read to sums[i] (device uint32/int32 tensor,
    one entry per work group)."""
    import torch
    if not isinstance(src, torch.Tensor) or not src.is_contiguous() or not src.is_cuda:
        raise ValueError("src must be a contiguous device tensor")
    if not isinstance(sums, torch.Tensor) or sums.dtype not in (torch.int32, torch.uint32) or sums.dim() != 1 \
            or not sums.is_contiguous() or sums.device != src.device:
        raise ValueError("sums must be a contiguous 1-D int32 tensor on src's device")
    _check(load_library().tq_stream_read(_ptr(src), int(src.numel() * src.element_size()), _ptr(sums),
                                         int(sums.numel()), _stream(stream)))
