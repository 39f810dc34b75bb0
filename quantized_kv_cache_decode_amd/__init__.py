"""MI355X-native decode attention over a rotated-scalar-codec KV cache.

The compute path is libtqattn.so (hand-written HIP for gfx950, C ABI declared
in include/tqattn.h); `binding` wraps it with ctypes.
"""
from .binding import (  # noqa: F401
    Cache,
    TqError,
    codebook_bits,
    load_library,
    tq_decode_attention,
    tq_decode_attention_fused,
    tq_decode_chunk_fused,
    tq_decode_step,
    tq_decode_step_noalloc,
    tq_decode_workspace_size,
    tq_encode_append,
    tq_inverse_rotate_out,
    tq_rotate_q,
    tq_stream_read,
)
