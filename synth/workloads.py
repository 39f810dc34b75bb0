"""The five decode workloads, as shapes and value distributions.

Head dim is 128 everywhere.  Formats: "turbo3" (3-bit codes + fp16 norm per
128-group), "turbo4" (4-bit codes + fp16 norm), "f16" (raw half-precision K, the
asymmetric Turbo4Asym mode of mlxcel PR #369, section "Change").
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    k_format: str          # "turbo3" | "turbo4" | "f16"
    v_format: str          # "turbo3" | "turbo4"
    context: Optional[int]  # fixed visible context per sequence (None: ragged)
    ragged_range: Optional[Tuple[int, int]] = None  # inclusive [lo, hi] when ragged
    q_dtype: str = "fp16"  # "fp16" | "fp32"
    k_outlier_channels: int = 0   # channels per KV head scaled by k_outlier_scale
    k_outlier_scale: float = 1.0
    k_heavy_tail_frac: float = 0.0  # fraction of K entries replaced by Student-t draws
    k_heavy_tail_nu: float = 3.0
    appends_per_step: int = 1     # new tokens written by each decode step
    note: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def symmetric(self) -> bool:
        return self.k_format != "f16"


WORKLOADS = {
    0: Workload(
        0, "tiny-turbo3", batch=1, num_q_heads=4, num_kv_heads=2,
        k_format="turbo3", v_format="turbo3", context=256, q_dtype="fp32",
        note="GQA 2:1, context 256, K,V ~N(0,1) fp16, q fp32 ~N(0,1)"),
    1: Workload(
        1, "qwen2.5-7b-layer-turbo3-8k", batch=1, num_q_heads=28, num_kv_heads=4,
        k_format="turbo3", v_format="turbo3", context=8192,
        k_outlier_channels=4, k_outlier_scale=8.0,
        note="K ~N(0,1) with 4 channels per KV head scaled x8, V ~N(0,1), q fp16"),
    2: Workload(
        2, "turbo4asym-16k", batch=1, num_q_heads=28, num_kv_heads=4,
        k_format="f16", v_format="turbo4", context=16384,
        note="fp16 K kept raw, V 4-bit; attention in the rotated V basis"),
    3: Workload(
        3, "llama3-8b-turbo4-b32-32k", batch=32, num_q_heads=32, num_kv_heads=8,
        k_format="turbo4", v_format="turbo4", context=32768,
        note="every sequence at context 32768 after the step's one-token append"),
    4: Workload(
        4, "ragged-turbo3-b16", batch=16, num_q_heads=64, num_kv_heads=8,
        k_format="turbo3", v_format="turbo3", context=None, ragged_range=(1024, 131072),
        k_heavy_tail_frac=0.02, k_heavy_tail_nu=3.0,
        note="per-sequence context ~U[1024,131072]; 2% of K entries Student-t(3)"),
}


def get_workload(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS.values():
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)
