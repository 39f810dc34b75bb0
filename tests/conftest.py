import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TABLE = os.path.join(ROOT, "quantized_kv_cache_decode_amd", "tables", "codebooks.json")


def load_codebook(fmt: str) -> np.ndarray:
    with open(TABLE) as f:
        t = json.load(f)
    return np.array([int(h, 16) for h in t[fmt]["codebook_fp16_hex"]], dtype=np.uint16).view(np.float16)


@pytest.fixture(scope="session")
def codebooks():
    return {"turbo3": load_codebook("turbo3"), "turbo4": load_codebook("turbo4")}
