"""Write the frozen codebook table used by both the oracle and the library.

Run:  python -m oracle.freeze_tables
Writes quantized_kv_cache_decode_amd/tables/codebooks.json from oracle code
only: the Lloyd-Max levels for N(0,1) (float64), their fp16 values after
scaling by 1/sqrt(128) (the codebook itself), the decision thresholds
(midpoints of adjacent fp16 entries) and the MSE of both.
"""
import json
import math
import os

import numpy as np

from .lloyd_max import decision_boundaries, frozen_codebook, lloyd_max_normal, mse_normal

OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "quantized_kv_cache_decode_amd", "tables", "codebooks.json")


def table() -> dict:
    out = {"head_dim": 128, "source": "Lloyd-Max for N(0,1), scaled by 1/sqrt(128), rounded to fp16 (RNE)"}
    for name, bits in (("turbo3", 3), ("turbo4", 4)):
        c64, _, iters = lloyd_max_normal(2 ** bits)
        c16 = frozen_codebook(bits)
        beta = decision_boundaries(c16)
        out[name] = {
            "levels": 2 ** bits,
            "lloyd_max_unit_variance": [float(v) for v in c64],
            "lloyd_max_iterations": int(iters),
            "mse_unit_variance": mse_normal(c64),
            "codebook_fp16_hex": ["0x%04x" % int(v) for v in c16.view(np.uint16)],
            "codebook_fp16_value": [float(v) for v in c16.astype(np.float64)],
            "mse_unit_variance_after_fp16": mse_normal(c16.astype(np.float64) * math.sqrt(128)),
            "thresholds": [float(v) for v in beta],
        }
    return out


def main():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    with open(OUT, "w") as f:
        json.dump(table(), f, indent=1)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
