"""Write the stored regression values for the 64x256 Linear (oracle only).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import hlwq_ref as ref  # noqa: E402


def main():
    w = synth.weight("linear_64x256", "W")
    packed, n16 = ref.quantize_c(w, 5)
    out = ref.dequantize_c(packed, n16, 256, 5)
    rec = {
        "source": "oracle.hlwq_ref Tier C on synth.weight('linear_64x256', 'W') (seed 0), Q5",
        "packed_hex": bytes(packed.ravel()).hex(),
        "norms_hex": bytes(n16.view(np.uint16).astype("<u2").ravel().view(np.uint8)).hex(),
        "dequant_hex": bytes(out.astype("<u2").ravel().view(np.uint8)).hex(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "linear_64x256_q5.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
