"""Write div_adversarial.json: bf16 (amax, x) pairs where the E4M3 code of
fp32(x / s) differs from the code of fp32(x * fp32(1 / s)), s = fp32(amax/448).

Inputs only: the file stores bf16 bit patterns; the expected codes are
computed in the test by an independent brute-force quantizer.  Calls numpy
and oracle.e4m3 only.  Run from the repository root:
    python tests/golden/make_div_adversarial.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import e4m3  # noqa: E402


def main():
    rng = np.random.default_rng(5)
    xs_bits = np.arange(1, 0x7F80, dtype=np.uint32)
    xs = (xs_bits << 16).view(np.float32)
    found = []
    amaxes = rng.choice(np.arange(0x0001, 0x7F80, dtype=np.uint32), size=3000, replace=False)
    for ab in amaxes:
        amax = np.array([ab << 16], dtype=np.uint32).view(np.float32)[0]
        s = np.float32(amax / np.float32(448))
        sel = xs <= amax
        x = xs[sel]
        q_div = (x / s).astype(np.float32)
        q_rcp = (x * np.float32(np.float32(1) / s)).astype(np.float32)
        diff = e4m3.encode(q_div) != e4m3.encode(q_rcp)
        for xb in xs_bits[sel][diff][:3]:
            found.append([int(ab), int(xb)])
        if len(found) >= 240:
            break
    out = {
        "source": "constructed: bf16 pairs where true fp32 division and reciprocal-multiply give different E4M3 codes",
        "generator": "tests/golden/make_div_adversarial.py",
        "pairs_amax_bits_x_bits": found,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "div_adversarial.json")
    json.dump(out, open(path, "w"))
    print(len(found), "pairs")


if __name__ == "__main__":
    main()
