"""Reader for the hand-worked quantiser fixtures in tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_quant_case(name):
    cols = None
    nz = {}
    data = None
    scale = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tag, *rest = line.split()
            if tag == "cols":
                cols = int(rest[0])
            elif tag == "w":
                nz[int(rest[0])] = int(rest[1], 16)
            elif tag == "bytes":
                data = bytes(int(v, 16) for v in rest)
            elif tag == "scale":
                scale = int(rest[0], 16)
    bits = np.zeros(cols, dtype=np.uint32)
    for k, v in nz.items():
        bits[k] = v
    return bits.view(np.float32).reshape(1, cols), data, scale
