"""Reader for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

from synth import to_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            fields[key] = vals
    out = {
        "dtype": fields["dtype"][0],
        "norm": {"none": 0, "rms": 1, "layer": 2}[fields["norm"][0]],
        "eps": float(fields["eps"][0]),
        "K": int(fields["K"][0]),
        "N": int(fields["N"][0]),
        "M": int(fields["M"][0]),
        "fmt": {"mxfp4": 0, "nvfp4": 1}[fields["fmt"][0]],
        "gscale": float(fields["gscale"][0]),
    }
    x = np.array([float(v) for v in fields["x"]], np.float32)
    out["x_f32"] = x
    out["x"] = to_bits(x, out["dtype"]).reshape(1, -1)
    for key in ("mask", "b_codes", "b_scales", "r_codes", "r_scales"):
        out[key] = np.array([int(v, 16) for v in fields[key]], np.uint8).reshape(1, -1)
    return out
