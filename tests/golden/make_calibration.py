"""Write tests/golden/calibration.json: per named workload, the planting
direction of every (layer, request) and the per-layer score bias.

Both come from the CPU oracle only: the direction is the oracle's
head-collapsed query, normalised; the bias puts the workload's target fraction
of the oracle's bias-free scores at or above zero (pooled over requests, on
the first ``calib_rows`` entries of each when the workload sets it).

Usage:  python tests/golden/make_calibration.py [workload ...]
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402

import lsa_inputs as gen  # noqa: E402
import lsa_fixtures as fx  # noqa: E402

OUT = os.path.join(HERE, "calibration.json")


def main(names):
    data = {"generator_version": gen.GENERATOR_VERSION, "workloads": {}}
    if os.path.exists(OUT):
        with open(OUT) as f:
            old = json.load(f)
        if old.get("generator_version") == gen.GENERATOR_VERSION:
            data = old
    for name in names:
        w = gen.WORKLOADS[name]
        t0 = time.time()
        c = fx.calibrate(w)
        data["workloads"][name] = {
            "u": [float(f"{v:.9g}") for v in c.u.ravel()],
            "bias": [float(v) for v in c.bias],
            "shape_u": [w.L, w.B, w.dI],
            "sel_frac": list(w.sel_frac),
        }
        print(f"{name}: bias={c.bias.tolist()} ({time.time() - t0:.1f}s)", flush=True)
    with open(OUT, "w") as f:
        json.dump(data, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or list(gen.WORKLOADS))
