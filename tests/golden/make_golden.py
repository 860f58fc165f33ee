"""Writes the oracle's full-size GroupNorm statistics for each workload.

    python tests/golden/make_golden.py [workload ...]

Calls only `oracle` (fp64 conv, slab by slab) and the seeded input module
`synth`.  For each workload it stores, per (n, group), the two-pass mean and
biased variance of the conv output y, plus rms(y) and rms(z) over the whole
tensor (gamma = 1, beta = 0).  The full-size GPU tests compare sampled y and z
against the oracle using these statistics, so the oracle never has to run a
full-size conv during a GPU test.  Floats are stored exactly (float.hex).
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402


def golden(name: str, slab: int = 8) -> dict:
    wl = synth.workload(name)
    t0 = time.time()
    x = synth.make_input(wl)
    w = oracle.widen(synth.make_weight(wl), wl.dtype)
    N, G, C = wl.batch, wl.groups, wl.cout
    gs = C // G
    y = np.empty((N, *wl.spatial, C), dtype=np.float64)
    for s0, ys in oracle.conv_same_slabbed(x, wl.dtype, w, None, slab=slab):
        y[:, s0:s0 + ys.shape[1]] = ys
        print(f"  {name}: conv rows {s0 + ys.shape[1]}/{wl.spatial[0]}  {time.time() - t0:.0f}s", flush=True)
    del x
    # two-pass moments per (n, g), accumulated over slabs of the outermost axis
    count = gs * int(np.prod(wl.spatial))
    s1 = np.zeros((N, G))
    sq = 0.0
    for s0 in range(0, wl.spatial[0], slab):
        part = y[:, s0:s0 + slab].reshape(N, -1, G, gs)
        s1 += part.sum(axis=(1, 3))
        sq += float((part * part).sum())
    mean = s1 / count
    s2 = np.zeros((N, G))
    for s0 in range(0, wl.spatial[0], slab):
        part = y[:, s0:s0 + slab].reshape(N, -1, G, gs)
        s2 += ((part - mean[:, None, :, None]) ** 2).sum(axis=(1, 3))
    var = s2 / count
    rms_y = float(np.sqrt(sq / y.size))
    rms_z = float(np.sqrt(np.mean(var / (var + wl.eps))))
    return {
        "workload": name,
        "source": "oracle.conv_same_slabbed (fp64) + two-pass GroupNorm moments",
        "groups": G, "eps": wl.eps, "count_per_group": count,
        "shards": [list(s) for s in wl.shards],
        "mean": [[v.hex() for v in row] for row in mean.tolist()],
        "var": [[v.hex() for v in row] for row in var.tolist()],
        "rms_y": rms_y.hex(), "rms_z": rms_z.hex(),
        "mean_approx": mean.tolist(), "var_approx": var.tolist(),
        "rms_y_approx": rms_y, "rms_z_approx": rms_z,
        "seconds": round(time.time() - t0, 1),
    }


def load(name: str) -> dict:
    with open(os.path.join(HERE, f"{name}.json")) as f:
        g = json.load(f)
    g["mean"] = np.array([[float.fromhex(v) for v in row] for row in g["mean"]])
    g["var"] = np.array([[float.fromhex(v) for v in row] for row in g["var"]])
    g["rms_y"] = float.fromhex(g["rms_y"])
    g["rms_z"] = float.fromhex(g["rms_z"])
    return g


def main(names):
    for name in names:
        g = golden(name)
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(g, f, indent=1)
        print(f"wrote {name}.json ({g['seconds']} s)", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.WORKLOADS))
