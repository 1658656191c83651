"""Writes dropout_gap_draws.json: for two dropout rates, one Philox4x32-10
draw that lies between floor(p * 2^32) (the rate as the binary64 number the
caller passes) and floor(f32(p) * 2^32) (the same rate first rounded to
binary32).  The two readings of the rate keep or drop that (row, key) pair
differently, so a GPU test on it shows which threshold the library applies.

Only oracle/ computes the draws and the threshold; numpy gives the binary32
rounding of the rate.  Run from the repository root:

    python tests/golden/make_dropout_gap_draws.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.dropout import keep_threshold, philox4x32_10  # noqa: E402


def find(p, n, seed, batch=1 << 14):
    """First (offset, row, key) of a square n x n single-head problem whose
    draw lies in the gap between the two thresholds of rate p."""
    t64 = keep_threshold(p)
    t32 = keep_threshold(float(np.float32(p)))
    lo, hi = min(t64, t32), max(t64, t32)
    i = np.arange(n, dtype=np.uint64)[:, None, None]
    g = np.arange((n + 3) // 4, dtype=np.uint64)[None, :, None]
    for start in range(0, 1 << 32, batch):
        off = np.arange(start, start + batch, dtype=np.uint64)[None, None, :]
        words = philox4x32_10((g, i, np.uint64(0), off), (seed & 0xFFFFFFFF, seed >> 32))
        for w, u in enumerate(words):
            hit = np.argwhere((u >= lo) & (u < hi))
            for row, grp, k in hit:
                key = 4 * int(grp) + w
                if key < n:
                    return {"p": p, "n": n, "seed": seed, "offset": start + int(k), "row": int(row),
                            "key": key, "draw": int(u[row, grp, k]), "threshold": t64,
                            "threshold_if_rate_were_f32": t32, "kept": bool(int(u[row, grp, k]) >= t64)}
    raise RuntimeError("no draw found")


def main():
    cases = [find(0.3, 8, 20241203), find(0.9, 64, 20241203)]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dropout_gap_draws.json")
    with open(path, "w") as f:
        json.dump({"source": "tests/golden/make_dropout_gap_draws.py (oracle.dropout only)",
                   "cases": cases}, f, indent=1)
        f.write("\n")
    print(json.dumps(cases))


if __name__ == "__main__":
    main()
