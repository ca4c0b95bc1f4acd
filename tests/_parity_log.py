"""Observed parity figures of the GPU tests (no method arithmetic here).

Every GPU parity test records what it measured against the oracle (largest
error relative to max|oracle|, BF16 ulps, cosine, or the number of
bit-exact arrays it compared). At the end of the session conftest prints a
compact summary, so that the tail of a pytest run carries the numbers, and,
when $NVFP4_PARITY_JSON names a file, writes them all there as JSON.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

RECORDS: list = []


def record(test: str, **metrics):
    """Keep the figures one test observed (floats, ints, bools or strings)."""
    clean = {}
    for k, v in metrics.items():
        if isinstance(v, (np.floating, np.integer)):
            v = v.item()
        if isinstance(v, float) and not math.isfinite(v):
            v = str(v)
        clean[k] = v
    RECORDS.append({"test": test, **clean})


def bf16_ulp(a):
    """Spacing of BF16 numbers at |a| (float64 array): 2^(e - 7) for |a| in
    [2^e, 2^(e+1)), the subnormal spacing 2^-133 at the bottom."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.maximum(np.exp2(e - 7), 2.0 ** -133)


def ulp_error(got, ref, floor_frac=2.0 ** -10):
    """Largest |got - ref| in BF16 ulps of max(|ref|, floor_frac * max|ref|):
    elements far below the largest one are measured in the ulps of that
    floor, since their float32 sums cancel and carry absolute, not relative,
    rounding differences."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    top = float(np.abs(ref).max())
    if top == 0.0:
        return 0.0 if not np.any(got) else float("inf")
    u = bf16_ulp(np.maximum(np.abs(ref), floor_frac * top))
    return float((np.abs(got - ref) / u).max())


def summary_lines():
    if not RECORDS:
        return []
    lines = [f"parity figures of {len(RECORDS)} GPU checks against the oracle:"]
    worst = {}
    for r in RECORDS:
        for k, v in r.items():
            if k in ("test", "S") or not isinstance(v, (int, float)) or isinstance(v, bool):
                continue
            better_low = not k.startswith("cos")
            cur = worst.get(k)
            if cur is None or (v > cur[0] if better_low else v < cur[0]):
                worst[k] = (v, r["test"])
    for k in sorted(worst):
        v, t = worst[k]
        tag = "min" if k.startswith("cos") else "max"
        lines.append(f"  {tag} {k} = {v:.4g}  ({t})")
    full = [r for r in RECORDS if r["test"].startswith("full:")]
    for r in full:
        parts = [f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}" for k, v in r.items() if k != "test"]
        lines.append(f"  {r['test']}: " + ", ".join(parts))
    return lines


def write_json():
    path = os.environ.get("NVFP4_PARITY_JSON")
    if not RECORDS or not path:
        return None
    with open(path, "w") as f:
        json.dump(RECORDS, f, indent=1)
    return path
