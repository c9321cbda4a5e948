"""Writes division_cases.json: rows whose codes depend on dividing by the
scale with one correctly rounded fp32 division (rather than multiplying by a
rounded reciprocal), and on ties going to even.

Candidates are found by a float32 search; every stored expected value is
computed by the exact-rational brute force in oracle/brute.py only.
Run from the repository root: python tests/golden/make_division_cases.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import brute  # noqa: E402


def candidates(limit=8):
    allh = np.arange(0x3C00, 0x5BF0, dtype=np.uint16).view(np.float16)   # fp16 in [1, 254)
    out = []
    for a in allh[::37]:
        s = np.float32(np.float32(a) / np.float32(127))
        inv = np.float32(np.float32(1) / s)
        xs = allh[allh <= a].astype(np.float32)
        bad = np.nonzero(np.rint(xs / s) != np.rint(xs * inv))[0]
        if len(bad):
            out.append((float(a), float(xs[bad[0]])))
        if len(out) >= limit:
            break
    return out


def main():
    cases = []
    for a, x in candidates():
        row = [a, x, -x]
        q, s = brute.quantize_row(row, 0, 127)
        cases.append({"x": row, "q": q, "s": float(s[0])})
    doc = {
        "citation": "Cider README, section 量化 (Quantization) table: symmetric INT8 per-token activations; section 说明 (Notes): min-max scales. The fp32 division and ties-to-even are this repository's readings.",
        "derivation": "Expected codes and scales computed by oracle/brute.py (exact rationals with explicit IEEE rounding) from rows [a, x, -x]; each x is one where x*fl(1/s) and fl(x/s) round to different integers.",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "division_cases.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1, ensure_ascii=False)
        f.write("\n")


if __name__ == "__main__":
    main()
