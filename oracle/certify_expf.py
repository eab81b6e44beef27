"""Certificate scan for the oracle's correctly rounded binary32 exp.

Scans every binary32 input (2^32 patterns, in parallel slices) with the oracle's
``oracle_crexpf_scan`` and writes ``tests/golden/expf_escalations.txt``: every
input whose double-precision exp lands within 2^-40 (relative) of a point halfway
between two binary32 numbers, with the binary32 result the oracle returns for it
(from its 113-bit evaluation) and how far that 113-bit value sits from the
midpoint. ``tests/test_oracle_expf.py`` re-derives each listed result from mpmath
at 200 bits with exact rational rounding.

Calls only the oracle. Usage: ``python -m oracle.certify_expf [--procs N]``.
"""

from __future__ import annotations

import argparse
import ctypes
import multiprocessing as mp
import pathlib
import time

import numpy as np

OUT = pathlib.Path(__file__).resolve().parent.parent / "tests" / "golden" / "expf_escalations.txt"
SLICES = 256
CAP = 1 << 16


def _scan(i: int):
    import oracle

    lib = oracle.load()
    count = (1 << 32) // SLICES
    first = i * count
    cand = np.zeros(CAP, dtype=np.uint32)
    gap = ctypes.c_double()
    n = lib.oracle_crexpf_scan(first, count, cand.ctypes.data, CAP, ctypes.byref(gap))
    if n > CAP:
        raise RuntimeError(f"slice {i}: {n} escalations exceed the buffer")
    out = []
    for u in cand[:n]:
        x = np.array([u], dtype=np.uint32).view(np.float32)[0]
        r = lib.oracle_crexpf(float(x))
        rb = int(np.array([r], dtype=np.float32).view(np.uint32)[0])
        out.append((int(u), rb))
    return i, out, (gap.value if n else None)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=8)
    args = ap.parse_args()
    import oracle

    oracle.build()
    t0 = time.time()
    rows, worst = [], None
    with mp.get_context("fork").Pool(args.procs) as pool:
        for i, out, g in pool.imap_unordered(_scan, range(SLICES)):
            rows.extend(out)
            if g is not None and (worst is None or g < worst):
                worst = g
    rows.sort()
    OUT.parent.mkdir(parents=True, exist_ok=True)
    with open(OUT, "w") as f:
        f.write("# Escalations of the oracle's correctly rounded binary32 exp over all 2^32 inputs.\n")
        f.write("# Written by oracle/certify_expf.py (calls only the oracle).\n")
        f.write("# Columns: input bits, binary32 result bits (hex).\n")
        f.write(f"# count {len(rows)}\n")
        f.write(f"# smallest log2 relative distance of a 113-bit value to its midpoint: {worst}\n")
        for u, r in rows:
            f.write(f"{u:08x} {r:08x}\n")
    print(f"{len(rows)} escalations, smallest log2 gap {worst}, {time.time() - t0:.1f} s")


if __name__ == "__main__":
    main()
