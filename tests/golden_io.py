"""Text fixtures under tests/golden/: named arrays, one value per token.

A fixture file holds comment lines (starting with '#') and arrays, each
introduced by a line 'array <name> <dtype> <rows> <cols>' and followed by its
values in row-major order, whitespace-separated.  float32 and float64 values
are written as C99 hex floats (exact), integers in decimal.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def write(path, header_lines, arrays):
    with open(path, "w") as f:
        for line in header_lines:
            f.write(f"# {line}\n" if line else "#\n")
        for name, a in arrays:
            a = np.atleast_2d(np.asarray(a))
            if a.dtype in (np.float32, np.float64):
                vals = [float(v).hex() for v in a.ravel()]
            else:
                vals = [str(int(v)) for v in a.ravel()]
            f.write(f"array {name} {a.dtype.name} {a.shape[0]} {a.shape[1]}\n")
            for i in range(0, len(vals), 16):
                f.write(" ".join(vals[i:i + 16]) + "\n")


def read(name):
    """{array name: ndarray} of tests/golden/<name>."""
    out, cur, want, vals = {}, None, 0, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if line.startswith("array "):
                _, nm, dt, r, c = line.split()
                cur, want, vals = (nm, np.dtype(dt), int(r), int(c)), int(r) * int(c), []
                continue
            vals.extend(line.split())
            if len(vals) == want:
                nm, dt, r, c = cur
                if dt in (np.float32, np.float64):
                    a = np.array([float.fromhex(v) for v in vals], dtype=dt)
                else:
                    a = np.array([int(v) for v in vals], dtype=dt)
                out[nm] = a.reshape(r, c)
    return out
