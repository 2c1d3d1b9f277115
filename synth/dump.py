"""Write a synthetic gradient set to one binary file for the native driver.

    python -m synth.dump NAME OUT

Layout (little-endian): 8-byte magic b"GCLIPSET", u32 version (1), u32 dtype
(0 f32, 1 f16, 2 bf16), u32 n_tensors, u32 error_if_nonfinite, f64 max_norm,
f64 avg_factor, i64 numel[n_tensors], then every tensor's raw storage in list
order.  Only draws and lays out numbers; no clipping arithmetic.
"""
import struct
import sys

import numpy as np

from . import gradsets as gs

CODES = {"f32": 0, "f16": 1, "bf16": 2}


def dump(g: gs.GradSet, path: str) -> None:
    with open(path, "wb") as f:
        f.write(b"GCLIPSET")
        f.write(struct.pack("<IIII", 1, CODES[g.dtype], len(g.arrays), int(g.error_if_nonfinite)))
        f.write(struct.pack("<dd", float(g.max_norm), float(g.avg_factor)))
        f.write(np.array([a.size for a in g.arrays], dtype=np.int64).tobytes())
        for a in g.arrays:
            f.write(np.ascontiguousarray(a).tobytes())


def main(argv):
    if len(argv) != 3:
        print(__doc__)
        return 2
    dump(gs.make(argv[1]), argv[2])
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
