"""Write tests/golden/tiny_forward.json from the oracle alone.

The pages print no worked numeric example, so this fixture only freezes the
oracle's own results on the seeded tiny workload (256x512 fp32 A, 512x512 W,
q = 0.99): a change to the oracle's arithmetic shows up as a diff here and
must name the passage that justifies it. Run from the repository root:

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as wl  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    L = wl.make_layer("tiny", seed=0)
    Y, ops = O.forward(L.A.f32, L.W.f32, L.q)
    out = {
        "workload": "tiny 256x512x512 fp32, q=0.99, seed 0",
        "k": ops.k,
        "tau_bits": int(np.float32(ops.tau).view(np.uint32)),
        "nnz": ops.delta.nnz,
        "coo_row_sha256": digest(ops.delta.row.astype(np.int32)),
        "coo_col_sha256": digest(ops.delta.col.astype(np.int32)),
        "coo_val32_sha256": digest(ops.delta.val32.astype(np.float32)),
        "row_ptr_sha256": digest(ops.delta.row_ptr.astype(np.int32)),
        "Aq_sha256": digest(ops.Aq),
        "sA_sha256": digest(ops.sA.astype(np.float32)),
        "Wq_sha256": digest(ops.Wq),
        "sW_sha256": digest(ops.sW.astype(np.float32)),
        "Y_fro": float(np.linalg.norm(Y)),
        "Y_00_03": [float(v) for v in Y[0, :4]],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_forward.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
