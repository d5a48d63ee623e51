"""Write tests/golden/tiny_expected.json from the CPU oracle.

The stored values are the tiny workload's seeded bf16 gradients (bit
patterns) and, for every rank, the oracle's fp32 reduce-scatter block (sum
and mean), the sum rounded to bf16, and the rank-major pack of that rank's
gradients (all as bit patterns).  Only the oracle and the seeded input generator are used; nothing
here touches the HIP library.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.WORKLOADS["tiny"]
    grads = workloads.all_grads(w)
    bits = [[workloads.bf16_bits(t).reshape(-1) for t in rank] for rank in grads]
    orc = oracle.default()
    rs = [orc.rs(w.shapes, w.world, R, bits) for R in range(w.world)]
    mean = [orc.rs(w.shapes, w.world, R, bits, avg=True) for R in range(w.world)]
    doc = {
        "_about": "tiny workload: 3 params [5,7],[16],[33,4], 4 ranks, bf16 ~N(0,1), "
                  "rank r seeded 0+r on a CPU generator; rs[R] = oracle fp32 block bits; "
                  "rs_mean[R] = the mean's block; rs_bf16[R] = the sum's block rounded to "
                  "bf16 (bits); pack[r] = rank r's gradients packed rank-major (bits)",
        "shapes": [list(s) for s in w.shapes],
        "world": w.world,
        "grads": [[b.tolist() for b in rank] for rank in bits],
        "rs": [b.view(np.uint32).tolist() for b in rs],
        "rs_mean": [b.view(np.uint32).tolist() for b in mean],
        "rs_bf16": [orc.round_bf16(b).tolist() for b in rs],
        "pack": [orc.pack(w.shapes, w.world, bits[r]).tolist() for r in range(w.world)],
    }
    with open(os.path.join(HERE, "tiny_expected.json"), "w") as f:
        json.dump(doc, f)
        f.write("\n")


if __name__ == "__main__":
    main()
