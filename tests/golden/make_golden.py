"""Write tests/golden/tiny_expected.json from the CPU oracle.

The stored values are the tiny workload's seeded bf16 gradients (bit
patterns) and the oracle's fp32 reduce-scatter block for every rank (bit
patterns).  Only the oracle and the seeded input generator are used; nothing
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
    rs = [orc.rs(w.shapes, w.world, R, bits).view(np.uint32).tolist() for R in range(w.world)]
    doc = {
        "_about": "tiny workload: 3 params [5,7],[16],[33,4], 4 ranks, bf16 ~N(0,1), "
                  "rank r seeded 0+r on a CPU generator; rs[R] = oracle fp32 block bits",
        "shapes": [list(s) for s in w.shapes],
        "world": w.world,
        "grads": [[b.tolist() for b in rank] for rank in bits],
        "rs": rs,
    }
    with open(os.path.join(HERE, "tiny_expected.json"), "w") as f:
        json.dump(doc, f)
        f.write("\n")


if __name__ == "__main__":
    main()
