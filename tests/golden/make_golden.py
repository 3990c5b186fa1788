"""Write the stored oracle values of the toy workload (7-node binary tree, fp32).

The pages print no output values for any input, so these are not the pages'
numbers: they are the fp64 oracle's outputs on the seeded toy inputs, written
here so that a later change to the oracle's arithmetic shows up as a diff.
This script calls only ``oracle/`` and the input generator.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oracle as O  # noqa: E402
from speculative_tree_verification_amd import workloads as W  # noqa: E402


def main():
    inp = W.make_inputs(0)
    y, st = O.verify_full(inp, W.F32)
    h, st2 = O.commit_full(inp, W.F32)
    depth, anc, st3 = O.tree_info(inp["parent"])
    doc = {
        "what": "fp64 oracle outputs for the toy workload (batch 1, 1 head, P 16, N 8, "
                "7-node complete binary tree, accepted path 0->1->4), seeded inputs "
                "make_inputs(0)",
        "source": "oracle/oracle.c via tests/golden/make_golden.py",
        "parent": inp["parent"].tolist(),
        "accepted": inp["accepted"].tolist(),
        "status_verify": st.tolist(),
        "status_commit": st2.tolist(),
        "depth": depth.tolist(),
        "anc_word0": [int(v) for v in anc[0, :, 0]],
        "y": y.tolist(),
        "h_commit": h.tolist(),
    }
    with open(os.path.join(HERE, "toy7_oracle.json"), "w") as f:
        json.dump(doc, f, indent=None, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
