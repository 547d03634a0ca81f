"""Write the stored expected values under tests/golden/ from the oracle alone.

The HSTU Attention page prints no worked numeric example, so no stored value
here comes from the page.  Each fixture is the fp64 oracle's output for a seeded
synthetic input, written by this script (which calls only ``oracle`` and the
input generator) so that a later change to the oracle's arithmetic shows up as
a diff of a committed file.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from generative_recommender_attention_amd.workloads import make_workload, named_workload  # noqa: E402


def dump(path, payload):
    with open(path, "w") as f:
        json.dump(payload, f, indent=1)
        f.write("\n")


def main():
    oracle.build(force=False)
    wl = named_workload("tiny_b2_h1_d16_causal")
    o = oracle.fwd_workload(wl)
    dump(os.path.join(HERE, "tiny_b2_h1_d16_causal_fwd.json"), {
        "workload": wl.name,
        "source": "oracle (fp64), written by tests/golden/make_golden.py",
        "cu_seqlens": wl.cu_seqlens_q.tolist(),
        "alpha_f32": float(wl.alpha),
        "scaling_seqlen": wl.scaling_seqlen,
        "o": [float(x) for x in o.ravel()],
    })
    wl = make_workload("tiny_bwd_b3_h2_d16_causal", 40, [6, 0, 9], 2, 16, True, with_do=True)
    dq, dk, dv = oracle.bwd_workload(wl)
    dump(os.path.join(HERE, "tiny_bwd_b3_h2_d16_causal.json"), {
        "workload": wl.name,
        "source": "oracle (fp64), written by tests/golden/make_golden.py",
        "make_workload": {"seed": 40, "lengths": [6, 0, 9], "H": 2, "D": 16, "causal": True,
                          "with_do": True},
        "dq": [float(x) for x in dq.ravel()],
        "dk": [float(x) for x in dk.ravel()],
        "dv": [float(x) for x in dv.ravel()],
    })


if __name__ == "__main__":
    main()
