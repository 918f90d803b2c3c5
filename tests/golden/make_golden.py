"""Write tests/golden/tiny_oracle_digests.json from the oracle alone.

The pages print no numeric worked example for this layer, so the stored
fixtures here are digests of the oracle's own outputs on the tiny seeded
workload (x [64,256] with 4 outlier columns, W [256,256], dY [64,256]).  They
guard the oracle against unintended changes; a deliberate change of its
arithmetic regenerates them and names the passage that justifies it.
Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def digests():
    t = wl.tiny(0)
    qw, sw, _ = oracle.rotate_quantize(t["w"])
    fwd = oracle.linear_fwd(t["x"], qw, sw)
    b8 = oracle.bwd_dx_int8(t["dy"], qw, sw)
    b16 = oracle.bwd_dx_bf16(t["dy"], qw, sw)
    arrs = dict(qw=qw, sw=sw, qx=fwd["qx"], sx=fwd["sx"], acc=fwd["acc"], y=fwd["y"],
                qg=b8["qg"], sg=b8["sg"], acc2=b8["acc2"], dx_int8=b8["dx"],
                what=b16["what"], dx_bf16=b16["dx"])
    return {k: hashlib.sha256(v.tobytes()).hexdigest() for k, v in arrs.items()}


if __name__ == "__main__":
    out = os.path.join(HERE, "tiny_oracle_digests.json")
    with open(out, "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
    print(out)
