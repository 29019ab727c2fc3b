"""Write tests/golden/small_pack_oracle.json: the fp64 oracle's outputs on a small pack.

Calls only ``oracle/`` (and numpy for the seeded inputs). The fixture is a regression
pin: a later change to the oracle's arithmetic that moves these values must name the
passage of the Zellige page that justifies it. The pack mixes a whole sequence, a head
subset (Ulysses shard, Table II) and a three-part ring group (KV split, §II-B).

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

PACK = dict(seq_q=[5, 3, 4], seq_kv=[5, 3, 6], heads=[2, 3, 2], d=4, scale=0.55,
            segments=[[0, 0, 2, 0, 5, 0, 5, -1], [1, 1, 3, 0, 3, 0, 3, -1],
                      [2, 0, 2, 0, 4, 0, 2, 0], [2, 0, 2, 0, 4, 2, 3, 1], [2, 0, 2, 0, 4, 3, 6, 2]])


def inputs():
    r = np.random.default_rng(2024)
    lay = oracle.PackLayout(PACK["seq_q"], PACK["seq_kv"], PACK["heads"])
    d = PACK["d"]
    # values on a 1/8 grid so that they are exact in every float format
    g = lambda n: np.round(r.normal(size=(n, d)) * 8) / 8
    return g(lay.q_rows), g(lay.kv_rows), g(lay.kv_rows), g(lay.q_rows)


def compute():
    q, k, v, do = inputs()
    args = (PACK["seq_q"], PACK["seq_kv"], PACK["heads"], [tuple(s) for s in PACK["segments"]], PACK["d"], PACK["scale"])
    f = oracle.pack_forward(*args, q, k, v)
    b = oracle.pack_backward(*args, q, k, v, f["o"], f["lse"], do)
    tolist = lambda a: [None if np.isnan(x) else float(x) for x in np.asarray(a).ravel()]
    return {"o": tolist(f["o"]), "lse": tolist(f["lse"]), "dq": tolist(b["dq"]), "dk": tolist(b["dk"]),
            "dv": tolist(b["dv"])}


if __name__ == "__main__":
    out = {"source": "tests/golden/make_golden.py (oracle only)", "pack": PACK, "values": compute()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "small_pack_oracle.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=0)
    print("wrote", path)
