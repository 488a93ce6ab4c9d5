"""Write tests/golden/tiny_layer.json: the oracle's output on the tiny seeded
layer (E=8, top-2, H=128, I=64, B=1).  Calls only the oracle and the seeded
input generator.  A regression fixture: it pins the generator's bits (by
digest) and the oracle's values against accidental change.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_decode_gate_amd import inputs as gen  # noqa: E402


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(a.tobytes())
    return h.hexdigest()


def main():
    cfg = gen.CONFIGS["tiny"]
    spec = cfg["spec"]
    L = gen.make_layer(spec)
    t = gen.make_tokens(spec, 1)
    y, act = oracle.moe_decode(t.x, t.ids, t.w, L.wgu, L.sgu, L.wd, L.sd)
    out = {
        "what": "oracle output on the tiny seeded MoE decode layer (E=8, top-2, H=128, I=64, B=1)",
        "made_by": "tests/golden/make_golden.py (oracle + seeded generator only)",
        "weights_sha256": digest(L.wgu, L.sgu, L.wd, L.sd),
        "tokens_sha256": digest(t.x, t.ids, t.w),
        "ids": t.ids.tolist(),
        "w": [float(v) for v in t.w.ravel()],
        "act_bits": act.ravel().tolist(),
        "y": [float(v).hex() for v in y.ravel()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
