"""Writes tests/golden/tiny_oracle_digest.json from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
The digest pins the oracle's results on the tiny workload (W 256x256 fp32
N(0,0.02) seed 0) so that any later change to the oracle's arithmetic shows up
as a test failure and has to be justified.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_digests():
    w = synth.tiny()["W"].numpy()
    out = {}
    for dq in (False, True):
        q = O.quantize(w, double_quant_on=dq)
        d = {"packed": digest(q["packed"]), "absmax": digest(q["absmax"]),
             "w_hat_bf16": digest(O.dequantize(q))}
        if dq:
            d.update(absmax_q=digest(q["absmax_q"]), scale=digest(q["scale"]),
                     mean_hex=f"{int(np.float32(q['mean']).view(np.uint32)):08x}")
        out["dq" if dq else "nodq"] = d
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_digest.json")
    with open(path, "w") as f:
        json.dump({"workload": "tiny: W 256x256 fp32 N(0,0.02) seed 0, blocksize 64",
                   "written_by": "tests/golden/make_golden.py (oracle only)",
                   "digests": tiny_digests()}, f, indent=1)
    print("wrote", path)
