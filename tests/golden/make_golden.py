"""Write tests/golden/tiny_chain.json from the CPU oracle (and the seeded inputs) only.

The vLLM pages on MXFP8 activations print no tensor values, so no fixture here
comes from them.  This file freezes the oracle's own output on the tiny chain
(M=4, 2 groups x 256 -> 128, wo_b 256 -> 256, seed 20260001) as SHA-256 digests
of every intermediate byte array plus a few float64 outputs, so that any later
change to the oracle's arithmetic shows up as a failing test and has to be
justified.  Run from the repository root: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth_inputs as si  # noqa: E402
from oracle import chain_ref as cr  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_chain_record() -> dict:
    inp = si.config_inputs("tiny")
    wa_q, wa_sf, wb_q, wb_sf = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
    r = cr.o_proj_chain(inp["x"], wa_q, wa_sf, wb_q, wb_sf)
    return {
        "config": "tiny: M=4, G=2, K=256, N=128, P=256, seed 20260001",
        "sha256": {
            "x_bf16": digest(inp["x"]), "wo_a_q": digest(wa_q), "wo_a_sf": digest(wa_sf),
            "wo_b_q": digest(wb_q), "wo_b_sf": digest(wb_sf), "x_q": digest(r.x_q), "x_sf": digest(r.x_sf),
            "z_bf16": digest(r.z_bf16), "z_q": digest(r.z_q), "z_sf": digest(r.z_sf),
            "out_bf16": digest(r.out_bf16),
        },
        "out64_row0_first8": [float(v) for v in r.out64[0, :8]],
        "z_sf_words_row0": [int(v) for v in r.z_sf[0]],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_chain.json")
    with open(path, "w") as f:
        json.dump(tiny_chain_record(), f, indent=1)
        f.write("\n")
    print("wrote", path)
