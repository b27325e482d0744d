"""Write tests/golden/cfg1_oracle.json from the CPU oracle (and nothing else).

Run from the repository root:  python tests/golden/make_golden.py
The file is a regression anchor for the oracle on the smallest workload
(H=256, I=128, M=1, seed 101) and the expected values of the GPU parity test
for that workload.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    c = synth.make_config("cfg1")
    g, u, o = oracle.expert_gate_up(c.slots[0], c.layout, c.x, c.H, c.I)
    doc = {
        "workload": "single expert H=256 I=128 M=1, seed 101 (synth.make_config('cfg1'))",
        "writer": "tests/golden/make_golden.py (oracle only)",
        "slot_sha256": synth.sha256_hex(c.slots),
        "x_sha256": synth.sha256_hex(c.x),
        "gate_f32_bits": [int(v) for v in g.view(np.uint32).ravel()],
        "up_f32_bits": [int(v) for v in u.view(np.uint32).ravel()],
        "out_bf16_bits": [int(v) for v in o.ravel()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg1_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
