"""Write the oracle's regression digests for the tiny workload (M=64, K=N=256).

Calls only the CPU oracle and the seeded input generator.  Run from the
repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from hadamard_rotated_w4a4_amd import synth  # noqa: E402


def main():
    d = synth.tiny()
    q4 = oracle.prepare_weights(d.w)
    codes, s = oracle.rotate_quantize_act(d.x)
    y = oracle.gemm(q4, codes, s, d.k)
    out = {
        "workload": d.name,
        "note": "sha256 of the oracle's outputs on synth.tiny(seed=0); regression anchor only",
        "q4_0_sha256": hashlib.sha256(q4.tobytes()).hexdigest(),
        "codes_sha256": hashlib.sha256(codes.tobytes()).hexdigest(),
        "scales_sha256": hashlib.sha256(s.tobytes()).hexdigest(),
        "y_sha256": hashlib.sha256(y.tobytes()).hexdigest(),
        "y_row0_first8_hex": [float(v).hex() for v in y[0, :8]],
    }
    with open(os.path.join(HERE, d.name + ".json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
