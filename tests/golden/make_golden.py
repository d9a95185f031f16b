"""Write tests/golden/oracle_regression.json: the oracle's outputs on small
seeded inputs, frozen so that any later change to the oracle's arithmetic
shows up as a test failure (and must then be justified).

Calls only oracle/ and the input generator (synth/).  Run from the repo root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

CASES = [
    # name, seed, layer, tensor_id, rows, cols, nbits, group_size, axis
    ("single_linear_rows0_31_4b_g64_axis1", synth.SEED_SINGLE, 0, 0, 32, 1024, 4, 64, 1),
    ("layer0_q_rows0_319_3b_g64_axis0", synth.SEED_7B, 0, 0, 320, 64, 3, 64, 0),
    ("layer0_gate_rows0_63_2b_g16_axis0", synth.SEED_7B, 0, 4, 64, 64, 2, 16, 0),
    ("70b_layer0_down_rows0_7_1b_g16_axis1", synth.SEED_70B, 0, 6, 8, 512, 1, 16, 1),
]


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def main():
    oracle.build(force=False)
    out = {"source": "written by tests/golden/make_golden.py from oracle/ outputs "
                     "(defaults p=0.7, beta0=10, kappa=1.01, iters=20)",
           "cases": []}
    for name, seed, layer, tid, rows, cols, nb, gs, axis in CASES:
        # a sub-block of the tensor: the first `rows` rows, the first `cols` columns
        full_cols = {0: 4096, 4: 4096, 6: 28672}[tid] if seed != synth.SEED_SINGLE else 1024
        W = synth.generate_np(seed, layer, tid, rows, full_cols, nrows=rows)[:, :cols].copy()
        packed, scale, zero = oracle.quantize(W, nb, gs, axis)
        out["cases"].append(dict(
            name=name, seed=seed, layer=layer, tensor_id=tid, rows=rows, cols=cols,
            full_cols=full_cols, nbits=nb, group_size=gs, axis=axis,
            W_sha256=digest(W), packed_sha256=digest(packed),
            scale=[float(x) for x in scale.ravel()[:64]], zero=[float(x) for x in zero.ravel()[:64]],
            scale_sha256=digest(scale), zero_sha256=digest(zero)))
    path = os.path.join(ROOT, "tests", "golden", "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
