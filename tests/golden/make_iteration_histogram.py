"""Write tests/golden/iteration_histogram.json: how many iterations the
solve's groups of the 7B-shaped 4b g64 stack take before their zero repeats,
on a fixed sample of that workload, from the oracle's per-iteration trace.

A group whose zero after iteration k equals its zero after iteration k - 1
(with W_e = 0 in every iteration so far) returns that zero in every later
iteration, so iterations after the k-th change nothing: k is the number of
iterations a solver that stops at a repeated zero runs.  Groups whose shrink
is active (some W_e != 0) before their zero repeats are counted apart.

Calls only oracle/ and the input generator (synth/).  Run from the repo root:
    python tests/golden/make_iteration_histogram.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

WORKLOAD = "llama7b_stack32_4b_g64"
LAYERS = (0, 15, 31)
ITERS = 20


def sample():
    """(tensor, row) pairs: 4 rows spread over every tensor of 3 layers."""
    out = []
    for t in synth.workload(WORKLOAD):
        if t["layer"] in LAYERS:
            R = t["rows"]
            for r in sorted({0, R // 3, (2 * R) // 3, R - 1}):
                out.append((t, r))
    return out


def group_iterations(w16: np.ndarray, nbits: int, gs: int):
    """Per group of one row: (iterations to a repeated zero, shrink active)."""
    w = oracle.f16_to_f32(w16)
    its, active = [], []
    for g in range(w.size // gs):
        tr = oracle.solve_group(w[g * gs:(g + 1) * gs], nbits, iters=ITERS, trace=True)
        z = tr["zero_trace"]
        n, act = ITERS, False
        for k in range(1, ITERS + 1):
            if np.any(tr["e"][k - 1] != 0):
                act = True
            if z[k] == z[k - 1]:
                n = k
                break
        if not act and n < ITERS:
            # the stop is exact: the zero never moves again
            assert np.all(z[n:] == z[n]), "zero moved after repeating"
        its.append(n)
        active.append(act)
    return its, active


def compute():
    oracle.build(force=False)
    hist = [0] * (ITERS + 1)
    n_groups = n_active = 0
    wave_max = []
    for t, r in sample():
        w16 = synth.generate_np(t["seed"], t["layer"], t["tensor_id"], t["rows"], t["cols"],
                                row0=r, nrows=1)[0]
        its, act = group_iterations(w16, t["nbits"], t["group_size"])
        for n, a in zip(its, act):
            n_groups += 1
            if a:
                n_active += 1
            else:
                hist[n] += 1
        # 64 consecutive groups of a row: one wave of the lane-per-group solve
        for j in range(0, len(its), 64):
            wave_max.append(max(its[j:j + 64]))
    done = n_groups - n_active
    mean = sum(k * h for k, h in enumerate(hist)) / max(done, 1)
    return dict(
        source="written by tests/golden/make_iteration_histogram.py from oracle/ traces",
        workload=WORKLOAD, layers=list(LAYERS), rows_per_tensor=4, iters=ITERS,
        groups=n_groups, shrink_active_groups=n_active,
        histogram={str(k): h for k, h in enumerate(hist) if h},
        mean_iterations=round(mean, 4),
        mean_max_over_64_consecutive_groups=round(float(np.mean(wave_max)), 4))


def main():
    out = compute()
    path = os.path.join(ROOT, "tests", "golden", "iteration_histogram.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path, json.dumps(out))


if __name__ == "__main__":
    main()
