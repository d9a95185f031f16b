"""The iterations a group of the 7B-shaped 4b g64 stack needs before its
zero repeats (the data dependence of the solve's run time), recomputed from
the oracle on the fixed sample and compared with the committed record.

The record (tests/golden/iteration_histogram.json) is written by
tests/golden/make_iteration_histogram.py, which calls only the oracle; the
recomputation also checks, for every sampled group with W_e = 0, that the
zero stays at its first repeated value through the last of the 20
iterations.  That is the exactness of stopping at a repeated zero: in the
alternating solve (lnwmold.com HQQ guide, section 2.1) the zero update reads
the codes W_q, the weights and W_e, and with W_e = 0 the codes are a
function of the zero alone, so an unchanged zero repeats for ever."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "golden"))


def test_iteration_histogram_matches_record():
    import make_iteration_histogram as m

    with open(os.path.join(ROOT, "tests", "golden", "iteration_histogram.json")) as f:
        rec = json.load(f)
    got = m.compute()
    assert got == rec
    hist = {int(k): v for k, v in rec["histogram"].items()}
    assert sum(hist.values()) + rec["shrink_active_groups"] == rec["groups"]
    # at least one iteration is needed to see a repeat, and the zero moves in
    # the first iteration of every group of this workload
    assert min(hist) >= 2
    # the mean is far below the 20 iterations the method prescribes, and the
    # slowest of 64 consecutive groups far above it
    assert rec["mean_iterations"] < 5.0 < rec["mean_max_over_64_consecutive_groups"]
