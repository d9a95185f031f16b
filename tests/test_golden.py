"""Frozen oracle outputs (tests/golden/oracle_regression.json, written by
tests/golden/make_golden.py from oracle/ alone).  A failure here means the
oracle's arithmetic or the input generator changed."""
import hashlib
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_regression.json")


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_oracle_regression(oracle_mod):
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        W = synth.generate_np(c["seed"], c["layer"], c["tensor_id"], c["rows"], c["full_cols"],
                              nrows=c["rows"])[:, :c["cols"]].copy()
        assert _digest(W) == c["W_sha256"], c["name"]
        packed, scale, zero = oracle_mod.quantize(W, c["nbits"], c["group_size"], c["axis"])
        assert _digest(packed) == c["packed_sha256"], c["name"]
        assert np.array_equal(scale.ravel()[:64], np.array(c["scale"], np.float32))
        assert np.array_equal(zero.ravel()[:64], np.array(c["zero"], np.float32))
        assert _digest(scale) == c["scale_sha256"] and _digest(zero) == c["zero_sha256"]
