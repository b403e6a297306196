"""The host Philox4x32-10 generator of the synthetic inputs reproduces the
published known-answer vectors (tests/golden/philox4x32_10_kat.json); the GPU
tests check the device generator against the host one row by row."""
import json
import os

import numpy as np

import lsa_synth as S


def test_philox4x32_10_known_answers():
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")
    with open(path) as f:
        kat = json.load(f)
    assert len(kat["vectors"]) == 3
    for v in kat["vectors"]:
        c = [np.array([int(x, 16)], np.uint32) for x in v["counter"]]
        k = [int(x, 16) for x in v["key"]]
        out = S.philox4x32_10(*c, k[0], k[1])
        assert [f"{int(w[0]):08x}" for w in out] == v["out"]
