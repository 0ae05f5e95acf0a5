"""The oracle against a hand-worked example (tests/golden/hand_example_b2.json)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_b2.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_hand_example():
    g = _load()
    L = np.array(g["layout"], dtype=np.uint8)
    b = g["block_size"]
    w = np.array(g["w"], dtype=np.float32)
    for key, (c, k) in g["ids"].items():
        assert oracle.block_coord(L, int(key)) == (c, k)
    for case in ("fprop_ones", "fprop_onehot"):
        x = np.array(g[case]["x"], dtype=np.float32)
        y = oracle.fprop(L, b, 1, x, w, x.shape[0])
        assert np.array_equal(y, np.array(g[case]["y"], dtype=np.float64)), case
        # feature_axis = 0 reads the same numbers transposed
        y0 = oracle.fprop(L, b, 0, np.ascontiguousarray(x.T), w, x.shape[0])
        assert np.array_equal(y0.T, y)
    dy = np.array(g["bprop_ones"]["dy"], dtype=np.float32)
    assert np.array_equal(oracle.bprop(L, b, 1, dy, w, 1), np.array(g["bprop_ones"]["dx"], dtype=np.float64))
    x = np.array(g["updat"]["x"], dtype=np.float32)
    dy = np.array(g["updat"]["dy"], dtype=np.float32)
    assert np.array_equal(oracle.updat(L, b, 1, [x], [dy], 1), np.array(g["updat"]["dw"], dtype=np.float64))
    assert np.array_equal(oracle.identity(L, b), np.array(g["identity"], dtype=np.float64))
