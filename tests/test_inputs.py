"""The seeded input recipe (CPU only)."""
import json
import os

import numpy as np

from gdr_inputs import make_inputs, round_bf16, varlen_lengths


def test_varlen_lengths_fixture():
    with open(os.path.join(os.path.dirname(__file__), "golden", "varlen_lengths_seed0.json")) as f:
        fx = json.load(f)
    lens = varlen_lengths(np.random.default_rng(0), 16, 128, 16384, 65536)
    assert list(map(int, lens)) == fx["lengths"]
    assert int(lens.sum()) == fx["total_tokens"]
    assert int(np.sum((lens + 63) // 64)) == fx["chunks_per_head"]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -9, 3.14159], np.float32)
    r = round_bf16(x)
    assert list(r[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, -1.0]
    assert abs(r[4] - 3.140625) < 1e-7
    assert np.all(round_bf16(r) == r)


def test_recipe_shapes_and_distributions():
    x = make_inputs(dict(B=2, T=300, Hq=2, Hv=4, K=64, V=32, dtype="bf16", h0=True), seed=0)
    assert x["q"].shape == (2, 300, 2, 64) and x["v"].shape == (2, 300, 4, 32)
    assert x["initial_state"].shape == (2, 4, 64, 32)
    n = np.linalg.norm(x["q"].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert np.all(x["g"] <= 0) and np.all((x["beta"] > 0) & (x["beta"] < 1))
    assert np.all(round_bf16(x["k"]) == x["k"])
    y = make_inputs(dict(lens=[5, 0, 70], Hq=1, Hv=2, K=8, V=8, dtype="bf16"), seed=0)
    assert list(y["cu_seqlens"]) == [0, 5, 5, 75] and y["q"].shape == (1, 75, 1, 8)
