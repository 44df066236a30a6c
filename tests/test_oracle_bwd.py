"""Pins for the oracle's backward (CPU only).

The gradients of L = <do, o> + <dht, final_state> are pinned by central finite
differences of the (separately pinned) forward, and, for the arguments L is
linear in (q; v and the initial state jointly), by exact differences with no
truncation error at all.
"""
import math

import numpy as np
import pytest

import oracle
from gdr_inputs import make_inputs

NAMES = ("q", "k", "v", "g", "beta", "initial_state")
GRAD = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", initial_state="dh0")


def loss(x, do, dht, chunk=64):
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                   initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"], chunk=chunk)
    return float(np.sum(r["o"] * do) + np.sum(r["final_state"] * dht))


def grads(x, do, dht, chunk=64):
    return oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["scale"],
                      initial_state=x["initial_state"], dht=dht, cu_seqlens=x["cu_seqlens"],
                      chunk=chunk)


def tiny(seed=3, lens=None):
    shape = dict(Hq=1, Hv=2, K=6, V=5, dtype="fp32", h0=True)
    if lens is None:
        shape.update(B=1, T=40)
    else:
        shape["lens"] = lens
    x = make_inputs(shape, seed=seed, grads=True)
    for n in NAMES:
        x[n] = np.asarray(x[n], np.float64)
    x["do"] = np.asarray(x["do"], np.float64)
    x["dht"] = np.asarray(x["dht"], np.float64)
    return x


@pytest.mark.parametrize("lens", [None, [20, 0, 37]])
def test_p7_every_coordinate_against_central_differences(lens):
    chunk = 16  # several chunks and a partial one, so the checkpointing is exercised
    x = tiny(lens=lens)
    d = grads(x, x["do"], x["dht"], chunk)
    eps = 1e-6
    for n in NAMES:
        base = x[n]
        fd = np.zeros(base.size)
        for i in range(base.size):
            xp = dict(x)
            arr = base.copy().reshape(-1)
            arr[i] += eps
            xp[n] = arr.reshape(base.shape)
            lp = loss(xp, x["do"], x["dht"], chunk)
            arr[i] -= 2 * eps
            xp[n] = arr.reshape(base.shape)
            lm = loss(xp, x["do"], x["dht"], chunk)
            fd[i] = (lp - lm) / (2 * eps)
        ad = d[GRAD[n]].reshape(-1)
        err = np.max(np.abs(fd - ad)) / np.max(np.abs(ad))
        assert err < 1e-7, (n, err)


def test_p7_exact_differences_for_linear_arguments():
    x = tiny(seed=5)
    d = grads(x, x["do"], x["dht"], 16)
    rng = np.random.default_rng(1)
    l0 = loss(x, x["do"], x["dht"], 16)
    # L is linear in q
    dq = rng.standard_normal(x["q"].shape)
    xq = dict(x, q=x["q"] + dq)
    assert math.isclose(loss(xq, x["do"], x["dht"], 16) - l0, float(np.sum(d["dq"] * dq)),
                        rel_tol=1e-11)
    # L is jointly linear in (v, initial_state)
    dv = rng.standard_normal(x["v"].shape)
    dh = rng.standard_normal(x["initial_state"].shape)
    xv = dict(x, v=x["v"] + dv, initial_state=x["initial_state"] + dh)
    lhs = loss(xv, x["do"], x["dht"], 16) - l0
    rhs = float(np.sum(d["dv"] * dv) + np.sum(d["dh0"] * dh))
    assert math.isclose(lhs, rhs, rel_tol=1e-11)


def test_p7_gqa_gradients_sum_over_the_group():
    shape = dict(B=1, T=50, Hq=2, Hv=6, K=8, V=8, dtype="fp32", h0=True)
    x = make_inputs(shape, seed=7, grads=True)
    d = grads(x, x["do"], x["dht"])
    rep = dict(x, q=np.repeat(x["q"], 3, axis=2), k=np.repeat(x["k"], 3, axis=2))
    dr = grads(rep, x["do"], x["dht"])
    for n in ("dq", "dk"):
        summed = dr[n].reshape(1, 50, 2, 3, 8).sum(axis=3)
        np.testing.assert_allclose(d[n], summed, rtol=0, atol=1e-13)
    for n in ("dv", "dg", "dbeta", "dh0"):
        np.testing.assert_array_equal(d[n], dr[n])


@pytest.mark.slow
def test_p7_directional_differences_on_training_slice():
    """B=1, T=128 slice of the training workload (H_q=32, H_v=64, K=V=128)."""
    shape = dict(B=1, T=128, Hq=32, Hv=64, K=128, V=128, dtype="bf16", h0=True)
    x = make_inputs(shape, seed=0, grads=True)
    for n in NAMES:
        x[n] = np.asarray(x[n], np.float64)
    d = grads(x, x["do"], x["dht"])
    rng = np.random.default_rng(2)
    for n in NAMES:
        delta = rng.standard_normal(x[n].shape) * np.sqrt(np.mean(x[n] ** 2))
        eps = 1e-5
        lp = loss(dict(x, **{n: x[n] + eps * delta}), x["do"], x["dht"])
        lm = loss(dict(x, **{n: x[n] - eps * delta}), x["do"], x["dht"])
        fd = (lp - lm) / (2 * eps)
        ad = float(np.sum(d[GRAD[n]] * delta))
        assert abs(fd - ad) <= 1e-6 * abs(ad), (n, fd, ad)
