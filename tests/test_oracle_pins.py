"""Pins for the fp64 oracle (CPU only).

The pages print no worked example, so every pin comes from mathematics:
exact rational brute force of the V x K form of the gated delta rule, a dense
transition-product formula, closed forms, a hand-derived scalar example
(tests/golden/scalar_worked_example.json), chunked-form equivalence,
invariants and the warm-up error bound.  Each is chosen so that a plausible
slip in the oracle (a dropped decay or erase term, a wrong sign, the wrong
q/k head for a v head, a transposed state) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gdr_inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    """max |a - b| / rms(b)."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(math.sqrt(float(np.mean(b * b))), 1e-300))


def problem(B=1, T=9, Hq=1, Hv=2, K=3, V=2, seed=1, h0=True, lens=None):
    shape = dict(Hq=Hq, Hv=Hv, K=K, V=V, dtype="fp32", h0=h0)
    if lens is not None:
        shape["lens"] = lens
    else:
        shape.update(B=B, T=T)
    return make_inputs(shape, seed=seed)


def run(x, **kw):
    return oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                      initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"], **kw)


# ---------------------------------------------------------------- P1 exact brute force
def brute_force_vk(x, chunk):
    """Exact rational evaluation of S_t = a_t S_{t-1}(I - b k k^T) + b v k^T,
    o_t = scale S_t q_t with S a V x K matrix.  a_t = exp(g_t) is the double the
    oracle also uses, taken exactly."""
    q, k, v, g, beta = (np.asarray(x[n], np.float64) for n in ("q", "k", "v", "g", "beta"))
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    G = Hv // Hq
    cu = x["cu_seqlens"]
    off = list(range(0, B * T + 1, T)) if cu is None else [int(c) for c in cu]
    qf, kf = q.reshape(-1, Hq, K), k.reshape(-1, Hq, K)
    vf, gf, bf = v.reshape(-1, Hv, V), g.reshape(-1, Hv), beta.reshape(-1, Hv)
    s = Fraction(float(x["scale"]))
    o = np.zeros((B * T, Hv, V))
    hT, hch = [], []
    for j in range(len(off) - 1):
        for hv in range(Hv):
            hq = hv // G
            if x["initial_state"] is None:
                S = [[Fraction(0)] * K for _ in range(V)]
            else:
                h0 = x["initial_state"][j, hv]
                S = [[Fraction(float(h0[kk, vv])) for kk in range(K)] for vv in range(V)]
            for t in range(off[j], off[j + 1]):
                if (t - off[j]) % chunk == 0:
                    hch.append(((j, (t - off[j]) // chunk, hv), [[float(S[vv][kk]) for vv in range(V)] for kk in range(K)]))
                a = Fraction(math.exp(float(gf[t, hv])))
                b = Fraction(float(bf[t, hv]))
                kt = [Fraction(float(z)) for z in kf[t, hq]]
                vt = [Fraction(float(z)) for z in vf[t, hv]]
                qt = [Fraction(float(z)) for z in qf[t, hq]]
                Sk = [sum(S[i][m] * kt[m] for m in range(K)) for i in range(V)]
                S = [[a * (S[i][jj] - b * Sk[i] * kt[jj]) + b * vt[i] * kt[jj] for jj in range(K)]
                     for i in range(V)]
                for i in range(V):
                    o[t, hv, i] = float(s * sum(S[i][jj] * qt[jj] for jj in range(K)))
            hT.append(((j, hv), [[float(S[vv][kk]) for vv in range(V)] for kk in range(K)]))
    return o.reshape(B, T, Hv, V), hT, hch


@pytest.mark.parametrize("case", [
    dict(B=2, T=9, Hq=1, Hv=2, K=3, V=2, h0=True),
    dict(B=1, T=11, Hq=2, Hv=2, K=2, V=4, h0=False),
    dict(lens=[5, 0, 7], Hq=1, Hv=2, K=3, V=2, h0=True),
])
def test_p1_exact_rational_bruteforce(case):
    chunk = 4
    x = problem(seed=11, **case)
    ref_o, ref_hT, ref_hch = brute_force_vk(x, chunk)
    r = run(x, chunk=chunk, want_h=True)
    assert rel(r["o"], ref_o) < 1e-13
    for (j, hv), h in ref_hT:
        np.testing.assert_allclose(r["final_state"][j, hv], np.array(h), rtol=0, atol=1e-13)
    hflat = r["h"].reshape(-1, *r["h"].shape[2:])
    off = [0]
    for j in range(r["final_state"].shape[0]):
        L = (x["cu_seqlens"][j + 1] - x["cu_seqlens"][j]) if x["cu_seqlens"] is not None else x["q"].shape[1]
        off.append(off[-1] + (L + chunk - 1) // chunk)
    for (j, c, hv), h in ref_hch:
        np.testing.assert_allclose(hflat[off[j] + c, hv], np.array(h), rtol=0, atol=1e-13)


def test_golden_scalar_worked_example():
    """K = V = 1 example derived by hand (tests/golden/scalar_worked_example.json)."""
    with open(os.path.join(GOLDEN, "scalar_worked_example.json")) as f:
        ex = json.load(f)
    a = np.array(ex["decay"], np.float64)
    T = len(a)
    sh = (1, T, 1, 1)
    r = oracle.fwd(np.array(ex["q"]).reshape(sh), np.array(ex["k"]).reshape(sh),
                   np.array(ex["v"]).reshape(sh), np.log(a).reshape(1, T, 1),
                   np.array(ex["beta"]).reshape(1, T, 1), ex["scale"],
                   initial_state=np.array(ex["h0"]).reshape(1, 1, 1, 1))
    expect_o = np.array([float(Fraction(s)) for s in ex["o"]])
    np.testing.assert_allclose(r["o"].reshape(-1), expect_o, rtol=1e-14)
    assert abs(r["final_state"].item() - float(Fraction(ex["final_state"]))) < 1e-14


# ------------------------------------------------------ P2 dense transition product
def transition_form(x):
    """h_t = Phi_t..Phi_1 h0 + sum_i Phi_t..Phi_{i+1} b_i k_i v_i^T with
    Phi_j = exp(g_j)(I - b_j k_j k_j^T), built from dense K x K matrices."""
    q, k, v, g, beta = (np.asarray(x[n], np.float64) for n in ("q", "k", "v", "g", "beta"))
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    G = Hv // Hq
    o = np.zeros((B, T, Hv, V))
    hT = np.zeros((B, Hv, K, V))
    for b in range(B):
        for hv in range(Hv):
            hq = hv // G
            h0 = np.zeros((K, V)) if x["initial_state"] is None else x["initial_state"][b, hv]
            Phi = [np.exp(g[b, t, hv]) * (np.eye(K) - beta[b, t, hv] * np.outer(k[b, t, hq], k[b, t, hq]))
                   for t in range(T)]
            for t in range(T):
                P = np.eye(K)
                for jj in range(t, -1, -1):
                    P = P @ Phi[jj]
                h = P @ h0
                for i in range(t + 1):
                    P = np.eye(K)
                    for jj in range(t, i, -1):
                        P = P @ Phi[jj]
                    h = h + P @ (beta[b, i, hv] * np.outer(k[b, i, hq], v[b, i, hv]))
                o[b, t, hv] = x["scale"] * h.T @ q[b, t, hq]
            hT[b, hv] = h
    return o, hT


def test_p2_transition_product_form():
    x = problem(B=2, T=40, Hq=2, Hv=4, K=8, V=6, seed=5)
    o, hT = transition_form(x)
    r = run(x)
    assert rel(r["o"], o) < 1e-12
    assert rel(r["final_state"], hT) < 1e-12


# ---------------------------------------------------------------- P3 closed forms
def test_p3a_literal_beta_zero_is_pure_decay():
    x = problem(B=1, T=100, Hq=2, Hv=4, K=8, V=6, seed=3)
    x["beta"] = np.zeros_like(x["beta"])
    r = run(x)
    G = 2
    cum = np.cumsum(np.asarray(x["g"], np.float64), axis=1)  # [B,T,Hv]
    h0 = np.asarray(x["initial_state"], np.float64)
    q = np.asarray(x["q"], np.float64)
    for hv in range(4):
        expect = x["scale"] * np.exp(cum[0, :, hv])[:, None] * (q[0, :, hv // G] @ h0[0, hv])
        assert rel(r["o"][0, :, hv], expect) < 1e-12
        assert rel(r["final_state"][0, hv], np.exp(cum[0, -1, hv]) * h0[0, hv]) < 1e-12


def orthogonal_keys(T, K, rng):
    Qm, _ = np.linalg.qr(rng.standard_normal((K, T)))
    return Qm.T  # T orthonormal rows


def gla_closed_form(q, k, v, g, beta, scale):
    """Gated linear attention with values beta*v: o = s (tril(QK^T) * Gam) diag(beta) V."""
    q, k, v, g, beta = (np.asarray(z, np.float64) for z in (q, k, v, g, beta))
    cum = np.cumsum(g)
    Gam = np.exp(cum[:, None] - cum[None, :])
    return scale * (np.tril(q @ k.T) * Gam) @ (beta[:, None] * v)


def test_p3b_orthogonal_keys_equal_gated_linear_attention():
    rng = np.random.default_rng(7)
    T, K, V = 24, 32, 5
    x = problem(B=1, T=T, Hq=1, Hv=1, K=K, V=V, seed=7, h0=False)
    x["k"] = orthogonal_keys(T, K, rng).reshape(1, T, 1, K)
    r = run(x)
    expect = gla_closed_form(x["q"][0, :, 0].astype(np.float64), x["k"][0, :, 0], x["v"][0, :, 0],
                             x["g"][0, :, 0], x["beta"][0, :, 0], x["scale"])
    assert rel(r["o"][0, :, 0], expect) < 1e-12
    # g = 0, beta = 1: the state is the running sum of k v^T
    x["g"] = np.zeros_like(x["g"])
    x["beta"] = np.ones_like(x["beta"])
    r = run(x)
    kk, vv = x["k"][0, :, 0], x["v"][0, :, 0].astype(np.float64)
    assert rel(r["final_state"][0, 0], kk.T @ vv) < 1e-12
    expect = x["scale"] * np.tril(x["q"][0, :, 0].astype(np.float64) @ kk.T) @ vv
    assert rel(r["o"][0, :, 0], expect) < 1e-12


def test_p3c_first_order_in_beta():
    x = problem(B=1, T=50, Hq=1, Hv=1, K=16, V=8, seed=9, h0=False)
    beta = np.asarray(x["beta"], np.float64)
    expect = gla_closed_form(x["q"][0, :, 0].astype(np.float64), x["k"][0, :, 0].astype(np.float64),
                             x["v"][0, :, 0], x["g"][0, :, 0], beta[0, :, 0], x["scale"])
    errs = []
    for eps in (1e-4, 1e-6):
        x["beta"] = eps * beta
        r = run(x)
        errs.append(rel(r["o"][0, :, 0] / eps, expect))
    assert errs[0] < 1e-2 and errs[1] < 1e-4 and errs[1] < errs[0] / 50


def test_p3d_delta_rule_overwrite_with_repeated_key():
    x = problem(B=1, T=30, Hq=1, Hv=1, K=8, V=6, seed=13, h0=True)
    kvec = x["k"][0, 0, 0].astype(np.float64)
    kvec /= np.linalg.norm(kvec)
    x["k"] = np.broadcast_to(kvec, x["k"].shape).copy()
    x["g"] = np.zeros_like(x["g"])
    x["beta"] = np.ones_like(x["beta"])
    r = run(x)
    P = np.eye(8) - np.outer(kvec, kvec)
    h0 = x["initial_state"][0, 0].astype(np.float64)
    q = x["q"][0, :, 0].astype(np.float64)
    expect = x["scale"] * ((q @ (P @ h0)) + (q @ kvec)[:, None] * x["v"][0, :, 0])
    assert rel(r["o"][0, :, 0], expect) < 1e-12
    assert rel(r["final_state"][0, 0], P @ h0 + np.outer(kvec, x["v"][0, -1, 0])) < 1e-12


# ------------------------------------------------------- P4 chunked-form equivalence
@pytest.mark.parametrize("case", [
    dict(B=1, T=256, Hq=2, Hv=2, K=64, V=64, h0=False),
    dict(B=2, T=200, Hq=2, Hv=4, K=16, V=24, h0=True),
    dict(lens=[70, 1, 130, 64, 0], Hq=1, Hv=2, K=16, V=8, h0=True),
])
def test_p4_chunked_form_equals_token_recurrence(case):
    x = problem(seed=17, **case)
    r = run(x, want_h=True)
    c = oracle.chunk_form(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                          initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"])
    assert rel(c["o"], r["o"]) < 1e-12
    assert rel(c["final_state"], r["final_state"]) < 1e-12
    assert rel(c["h"], r["h"]) < 1e-12
    assert rel(c["gam"], r["g_cum"]) < 1e-14


# ------------------------------------------ P4 chunked intermediates (T, W, U) pinned
def delta_errors(kc, vc, gc, bc, S0):
    """Per-token delta-rule errors u_t = beta_t (v_t - exp(g_t) S_{t-1} k_t) of the
    recurrence S_t = exp(g_t) S_{t-1} + k-write, run in the V x K form over one
    chunk from the start state S0 (V x K).  Written from the recurrence alone."""
    S = np.array(S0, np.float64)
    out = []
    for t in range(len(gc)):
        a = math.exp(gc[t])
        u = bc[t] * (vc[t] - a * (S @ kc[t]))
        S = a * S + np.outer(u, kc[t])
        out.append(u)
    return np.array(out)


def chunk_spans(x, chunk=64):
    """(sequence, first token, token count) of every chunk of a packed problem."""
    B, T = x["q"].shape[0], x["q"].shape[1]
    cu = x["cu_seqlens"]
    off = list(range(0, B * T + 1, T)) if cu is None else [int(c) for c in cu]
    for j in range(len(off) - 1):
        for s in range(off[j], off[j + 1], chunk):
            yield j, s, min(chunk, off[j + 1] - s)


@pytest.mark.parametrize("case", [
    dict(B=1, T=150, Hq=1, Hv=2, K=16, V=8, h0=True),
    dict(lens=[70, 1, 130, 0, 64], Hq=1, Hv=2, K=8, V=4, h0=False),
    dict(B=1, T=64, Hq=2, Hv=4, K=64, V=16, h0=True),
])
def test_p4_chunk_intermediates_match_the_recurrence(case):
    """chunk_form's per-chunk T, W and U, pinned by the token recurrence itself.
    Row r of U - W h is the delta-rule error u_r of token r when the chunk starts
    from state h, so with the recurrence run over the chunk alone:
      U        = errors from a zero start with the chunk's values,
      W[:, d]  = -errors from the start state with h[d, 0] = 1 and zero values,
      T[:, i]  = errors from a zero start with a unit value at token i only, / beta_i;
    and T is zero past the chunk end.  Also the residuals of the definitions
    (efeozkan, "2. Hardware-Friendly Algebraic Reformulation": A, then W and U):
    |T (I + A) - I|, |(I + A) U - diag(beta) V|, |(I + A) W - diag(beta e^gam) K|."""
    x = problem(seed=23, **case)
    c = oracle.chunk_form(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                          initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"])
    Hq, K = x["q"].shape[2], x["q"].shape[3]
    Hv, V = x["v"].shape[2], x["v"].shape[3]
    G = Hv // Hq
    kf, vf = x["k"].reshape(-1, Hq, K).astype(np.float64), x["v"].reshape(-1, Hv, V).astype(np.float64)
    gf, bf = x["g"].reshape(-1, Hv).astype(np.float64), x["beta"].reshape(-1, Hv).astype(np.float64)
    Tr, Wf, Uf = c["T_rows"].reshape(-1, Hv, 64), c["W"].reshape(-1, Hv, K), c["U"].reshape(-1, Hv, V)
    worst = 0.0
    for _, s, n in chunk_spans(x):
        for hv in range(Hv):
            kc, vc = kf[s:s + n, hv // G], vf[s:s + n, hv]
            gc, bc = gf[s:s + n, hv], bf[s:s + n, hv]
            U_pin = delta_errors(kc, vc, gc, bc, np.zeros((V, K)))
            W_pin = np.zeros((n, K))
            for d in range(K):
                S0 = np.zeros((1, K))
                S0[0, d] = 1.0
                W_pin[:, d] = -delta_errors(kc, np.zeros((n, 1)), gc, bc, S0)[:, 0]
            T_pin = np.zeros((n, n))
            for i in range(n):
                e = np.zeros((n, 1))
                e[i, 0] = 1.0
                T_pin[:, i] = delta_errors(kc, e, gc, bc, np.zeros((1, K)))[:, 0] / bc[i]
            Tc = Tr[s:s + n, hv, :n]
            assert np.all(Tr[s:s + n, hv, n:] == 0.0)
            for got, want in ((Uf[s:s + n, hv], U_pin), (Wf[s:s + n, hv], W_pin), (Tc, T_pin)):
                e_ = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-300)
                worst = max(worst, e_)
                assert e_ < 1e-12
            # residuals of the definitions
            gam = np.cumsum(gc)
            A = np.tril(bc[:, None] * (kc @ kc.T) * np.exp(gam[:, None] - gam[None, :]), -1)
            IA = np.eye(n) + A
            assert np.max(np.abs(Tc @ IA - np.eye(n))) < 1e-12
            assert np.max(np.abs(IA @ Uf[s:s + n, hv] - bc[:, None] * vc)) < 1e-12
            assert np.max(np.abs(IA @ Wf[s:s + n, hv] - (bc * np.exp(gam))[:, None] * kc)) < 1e-12
    print("worst relative deviation of T, W, U from the recurrence: %.3g" % worst)


def test_p4_numpy_twin_matches_c():
    x = problem(B=2, T=70, Hq=2, Hv=4, K=8, V=8, seed=19)
    o, hT = oracle.token_recurrence_np(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                                       x["initial_state"])
    r = run(x)
    assert rel(r["o"], o) < 1e-13 and rel(r["final_state"], hT) < 1e-13


# ---------------------------------------------------------------- P5 invariants
def test_p5_state_continuation():
    x = problem(B=1, T=200, Hq=2, Hv=4, K=16, V=16, seed=21)
    full = run(x)
    t = 77
    a = {n: x[n][:, :t] for n in ("q", "k", "v", "g", "beta")}
    b = {n: x[n][:, t:] for n in ("q", "k", "v", "g", "beta")}
    ra = oracle.fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], x["scale"], x["initial_state"])
    rb = oracle.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], x["scale"], ra["final_state"])
    assert rel(np.concatenate([ra["o"], rb["o"]], axis=1), full["o"]) < 1e-12
    assert rel(rb["final_state"], full["final_state"]) < 1e-12


def test_p5_joint_linearity_in_v_and_h0():
    x = problem(B=1, T=90, Hq=1, Hv=2, K=8, V=8, seed=23)
    rng = np.random.default_rng(0)
    v2 = rng.standard_normal(x["v"].shape)
    h2 = rng.standard_normal(x["initial_state"].shape)
    r1 = run(x)
    r2 = oracle.fwd(x["q"], x["k"], v2, x["g"], x["beta"], x["scale"], h2)
    r3 = oracle.fwd(x["q"], x["k"], 2.0 * x["v"] - 3.0 * v2, x["g"], x["beta"], x["scale"],
                    2.0 * x["initial_state"] - 3.0 * h2)
    assert rel(r3["o"], 2.0 * r1["o"] - 3.0 * r2["o"]) < 1e-12
    assert rel(r3["final_state"], 2.0 * r1["final_state"] - 3.0 * r2["final_state"]) < 1e-12


def test_p5_varlen_equals_separate_calls():
    lens = [33, 64, 1, 100]
    x = problem(lens=lens, Hq=2, Hv=4, K=8, V=8, seed=25)
    r = run(x, want_h=True)
    cu = x["cu_seqlens"]
    hflat = r["h"].reshape(-1, *r["h"].shape[2:])
    cbase = 0
    for j, L in enumerate(lens):
        sl = slice(int(cu[j]), int(cu[j + 1]))
        rj = oracle.fwd(*(x[n][:, sl] for n in ("q", "k", "v", "g", "beta")), x["scale"],
                        x["initial_state"][j:j + 1], want_h=True)
        assert np.array_equal(rj["o"][0], r["o"][0, sl])
        assert np.array_equal(rj["final_state"][0], r["final_state"][j])
        nc = (L + 63) // 64
        assert np.array_equal(rj["h"][0], hflat[cbase:cbase + nc])
        cbase += nc


def test_p5_gqa_equals_explicit_repetition():
    x = problem(B=1, T=80, Hq=2, Hv=6, K=8, V=8, seed=27)
    r = run(x)
    rep = dict(x)
    rep["q"] = np.repeat(x["q"], 3, axis=2)
    rep["k"] = np.repeat(x["k"], 3, axis=2)
    rr = run(rep)
    assert np.array_equal(r["o"], rr["o"])
    assert np.array_equal(r["final_state"], rr["final_state"])


def test_p5_head_permutation_equivariance():
    x = problem(B=1, T=60, Hq=3, Hv=6, K=8, V=8, seed=29)
    r = run(x)
    perm_q = np.array([2, 0, 1])
    perm_v = np.concatenate([[2 * p, 2 * p + 1] for p in perm_q])
    y = dict(x)
    y["q"], y["k"] = x["q"][:, :, perm_q], x["k"][:, :, perm_q]
    for n in ("v", "g", "beta"):
        y[n] = x[n][:, :, perm_v]
    y["initial_state"] = x["initial_state"][:, perm_v]
    ry = run(y)
    assert np.array_equal(ry["o"], r["o"][:, :, perm_v])
    assert np.array_equal(ry["final_state"], r["final_state"][:, perm_v])


def test_p5_non_expansive_state_norm():
    x = problem(B=1, T=64, Hq=1, Hv=2, K=16, V=8, seed=31)
    r = run(x, chunk=1, want_h=True)  # chunk of one token: every per-token state
    h = r["h"][0]  # [T, Hv, K, V]: state before each token
    hs = np.concatenate([h, r["final_state"]], axis=0)
    for hv in range(2):
        for t in range(64):
            bound = np.exp(x["g"][0, t, hv]) * np.linalg.norm(hs[t, hv]) + \
                x["beta"][0, t, hv] * np.linalg.norm(x["k"][0, t, 0]) * np.linalg.norm(x["v"][0, t, hv])
            assert np.linalg.norm(hs[t + 1, hv]) <= bound * (1 + 1e-12)


# ---------------------------------------------------------------- P6 warm-up split
def split(x, L, Wm, **kw):
    return oracle.fwd_split(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], L, Wm,
                            initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"], **kw)


def test_p6_full_window_is_exact():
    x = problem(B=2, T=64 * 10 + 5, Hq=1, Hv=2, K=8, V=8, seed=33)
    ex = run(x, want_h=True)
    for L, Wm in ((3, 100), (11, 0), (4, 11)):
        s = split(x, L, Wm, want_h=True)
        assert np.array_equal(s["o"], ex["o"]) and np.array_equal(s["h"], ex["h"])
        assert np.array_equal(s["final_state"], ex["final_state"])


def test_p6_warmup_error_bound_and_convergence():
    x = problem(B=1, T=64 * 24, Hq=1, Hv=2, K=16, V=16, seed=35, h0=True)
    x["g"] = 0.01 * x["g"]  # weak decay, so the warm-up error is visible
    ex = run(x, want_h=True)
    gcum = np.concatenate([[0.0], np.cumsum(x["g"][0, :, 0].astype(np.float64))])
    L = 5
    errs = []
    for Wm in (1, 2, 4, 8, 16):
        s = split(x, L, Wm, want_h=True)
        for cs in range(L, 24, L):
            if cs - Wm <= 0:
                assert np.array_equal(s["h"][0, cs, 0], ex["h"][0, cs, 0])
                continue
            err = np.linalg.norm(s["h"][0, cs, 0] - ex["h"][0, cs, 0])
            window = gcum[cs * 64] - gcum[(cs - Wm) * 64]
            assert err <= np.exp(window) * np.linalg.norm(ex["h"][0, cs - Wm, 0]) * (1 + 1e-9) + 1e-14
        errs.append(rel(s["o"], ex["o"]))
    assert all(b <= a * 1.0001 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < errs[0]


def test_p6_config_gates_make_warmup_exact_in_fp64():
    """At the workload's gate scale (per-chunk log-decay about -26) an 8-chunk
    window makes the split agree with the exact scan to rounding."""
    x = problem(B=1, T=64 * 40, Hq=1, Hv=2, K=32, V=32, seed=37, h0=False)
    ex = run(x)
    s = split(x, 7, 8)
    assert rel(s["o"], ex["o"]) < 1e-12


def test_p6_exact_split_carry_reproduces_the_unsplit_state():
    """The exact sequence split rests on the recurrence being affine in its start
    state: over a segment, start h -> M h + b with M the end state from h = I over
    zero values (as many value columns as keys) and b the end state from zero over
    the real values.  Chaining start(s+1) = M_s start(s) + b_s over three segments
    from a random start must give the unsplit final state (fp64)."""
    x = make_inputs(dict(B=1, T=64 * 3 + 21, Hq=1, Hv=2, K=8, V=5, dtype="fp32", h0=True), seed=11)
    q, k, v, g, beta, sc = x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"]
    K = q.shape[3]
    bounds = [0, 64, 128 + 17, q.shape[1]]
    h = x["initial_state"].astype(np.float64)
    eye = np.broadcast_to(np.eye(K), (1, 2, K, K)).copy()
    for a, b in zip(bounds[:-1], bounds[1:]):
        sl = lambda t: np.ascontiguousarray(t[:, a:b])
        zero_v = np.zeros((1, b - a, 2, K))
        M = oracle.fwd(sl(q), sl(k), zero_v, sl(g), sl(beta), sc, initial_state=eye)["final_state"]
        off = oracle.fwd(sl(q), sl(k), sl(v), sl(g), sl(beta), sc)["final_state"]
        h = np.einsum("nhij,nhjv->nhiv", M, h) + off
    want = oracle.fwd(q, k, v, g, beta, sc, initial_state=x["initial_state"])["final_state"]
    assert np.max(np.abs(h - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
