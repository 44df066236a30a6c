"""GPU parity of the forward (HIP kernels through the C ABI) against the fp64 oracle.

Metric per output tensor: max |gpu - oracle| / rms(oracle); bar 1e-4 for fp32
inputs and 2e-2 for bf16 inputs (o in fp32).  Small cases compare every
element and span several chunks with a ragged tail; the full-size workloads
compare whole (sequence, q/k-head group) units that the oracle computes
exactly, since units of the recurrence are independent.
"""
import numpy as np
import pytest
import torch

import oracle
from gdr_inputs import make_inputs
from gpu_helpers import gpu_inputs, host, rel, run_fwd, slice_units, tol

pytestmark = pytest.mark.gpu


def ora(x, **kw):
    return oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                      initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"], **kw)


def check_all(x, out, ref, chunked=None, t=None):
    t = tol(x) if t is None else t
    g_cum, A, o, h, ht = out[:5]
    errs = {"o": rel(host(o), ref["o"]), "final_state": rel(host(ht), ref["final_state"])}
    errs["g_cum"] = rel(host(g_cum), ref["g_cum"])
    if h is not None:
        errs["h"] = rel(host(h), ref["h"])
    if chunked is not None:
        errs["A"] = rel(host(A), chunked["T_rows"])
    print({k: "%.3g" % v for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= t, (k, e)
    return errs


def test_tiny_fp32_workload():
    """B=1, T=256, H_q=H_v=2, K=V=64, fp32 (every element, every output)."""
    x = make_inputs("tiny_fp32", seed=0)
    out = run_fwd(x, return_wu=True)
    ref = ora(x, want_h=True)
    ch = oracle.chunk_form(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    check_all(x, out, ref, ch)
    assert rel(host(out[5]), ch["W"]) <= 1e-4
    assert rel(host(out[6]), ch["U"]) <= 1e-4


@pytest.mark.parametrize("shape", [
    dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
    dict(B=1, T=200, Hq=1, Hv=1, K=64, V=128, dtype="bf16", h0=True),
    dict(B=1, T=130, Hq=2, Hv=2, K=128, V=64, dtype="bf16", h0=False),
    dict(B=2, T=250, Hq=2, Hv=6, K=64, V=64, dtype="bf16", h0=True),
    dict(B=3, T=77, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True),
    dict(B=1, T=190, Hq=1, Hv=3, K=128, V=128, dtype="fp32", h0=True),
])
def test_small_ragged(shape):
    x = make_inputs(shape, seed=1)
    out = run_fwd(x, return_wu=True)
    ref = ora(x, want_h=True)
    ch = oracle.chunk_form(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                           initial_state=x["initial_state"])
    check_all(x, out, ref, ch)
    t = tol(x)
    assert rel(host(out[5]), ch["W"]) <= t
    assert rel(host(out[6]), ch["U"]) <= t


@pytest.mark.parametrize("h0", [True, False])
def test_no_tokens_returns_the_initial_state(h0):
    """T = 0: nothing to scan; o is empty and the final state is the initial state
    (zeros without one), as the recurrence over an empty sequence gives."""
    x = make_inputs(dict(B=2, T=0, Hq=1, Hv=2, K=64, V=64, dtype="bf16", h0=h0), seed=5)
    out = run_fwd(x)
    assert tuple(out[2].shape) == (2, 0, 2, 64)
    ht = host(out[4])
    want = x["initial_state"] if h0 else np.zeros((2, 2, 64, 64))
    assert np.array_equal(ht, np.asarray(want, np.float64))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 128])
def test_short_sequences(T):
    x = make_inputs(dict(B=2, T=T, Hq=1, Hv=2, K=128, V=128, dtype="bf16", h0=True), seed=2)
    check_all(x, run_fwd(x), ora(x, want_h=True))


def test_varlen_small_with_empty_sequence():
    x = make_inputs(dict(lens=[70, 1, 130, 0, 64, 200], Hq=2, Hv=4, K=128, V=128, dtype="bf16",
                         h0=True), seed=3)
    out = run_fwd(x)
    check_all(x, out, ora(x, want_h=True))
    # the empty sequence returns its initial state
    assert np.array_equal(host(out[4])[3], x["initial_state"][3].astype(np.float64))


def test_varlen_lengths_increasing_longest_first():
    """Packed sequences are scanned longest first: lengths in increasing order (the
    dispatch reverses them), fp32 with G = 3 and two value blocks."""
    x = make_inputs(dict(lens=[1, 63, 64, 65, 128, 190, 257, 300], Hq=1, Hv=3, K=64, V=128,
                         dtype="fp32", h0=True), seed=5)
    check_all(x, run_fwd(x), ora(x, want_h=True))


def test_varlen_many_short_sequences_natural_order():
    """More than 8192 packed sequences keep their natural order (no length sort)."""
    rng = np.random.default_rng(7)
    lens = [int(v) for v in rng.integers(0, 5, size=8300)]
    x = make_inputs(dict(lens=lens, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), seed=6)
    check_all(x, run_fwd(x), ora(x, want_h=True))


@pytest.mark.parametrize("shape,L", [
    (dict(B=1, T=64 * 20 + 5, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), 3),
    (dict(B=2, T=64 * 9, Hq=1, Hv=2, K=128, V=64, dtype="bf16", h0=True), 2),
    (dict(lens=[300, 1, 0, 700, 64, 129], Hq=2, Hv=4, K=64, V=128, dtype="fp32", h0=True), 3),
    (dict(lens=[1000, 130, 5], Hq=1, Hv=1, K=128, V=128, dtype="bf16", h0=False), 4),
    (dict(B=1, T=64 * 6, Hq=2, Hv=4, K=64, V=64, dtype="bf16", h0=True), 1),
    (dict(lens=[64] * 5 + [900, 0, 3], Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), 5),
    (dict(B=1, T=1, Hq=1, Hv=1, K=64, V=64, dtype="fp32", h0=True), 1),
])
def test_exact_sequence_split(shape, L):
    """Exact split: every segment's transition matrix and zero-start end state in
    parallel, the serial carry, then the segments again from their true start
    states: the result of the unsplit recurrence, chunk-start states included."""
    x = make_inputs(shape, seed=8)
    out = run_fwd(x, cp_mode="exact", cp_segment_chunks=L)
    check_all(x, out, ora(x, want_h=True))


def test_exact_split_where_the_warmup_fails():
    """Gates that do not decay (g = 0 on one v head): the warm-up split is off by
    far more than the bar, the exact split is not."""
    x = make_inputs(dict(B=1, T=64 * 24, Hq=1, Hv=2, K=128, V=128, dtype="bf16", h0=True), seed=9)
    x["g"][:, :, 1] = 0.0
    ref = ora(x)
    ex = host(run_fwd(x, cp_mode="exact", cp_segment_chunks=5)[2])
    wu = host(run_fwd(x, cp_mode="warmup", cp_segment_chunks=5, cp_warmup_chunks=2)[2])
    e_ex, e_wu = rel(ex, ref["o"]), rel(wu, ref["o"])
    print("g = 0 head: exact split %.3g, warm-up split %.3g" % (e_ex, e_wu), flush=True)
    assert e_ex <= 2e-2
    assert e_wu > 2e-2


def test_prefill_shard_full_size_every_unit():
    """B=4, T=4096, H_q=16, H_v=32, K=V=128, bf16 (the timed workload), launched whole:
    every element of o, the final state, the chunk-start states h, g_cum and A
    (T, one row per token) against the oracle over all 128 (sequence, v head)
    units; A against the chunked form, one (sequence, q/k head) group at a time."""
    x = make_inputs("prefill_shard", seed=0)
    g_cum, A, o, h, ht = run_fwd(x, return_h=True)
    ref = ora(x, want_h=True)
    errs = {"o": rel(host(o), ref["o"]), "final_state": rel(host(ht), ref["final_state"]),
            "g_cum": rel(host(g_cum), ref["g_cum"])}
    del o, ht, g_cum
    errs["h"] = rel(host(h), ref["h"])
    del h, ref
    A = host(A)
    worst = 0.0
    rms = 0.0
    for b in range(4):
        for hq in range(16):
            y, hs = slice_units(x, b, hq)
            c = oracle.chunk_form(y["q"], y["k"], y["v"], y["g"], y["beta"], y["scale"], y["initial_state"])
            worst = max(worst, float(np.max(np.abs(A[b:b + 1, :, hs] - c["T_rows"]))))
            rms += float(np.sum(c["T_rows"] ** 2))
    errs["A"] = worst / np.sqrt(rms / A.size)
    print({k: "%.3g" % v for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)


def test_strong_decay_past_fp32_exp_range():
    """Gates eight times the recipe's (mean log-decay about -3.2 per token): the
    running log-gate of a chunk spans about -200, past the fp32 range of exp, so
    e^gam of the chunk's later tokens underflows and only the difference form
    exp(gam_r - gam_i) keeps the in-chunk decays.  Every element against the oracle,
    bf16 and fp32, with ragged tails and an initial state."""
    for shape in (dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
                  dict(B=1, T=190, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True)):
        x = make_inputs(shape, seed=14)
        x["g"] = (x["g"] * 8.0).astype(np.float32)
        span = float(np.min(oracle.chunk_cumsum(x["g"], np.arange(x["q"].shape[0] + 1) * x["q"].shape[1])))
        print(shape["dtype"], "most negative in-chunk running log-gate %.1f" % span, flush=True)
        assert span < -88.0
        check_all(x, run_fwd(x), ora(x, want_h=True))


def test_bf16_output_within_rounding_bound():
    x = make_inputs(dict(B=1, T=256, Hq=1, Hv=2, K=128, V=128, dtype="bf16", h0=True), seed=4)
    o = host(run_fwd(x, output_dtype=torch.bfloat16)[2])
    ref = ora(x)["o"]
    rms = np.sqrt(np.mean(ref ** 2))
    # bf16 rounding of the result adds at most 2^-8 |o| per element
    assert np.all(np.abs(o - ref) <= 2e-2 * rms + 2.0 ** -8 * np.abs(ref))


def test_run_to_run_bitwise_determinism():
    x = make_inputs(dict(B=2, T=333, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=5)
    a = run_fwd(x)
    b = run_fwd(x)
    for ta, tb in zip(a, b):
        if ta is not None:
            assert torch.equal(ta, tb)


def test_timing_events_with_null_entries():
    """The events hook records only the non-NULL entries (here the scan's pair)
    and changes no result."""
    import ctypes
    from gated_delta_rule_85_amd import _lib
    x = make_inputs(dict(B=1, T=200, Hq=1, Hv=2, K=64, V=64, dtype="bf16", h0=True), seed=6)
    ref = run_fwd(x, return_h=False, cp_mode="off")
    d = gpu_inputs(x)
    B, T, Hq, K = d["q"].shape
    Hv, V = d["v"].shape[2], d["v"].shape[3]
    o = torch.empty((B, T, Hv, V), device="cuda")
    ht = torch.empty((B, Hv, K, V), device="cuda")
    gc = torch.empty((B, T, Hv), device="cuda")
    A = torch.empty((B, T, Hv, 64), device="cuda")
    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, B
    a.dtype, a.out_dtype, a.scale, a.cp_mode = _lib.BF16, _lib.F32, float(x["scale"]), _lib.CP_OFF
    a.q, a.k, a.v = d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr()
    a.g, a.beta, a.initial_state = d["g"].data_ptr(), d["beta"].data_ptr(), d["initial_state"].data_ptr()
    a.o, a.final_state, a.g_cum, a.A = o.data_ptr(), ht.data_ptr(), gc.data_ptr(), A.data_ptr()
    ws = torch.empty(max(_lib.fwd_workspace(a), 1), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    arr = (ctypes.c_void_p * (2 * _lib.FWD_STAGES))()
    for i in (2, 3):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        arr[i] = e.value
    a.events = ctypes.addressof(arr)
    _lib.fwd(a, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    f = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(f), arr[2], arr[3]) == 0 and f.value > 0.0
    for i in (2, 3):
        hip.hipEventDestroy(arr[i])
    assert torch.equal(o, ref[2]) and torch.equal(ht, ref[4])
    assert torch.equal(gc, ref[0]) and torch.equal(A, ref[1])


def test_device_offsets_are_clamped():
    """Offsets on the device are never read on the host; the library clamps each to
    [previous, T] before any kernel uses them.  Offsets with a decreasing entry and a
    last entry past T give the result of the clamped offsets [0, 70, 70, 200, 260]:
    an empty second sequence (final state = initial state) and a last one that ends
    at T."""
    x = make_inputs(dict(lens=[70, 0, 130, 60], Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=13)
    d = gpu_inputs(x)
    bad = torch.tensor([0, 70, 60, 200, 400], dtype=torch.int32, device="cuda")
    from gated_delta_rule_85_amd import chunk_gated_delta_rule_fwd
    _, _, o, _, ht = chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"],
                                                d["initial_state"], bad, return_h=False)
    torch.cuda.synchronize()
    ref = ora(x)
    eo, eh = rel(host(o), ref["o"]), rel(host(ht), ref["final_state"])
    print("clamped offsets: o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2
    assert np.array_equal(host(ht)[1], x["initial_state"][1].astype(np.float64))
