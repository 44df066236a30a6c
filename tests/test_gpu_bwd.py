"""GPU parity of the backward (HIP kernels through the C ABI) against the fp64 oracle.

The backward takes the forward's g_cum and A (as the README's low-level API
does) and the raw q, k, v, beta, do, dht, initial state; the oracle
differentiates the token recurrence from the raw inputs alone.  Metric per
gradient: max |gpu - oracle| / rms(oracle), bar 1e-4 for fp32 inputs and
2e-2 for bf16 inputs, with dq, dk, dv requested in fp32 (dbeta, dg, dh0 are
always fp32).  A bf16 dq/dk/dv adds one rounding per element, which the
max/rms metric cannot absorb where the gradient is heavy-tailed (the last
token of a sequence takes dht directly), so bf16 gradients are checked
element-wise against |gpu - oracle| <= 2^-8 |oracle| + 1e-3 rms(oracle).
The full training shape is checked on whole (sequence, q/k head group)
units, which the oracle computes exactly on their own.
"""
import numpy as np
import pytest
import torch

import oracle
from gdr_inputs import make_inputs
from gpu_helpers import dev, gpu_inputs, host, rel, slice_units, tol

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dh0")


def run_bwd(x, with_dht=True, grad_dtype=torch.float32, fwd_states=False, fwd_cp="off",
            fwd_seg=0, fwd_ga=True, rebuild_tblocks=False, recompute_states=False, **kw):
    """The forward (g_cum and A unless not fwd_ga; with fwd_states also its
    chunk-start states and T blocks, split as fwd_cp / fwd_seg), then the backward
    (rebuild_tblocks: with the forward's states but T blocks rebuilt from A;
    recompute_states: with the forward's T blocks but the states recomputed)."""
    from gated_delta_rule_85_amd import (SavedForBackward, chunk_gated_delta_rule_bwd,
                                         chunk_gated_delta_rule_fwd)
    d = gpu_inputs(x)
    dt = d["q"].dtype
    g_cum, A, _, hb, _ = chunk_gated_delta_rule_fwd(
        d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"], d["initial_state"],
        d["cu_seqlens"], output_final_state=False, return_h=False, cp_mode=fwd_cp,
        cp_segment_chunks=fwd_seg, return_h_bwd=fwd_states, return_ga=fwd_ga)
    if fwd_states:
        kw["h_bwd"] = SavedForBackward(hb.states, None) if rebuild_tblocks else \
            SavedForBackward(None, hb.tblocks) if recompute_states else hb
    do = dev(x["do"], dt)
    dht = dev(x["dht"]) if with_dht else None
    out = chunk_gated_delta_rule_bwd(d["q"], d["k"], d["v"], g_cum, d["beta"], A, do, dht,
                                     x["scale"], d["initial_state"], d["cu_seqlens"],
                                     grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    return dict(zip(NAMES, out))



@pytest.mark.parametrize("with_dht", [True, False])
def test_no_tokens_passes_the_state_gradient_through(with_dht):
    """T = 0: the final state is the initial state, so dh0 = dht (zeros without
    it) and every other gradient is empty."""
    x = make_inputs(dict(B=2, T=0, Hq=1, Hv=2, K=64, V=64, dtype="bf16", h0=True), seed=5, grads=True)
    got = run_bwd(x, with_dht=with_dht)
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        assert got[name].numel() == 0, name
    want = x["dht"] if with_dht else np.zeros((2, 2, 64, 64))
    assert np.array_equal(host(got["dh0"]), np.asarray(want, np.float64))

def ora_bwd(x, with_dht=True):
    return oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], x["scale"],
                      initial_state=x["initial_state"], dht=x["dht"] if with_dht else None,
                      cu_seqlens=x["cu_seqlens"])


def compare(x, got, ref, t=None, names=NAMES):
    t = tol(x) if t is None else t
    errs = {}
    for n in names:
        if got.get(n) is None:
            continue
        errs[n] = rel(host(got[n]), ref[n])
    print({k: "%.3g" % v for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= t, (n, e)
    return errs


@pytest.mark.parametrize("shape", [
    dict(B=1, T=256, Hq=2, Hv=2, K=64, V=64, dtype="fp32", h0=True),
    dict(B=3, T=77, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True),
    dict(B=1, T=190, Hq=1, Hv=3, K=128, V=128, dtype="fp32", h0=True),
    dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
    dict(B=1, T=200, Hq=1, Hv=1, K=64, V=128, dtype="bf16", h0=True),
    dict(B=1, T=130, Hq=2, Hv=2, K=128, V=64, dtype="bf16", h0=False),
    dict(B=2, T=250, Hq=2, Hv=6, K=64, V=64, dtype="bf16", h0=True),
])
def test_small_ragged(shape):
    """Every element of every gradient; several chunks and a ragged tail."""
    x = make_inputs(shape, seed=2, grads=True)
    print(shape, flush=True)
    compare(x, run_bwd(x), ora_bwd(x))


@pytest.mark.parametrize("shape,L", [
    (dict(B=1, T=64 * 9 + 30, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), 2),
    (dict(B=2, T=64 * 7, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), 3),
    (dict(B=1, T=64 * 5 + 1, Hq=1, Hv=1, K=128, V=64, dtype="fp32", h0=False), 1),
    (dict(lens=[400, 0, 65, 300, 1], Hq=1, Hv=2, K=64, V=128, dtype="fp32", h0=True), 2),
    (dict(B=1, T=64 * 6, Hq=2, Hv=4, K=64, V=64, dtype="bf16", h0=True), 1),
    (dict(lens=[64] * 5 + [900, 0, 3], Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=False), 5),
])
def test_exact_split_backward(shape, L):
    """The backward's exact sequence split: the forward's split for the chunk-start
    states, and for the reverse scan each segment's start gradient from a zero end
    gradient, the carry with the transposed transitions, the scan from the true end
    gradients.  Every element of every gradient against the unsplit oracle."""
    x = make_inputs(shape, seed=12, grads=True)
    print(shape, "segments of", L, flush=True)
    compare(x, run_bwd(x, cp_mode="exact", cp_segment_chunks=L), ora_bwd(x))


@pytest.mark.parametrize("shape,fwd_cp,fwd_seg,bwd_cp,bwd_seg", [
    (dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), "off", 0, "off", 0),
    (dict(B=3, T=77, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), "off", 0, "off", 0),
    (dict(B=1, T=200, Hq=1, Hv=1, K=64, V=128, dtype="bf16", h0=False), "off", 0, "off", 0),
    (dict(B=1, T=64 * 9 + 30, Hq=1, Hv=2, K=128, V=64, dtype="fp32", h0=True), "exact", 2, "exact", 3),
    (dict(B=2, T=64 * 7, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), "exact", 3, "exact", 2),
    (dict(lens=[400, 0, 65, 300, 1], Hq=1, Hv=2, K=64, V=128, dtype="bf16", h0=True), "off", 0, "exact", 2),
    (dict(lens=[2300, 1, 0, 700, 129, 64], Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
     "auto", 0, "auto", 0),
])
def test_backward_with_forward_states(shape, fwd_cp, fwd_seg, bwd_cp, bwd_seg):
    """The forward hands its chunk-start states (h_bwd) to the backward, which then
    skips its own states pass (with a split it still forms the transitions for the
    reverse carry).  Every gradient element against the oracle, and against the
    backward that recomputes the states (same bar)."""
    x = make_inputs(shape, seed=16, grads=True)
    print(shape, fwd_cp, fwd_seg, bwd_cp, bwd_seg, flush=True)
    ref = ora_bwd(x)
    # bf16: the forward writes neither g_cum nor A, which the backward then does not read
    got = run_bwd(x, fwd_states=True, fwd_cp=fwd_cp, fwd_seg=fwd_seg, cp_mode=bwd_cp,
                  cp_segment_chunks=bwd_seg, fwd_ga=x["dtype"] != "bf16")
    compare(x, got, ref)
    # the forward's T blocks are those the backward rebuilds from A and g_cum, bit for bit
    reb = run_bwd(x, fwd_states=True, fwd_cp=fwd_cp, fwd_seg=fwd_seg, cp_mode=bwd_cp,
                  cp_segment_chunks=bwd_seg, rebuild_tblocks=True)
    for n in NAMES:
        if got[n] is not None:
            assert torch.equal(got[n], reb[n]), n
    own = run_bwd(x, cp_mode=bwd_cp, cp_segment_chunks=bwd_seg)
    t = tol(x)
    for n in NAMES:
        if got[n] is not None:
            e = rel(host(got[n]), host(own[n]).astype(np.float64))
            assert e <= t, (n, e)


@pytest.mark.parametrize("shape,cp,seg", [
    (dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), "off", 0),
    (dict(B=1, T=64 * 9 + 30, Hq=1, Hv=2, K=64, V=128, dtype="fp32", h0=True), "exact", 3),
    (dict(lens=[400, 0, 65, 300, 1], Hq=1, Hv=2, K=64, V=64, dtype="bf16", h0=True), "exact", 2),
])
def test_backward_with_forward_tblocks_only(shape, cp, seg):
    """The forward's T blocks without its states: the backward's states pass (and,
    split, its transitions) runs on the handed-over blocks; bf16 inputs without
    g_cum and A.  Every gradient element against the oracle."""
    x = make_inputs(shape, seed=17, grads=True)
    print(shape, cp, seg, flush=True)
    got = run_bwd(x, fwd_states=True, recompute_states=True, fwd_ga=x["dtype"] != "bf16",
                  cp_mode=cp, cp_segment_chunks=seg)
    compare(x, got, ora_bwd(x))


def test_forward_states_refused_with_warmup_split():
    from gated_delta_rule_85_amd import chunk_gated_delta_rule_fwd
    x = make_inputs(dict(B=1, T=256, Hq=1, Hv=1, K=64, V=64, dtype="fp32", h0=False), seed=1)
    d = gpu_inputs(x)
    with pytest.raises(ValueError):
        chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"],
                                   cp_mode="warmup", return_h_bwd=True)


def test_exact_split_backward_non_decaying_head():
    x = make_inputs(dict(B=1, T=64 * 12, Hq=1, Hv=2, K=128, V=128, dtype="fp32", h0=True), seed=13,
                    grads=True)
    x["g"][:, :, 0] = 0.0
    compare(x, run_bwd(x, cp_mode="exact", cp_segment_chunks=3), ora_bwd(x))


def test_small_head_long_sequence_backward_auto_split():
    """B=1, T=8192, H_q=2, H_v=4, bf16: B*H_v = 4 triggers the split; the auto
    backward (split) and the unsplit one both match the oracle."""
    x = make_inputs(dict(B=1, T=8192, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=14,
                    grads=True)
    ref = ora_bwd(x)
    for mode in ("auto", "off"):
        print(mode, flush=True)
        got = run_bwd(x, cp_mode=mode)
        compare(x, got, ref)


def check_rounded(got, ref, names=("dq", "dk", "dv")):
    """bf16 gradients: within one bf16 rounding of the exact value plus 1e-3 rms."""
    for n in names:
        a, b = host(got[n]), ref[n]
        bound = 2.0 ** -8 * np.abs(b) + 1e-3 * np.sqrt(np.mean(b * b))
        worst = float(np.max(np.abs(a - b) / bound))
        print(n, "worst/bound %.3g" % worst, flush=True)
        assert worst <= 1.0, (n, worst)


@pytest.mark.parametrize("shape", [
    dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
    dict(B=1, T=130, Hq=2, Hv=2, K=64, V=64, dtype="bf16", h0=False),
])
def test_bf16_gradients_within_rounding(shape):
    """The README's default: dq, dk, dv in the input dtype."""
    x = make_inputs(shape, seed=2, grads=True)
    got, ref = run_bwd(x, grad_dtype=torch.bfloat16), ora_bwd(x)
    assert got["dq"].dtype == torch.bfloat16
    check_rounded(got, ref)
    compare(x, got, ref, names=("dbeta", "dg", "dh0"))


@pytest.mark.parametrize("T", [1, 63, 64, 65])
def test_short_sequences(T):
    x = make_inputs(dict(B=2, T=T, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), seed=3,
                    grads=True)
    compare(x, run_bwd(x), ora_bwd(x))


def test_without_final_state_gradient():
    """dht = None is a zero gradient of the final state."""
    x = make_inputs(dict(B=2, T=150, Hq=2, Hv=4, K=64, V=64, dtype="fp32", h0=True), seed=4,
                    grads=True)
    compare(x, run_bwd(x, with_dht=False), ora_bwd(x, with_dht=False))


def test_varlen_with_empty_sequence():
    """Packed sequences, one of them empty: its dh0 is dht, nothing else is touched."""
    x = make_inputs(dict(lens=[70, 0, 129, 5, 64], Hq=2, Hv=4, K=128, V=64, dtype="bf16",
                         h0=True), seed=5, grads=True)
    got, ref = run_bwd(x), ora_bwd(x)
    compare(x, got, ref)
    assert np.array_equal(host(got["dh0"])[1], x["dht"][1].astype(np.float64))


def test_autograd_function_matches_low_level():
    """chunk_gated_delta_rule(...).backward() routes to the same kernels."""
    from gated_delta_rule_85_amd import chunk_gated_delta_rule
    x = make_inputs(dict(B=1, T=200, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=6,
                    grads=True)
    d = gpu_inputs(x)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta",
                                                             "initial_state")}
    o, ht = chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"],
                                   leaves["beta"], x["scale"], leaves["initial_state"],
                                   output_final_state=True)
    loss = (o * dev(x["do"])).sum() + (ht * dev(x["dht"])).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = ora_bwd(x)
    got = dict(dq=leaves["q"].grad, dk=leaves["k"].grad, dv=leaves["v"].grad,
               dbeta=leaves["beta"].grad, dg=leaves["g"].grad, dh0=leaves["initial_state"].grad)
    assert got["dq"].dtype == torch.bfloat16
    check_rounded(got, ref)
    compare(x, got, ref, names=("dbeta", "dg", "dh0"))


def test_autograd_small_heads_long_sequence_splits_exactly():
    """B*H_v = 2 and 40 chunks: the trigger fires, so the differentiable API runs
    the forward's exact split and the backward's; o and every gradient against the
    oracle (fp32 inputs, bar 1e-4)."""
    from gated_delta_rule_85_amd import chunk_gated_delta_rule
    x = make_inputs(dict(B=1, T=64 * 40 - 7, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), seed=15,
                    grads=True)
    d = gpu_inputs(x)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta",
                                                             "initial_state")}
    o, ht = chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"],
                                   leaves["beta"], x["scale"], leaves["initial_state"],
                                   output_final_state=True)
    loss = (o * dev(x["do"])).sum() + (ht * dev(x["dht"])).sum()
    loss.backward()
    torch.cuda.synchronize()
    fwd = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"])
    e_o = rel(host(o.detach()), fwd["o"])
    print("o %.3g" % e_o, flush=True)
    assert e_o <= 1e-4
    got = dict(dq=leaves["q"].grad, dk=leaves["k"].grad, dv=leaves["v"].grad,
               dbeta=leaves["beta"].grad, dg=leaves["g"].grad, dh0=leaves["initial_state"].grad)
    compare(x, got, ora_bwd(x))


def test_training_shape_full_size_every_unit_bf16():
    """B=8, T=4096, H_q=32, H_v=64, K=V=128, bf16, as the training step runs it
    (chunk-start states and T blocks handed over by the forward, no A or g_cum) with
    the README's bf16 dq, dk, dv: every element of every gradient of all 512
    (sequence, v head) units against the oracle, dq/dk/dv within one bf16 rounding,
    dbeta/dg/dh0 at the bar."""
    x = make_inputs("training", seed=0)
    got = run_bwd(x, fwd_states=True, fwd_ga=False, grad_dtype=torch.bfloat16)
    assert got["dq"].dtype == torch.bfloat16
    got = {n: host(t) for n, t in got.items()}
    torch.cuda.empty_cache()
    ref = ora_bwd(x)
    check_rounded(got, ref)
    compare(x, got, ref, names=("dbeta", "dg", "dh0"))


def test_training_shape_recomputed_states_sampled_units():
    """The same shape with the backward recomputing the chunk-start states and
    rebuilding the T blocks from the forward's g_cum and A (fp32 gradients): four
    (sequence, q/k head) units against the oracle."""
    x = make_inputs("training", seed=0)
    got = run_bwd(x)
    for b, hq in [(0, 0), (3, 17), (5, 9), (7, 31)]:
        y, hs = slice_units(x, b, hq)
        y["do"] = x["do"][b:b + 1, :, hs]
        y["dht"] = x["dht"][b:b + 1, hs]
        ref = ora_bwd(y)
        sub = dict(dq=got["dq"][b:b + 1, :, hq:hq + 1], dk=got["dk"][b:b + 1, :, hq:hq + 1],
                   dv=got["dv"][b:b + 1, :, hs], dbeta=got["dbeta"][b:b + 1, :, hs],
                   dg=got["dg"][b:b + 1, :, hs], dh0=got["dh0"][b:b + 1, hs])
        print((b, hq), end=" ")
        compare(y, sub, ref)


def test_varlen_packed_batch_full_size():
    """16 packed sequences (61,412 tokens, lengths 129 to 11,956), H_q=16, H_v=32,
    K=V=128, bf16, as a training step runs it (states and T blocks from the
    forward, sequences scanned longest first): every element of every gradient,
    all 16 q/k heads, against the oracle."""
    x = make_inputs("varlen", seed=0, grads=True)
    got = run_bwd(x, fwd_states=True, fwd_ga=False)
    compare(x, got, ora_bwd(x), names=("dq", "dk", "dv", "dbeta", "dg"))


def test_strong_decay_past_fp32_exp_range():
    """Gates eight times the recipe's: the in-chunk running log-gate spans past the
    fp32 range of exp (about -200 over a chunk).  Every element of every gradient,
    bf16 and fp32 inputs, ragged tails."""
    for shape in (dict(B=2, T=300, Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
                  dict(B=1, T=190, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True)):
        x = make_inputs(shape, seed=14, grads=True)
        x["g"] = (x["g"] * 8.0).astype(np.float32)
        print(shape["dtype"], end=" ")
        compare(x, run_bwd(x), ora_bwd(x))


def test_long_sequence_full_size_split_with_forward_states():
    """B=1, T=32768, H_q=4, H_v=8, K=V=128, bf16 (512 chunks per head), as a training
    step runs it: the forward's exact split writes the states and T blocks, and the
    backward's own exact split (the device model's segment length) forms only the
    transitions for its reverse carry.  Every gradient element against the oracle."""
    x = make_inputs("small_head_long", seed=0, grads=True)
    got = run_bwd(x, fwd_states=True, fwd_ga=False, fwd_cp="auto_exact", cp_mode="auto")
    compare(x, got, ora_bwd(x))


def test_varlen_mixed_lengths_bf16():
    """Packed batch with lengths from 1 to ~2.3k tokens (ragged tails, single-token
    and empty sequences), the GQA shape of the workloads; every gradient element."""
    x = make_inputs(dict(lens=[2300, 1, 0, 700, 129, 64, 1500], Hq=2, Hv=4, K=128, V=128,
                         dtype="bf16", h0=True), seed=7, grads=True)
    compare(x, run_bwd(x), ora_bwd(x))


def test_fp32_inputs_longer_sequence():
    """fp32 inputs (fp32-MFMA kernels) over 1000 tokens with K = V = 128."""
    x = make_inputs(dict(B=1, T=1000, Hq=1, Hv=2, K=128, V=128, dtype="fp32", h0=True), seed=8,
                    grads=True)
    compare(x, run_bwd(x), ora_bwd(x))


def test_varlen_autograd_step_without_host_sync():
    """A differentiable varlen step (forward handing its states and T blocks to the
    backward, offsets on the device) makes no host synchronisation: torch's sync
    debug mode raises on any .cpu(), .item() or blocking copy on the path."""
    from gated_delta_rule_85_amd import chunk_gated_delta_rule
    x = make_inputs(dict(lens=[300, 1, 0, 700, 129], Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True),
                    seed=17, grads=True)
    d = gpu_inputs(x)
    leaves = {n: d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta",
                                                             "initial_state")}
    do, dht = dev(x["do"]), dev(x["dht"])
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        o, ht = chunk_gated_delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["beta"],
                                       x["scale"], leaves["initial_state"], output_final_state=True,
                                       cu_seqlens=d["cu_seqlens"])
        loss = (o * do).sum() + (ht * dht).sum()
        loss.backward()
    finally:
        torch.cuda.set_sync_debug_mode(0)
    torch.cuda.synchronize()
    ref = ora_bwd(x)
    got = dict(dq=leaves["q"].grad, dk=leaves["k"].grad, dv=leaves["v"].grad,
               dbeta=leaves["beta"].grad, dg=leaves["g"].grad, dh0=leaves["initial_state"].grad)
    check_rounded(got, ref)
    compare(x, got, ref, names=("dbeta", "dg", "dh0"))
