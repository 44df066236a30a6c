"""GPU parity on the full-size workloads (sampled units) and the sequence split.

Every launch covers the whole workload; the fp64 oracle recomputes whole
(sequence, q/k-head group) units, exact because units are independent.
"""
import numpy as np
import pytest

import oracle
from gdr_inputs import make_inputs
from gpu_helpers import host, rel, run_fwd, slice_units

pytestmark = pytest.mark.gpu


def test_varlen_packed_batch_full_size():
    """16 packed sequences (61,412 tokens, seed-0 lengths), H_q=16, H_v=32,
    K=V=128, bf16, zero initial states, per-sequence final states: every element
    of o and of every final state, all 16 q/k heads."""
    x = make_inputs("varlen", seed=0)
    g_cum, A, o, h, ht = run_fwd(x, return_h=False)
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], cu_seqlens=x["cu_seqlens"])
    eo, eh = rel(host(o), r["o"]), rel(host(ht), r["final_state"])
    print("o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


def test_training_shape_forward_full_size():
    """B=8, T=4096, H_q=32, H_v=64, K=V=128, bf16 with initial state (forward part):
    every element of o and of the final states, all 512 (sequence, v head) units."""
    x = make_inputs("training", seed=0, grads=False)
    g_cum, A, o, h, ht = run_fwd(x, return_h=False)
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"])
    eo, eh = rel(host(o), r["o"]), rel(host(ht), r["final_state"])
    print("o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


@pytest.mark.parametrize("Hv", [64, 48, 24, 16])
def test_family_head_counts(Hv):
    """The head counts the pages benchmark (64 to 8, TP1 to TP8) with H_q = H_v / 2,
    B=2, T=2048, bf16, launched whole; two (sequence, q/k head) units sampled."""
    x = make_inputs(dict(B=2, T=2048, Hq=Hv // 2, Hv=Hv, K=128, V=128, dtype="bf16", h0=True), seed=16)
    g_cum, A, o, h, ht = run_fwd(x, return_h=False)
    o, ht = host(o), host(ht)
    for b, hq in ((0, 0), (1, Hv // 2 - 1)):
        y, hs = slice_units(x, b, hq)
        r = oracle.fwd(y["q"], y["k"], y["v"], y["g"], y["beta"], y["scale"], y["initial_state"])
        eo, eh = rel(o[b:b + 1, :, hs], r["o"]), rel(ht[b:b + 1, hs], r["final_state"])
        print("H_v=%d b=%d hq=%d o %.3g final %.3g" % (Hv, b, hq, eo, eh), flush=True)
        assert eo <= 2e-2 and eh <= 2e-2


@pytest.fixture(scope="module")
def long_seq():
    """B=1, T=32768, H_q=4, H_v=8, K=V=128, bf16: 512 chunks per head."""
    return make_inputs("small_head_long", seed=0)


def test_long_sequence_exact_scan(long_seq):
    x = long_seq
    o = host(run_fwd(x, return_h=False, cp_mode="off")[2])
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    e = rel(o, r["o"])
    print("exact o %.3g" % e, flush=True)
    assert e <= 2e-2


@pytest.mark.parametrize("wm", [6, 7, 8])
def test_long_sequence_warmup_split(long_seq, wm):
    """Segments of L = ceil(sqrt(512)) = 23 chunks, each warmed up over wm chunks
    from a zero state; compared with the oracle of the same split (the bar), and
    the split's own deviation from the exact result reported separately."""
    x = long_seq
    L = 23
    _, _, o, _, ht = run_fwd(x, return_h=False, cp_mode="warmup", cp_segment_chunks=L,
                             cp_warmup_chunks=wm)
    o, ht = host(o), host(ht)
    rs = oracle.fwd_split(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], L, wm)
    re = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    e_split, e_final = rel(o, rs["o"]), rel(ht, rs["final_state"])
    e_vs_exact = rel(o, re["o"])
    e_method = rel(rs["o"], re["o"])
    print("wm=%d gpu-vs-split %.3g final %.3g | gpu-vs-exact %.3g | split-vs-exact (fp64) %.3g"
          % (wm, e_split, e_final, e_vs_exact, e_method), flush=True)
    assert e_split <= 2e-2 and e_final <= 2e-2
    assert e_vs_exact <= 2e-2  # decaying gates: the split meets the same bar


def split_chunks(N, W, slots, wm):
    """Segment length of the device model for the warm-up split: the segment count
    S (up to eight rounds of the device) minimising ceil(W S / slots) * (L + wm),
    L = ceil(N / S), fewer segments on ties."""
    best = None
    for S in range(1, min(N, 8 * -(-slots // W)) + 1):
        L = -(-N // S)
        if -(-N // L) != S:
            continue
        t = -(-W * S // slots) * (L + (wm if S > 1 else 0))
        if best is None or t < best[0]:
            best = (t, L if S > 1 else N + 1)
    return best[1]


def test_segment_model_values():
    # 8 v heads x 2 value blocks over 512 chunks on 256 CUs: 16 segments of 32 fill
    # the device once; the full-width shard (256 workgroups) is not split
    assert split_chunks(512, 16, 256, 8) == 32
    assert split_chunks(64, 256, 256, 8) == 65


def test_auto_mode_splits_the_long_sequence(long_seq):
    """AutoCP on the 32K-token sequence: "auto" splits with the device model's
    segment length (the window priced at one chunk) and a gate-driven window.  The workload's gates decay by far
    more than 2^-24 within every chunk, so each window is one chunk: the result
    is bitwise that of the fixed one-chunk warm-up.  "auto_pages" (the pages'
    trigger, B*H_v = 8 <= 40) is the fixed 8-chunk warm-up."""
    import torch
    x = long_seq
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = split_chunks(512, 8 * 2, cus, 1)
    Lp = split_chunks(512, 8 * 2, cus, 8)
    print("compute units %d: segments of %d (auto) and %d (auto_pages) chunks" % (cus, L, Lp), flush=True)
    auto = host(run_fwd(x, return_h=False, cp_mode="auto")[2])
    forced = host(run_fwd(x, return_h=False, cp_mode="warmup", cp_segment_chunks=L,
                          cp_warmup_chunks=1)[2])
    assert np.array_equal(auto, forced)
    pages = host(run_fwd(x, return_h=False, cp_mode="auto_pages")[2])
    forced8 = host(run_fwd(x, return_h=False, cp_mode="warmup", cp_segment_chunks=Lp,
                           cp_warmup_chunks=8)[2])
    assert np.array_equal(pages, forced8)
    re = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    e, ep = rel(auto, re["o"]), rel(pages, re["o"])
    print("auto split vs exact %.3g, auto_pages %.3g" % (e, ep), flush=True)
    assert e <= 2e-2 and ep <= 2e-2


def test_auto_mode_with_gates_that_do_not_decay():
    """"auto" on heads whose gates do not decay (g = 0), beside a decaying head and
    one that decays slowly: the gate-driven window reaches back to the sequence
    start where it must, so every head meets the bar against the exact oracle,
    while the fixed 8-chunk warm-up of the pages' trigger does not."""
    x = make_inputs(dict(B=1, T=64 * 40 - 9, Hq=1, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=21)
    x["g"][:, :, 1] = 0.0
    x["g"][:, :, 2] = (x["g"][:, :, 2] * 0.02).astype(np.float32)
    ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"])
    _, _, o, _, ht = run_fwd(x, return_h=False, cp_mode="auto")
    o, ht = host(o), host(ht)
    off = host(run_fwd(x, return_h=False, cp_mode="off")[2])
    pages = host(run_fwd(x, return_h=False, cp_mode="auto_pages")[2])
    for hv in range(4):
        eo = rel(o[:, :, hv], ref["o"][:, :, hv])
        eh = rel(ht[:, hv], ref["final_state"][:, hv])
        print("head %d: auto o %.3g final %.3g | off %.3g | auto_pages %.3g" % (
            hv, eo, eh, rel(off[:, :, hv], ref["o"][:, :, hv]), rel(pages[:, :, hv], ref["o"][:, :, hv])),
            flush=True)
        assert eo <= 2e-2 and eh <= 2e-2
    assert rel(pages[:, :, 1], ref["o"][:, :, 1]) > 2e-2


def test_long_sequence_exact_split(long_seq):
    """The exact split (segment transitions, serial carry, second pass) on the
    32K-token sequence with the device's segment length: the exact result."""
    x = long_seq
    _, _, o, _, ht = run_fwd(x, return_h=False, cp_mode="exact")
    o, ht = host(o), host(ht)
    re = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    eo, eh = rel(o, re["o"]), rel(ht, re["final_state"])
    print("exact split: o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2


@pytest.mark.parametrize("scale_g", [0.03, 0.01])
def test_weak_decay_split_diagnostic(scale_g):
    """Weak gates (g scaled down): the warm-up error becomes visible.  Reported,
    and the GPU must still match the oracle of the same split."""
    x = make_inputs(dict(B=1, T=64 * 48, Hq=1, Hv=2, K=128, V=128, dtype="bf16", h0=False), seed=0)
    x["g"] = (x["g"] * scale_g).astype(np.float32)
    L, wm = 7, 8
    o = host(run_fwd(x, return_h=False, cp_mode="warmup", cp_segment_chunks=L,
                     cp_warmup_chunks=wm)[2])
    rs = oracle.fwd_split(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], L, wm)
    re = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"])
    print("g x %.2f: split-vs-exact (fp64) %.3g, gpu-vs-split %.3g"
          % (scale_g, rel(rs["o"], re["o"]), rel(o, rs["o"])), flush=True)
    assert rel(o, rs["o"]) <= 2e-2


@pytest.mark.parametrize("B,T,Hv", [(4, 1024, 64), (2, 2048, 16), (1, 64 * 40, 2)])
def test_auto_rule(B, T, Hv):
    """The device rule of "auto": the segment length minimising rounds x (L + 1) over
    the compute units (the gate-driven window priced at one chunk).  Where it keeps
    one segment (4 x 1024 at 64 heads: 512 workgroups already take two rounds) the
    output is bitwise the unsplit scan's; where it splits, the workload's gates decay
    below 2^-24 within one chunk, so the output is bitwise the one-chunk warm-up of
    that length; both against the oracle at the bar."""
    import torch
    x = make_inputs(dict(B=B, T=T, Hq=max(1, Hv // 2), Hv=Hv, K=128, V=128, dtype="bf16", h0=True), seed=22)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = -(-T // 64)
    L = split_chunks(N, B * Hv * 2, cus, 1)
    auto = host(run_fwd(x, return_h=False, cp_mode="auto")[2])
    if L > N:
        same = host(run_fwd(x, return_h=False, cp_mode="off")[2])
    else:
        same = host(run_fwd(x, return_h=False, cp_mode="warmup", cp_segment_chunks=L, cp_warmup_chunks=1)[2])
    print("%d x %d, H_v=%d: %s" % (B, T, Hv, "no split" if L > N else "segments of %d chunks" % L), flush=True)
    assert np.array_equal(auto, same)
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"])
    e = rel(auto, r["o"])
    print("auto vs exact %.3g" % e, flush=True)
    assert e <= 2e-2
