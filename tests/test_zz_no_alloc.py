"""gdr_fwd_noalloc (the forward on the library's static per-device scratch) through
the C ABI, against gdr_fwd on a caller workspace and against the fp64 oracle.

Three calls in a row, each smaller than the one before, so that every call runs
on scratch holding the previous call's data: the prefill shard at full size
(B=4, T=4096, H_q=16, H_v=32, K=V=128, bf16), packed sequences with an empty one
under the exact sequence split (its transitions and states also live in the
scratch), and a short fp32 problem.  The two entry points run the same kernels,
so their outputs must agree bit for bit; the oracle holds both to the bar
(2e-2 for bf16 inputs, 1e-4 for fp32).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gdr_inputs import make_inputs
from gpu_helpers import gpu_inputs, host, rel, slice_units, tol

pytestmark = pytest.mark.gpu


def run(x, noalloc, cp_mode, seg=0):
    from gated_delta_rule_85_amd import _lib
    d = gpu_inputs(x)
    B, T, Hq, K = d["q"].shape
    Hv, V = d["v"].shape[2], d["v"].shape[3]
    cu = d["cu_seqlens"]
    n_seq = B if cu is None else cu.numel() - 1
    o = torch.full((B, T, Hv, V), float("nan"), device="cuda")
    ht = torch.full((n_seq, Hv, K, V), float("nan"), device="cuda")
    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, n_seq
    a.dtype = _lib.BF16 if x["dtype"] == "bf16" else _lib.F32
    a.out_dtype = _lib.F32
    a.scale = float(x["scale"])
    a.cp_mode = cp_mode
    a.cp_segment_chunks = seg
    a.q, a.k, a.v = d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr()
    a.g, a.beta = d["g"].data_ptr(), d["beta"].data_ptr()
    a.initial_state = None if d["initial_state"] is None else d["initial_state"].data_ptr()
    a.cu_seqlens = None if cu is None else cu.data_ptr()
    a.o, a.final_state = o.data_ptr(), ht.data_ptr()
    need = _lib.fwd_workspace(a)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        assert need <= _lib.SCRATCH_BYTES
        print("gdr_fwd_noalloc: %d bytes of scratch" % need, flush=True)
        rc = _lib.lib.gdr_fwd_noalloc(ctypes.byref(a), ctypes.c_void_p(stream))
    else:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), need
        rc = _lib.lib.gdr_fwd(ctypes.byref(a), ctypes.c_void_p(stream))
    assert rc == 0, _lib.strerror(rc)
    torch.cuda.synchronize()
    return o, ht


def test_noalloc_matches_the_workspace_forward_on_calls_of_decreasing_size():
    from gated_delta_rule_85_amd import _lib
    # 1: the prefill shard, unsplit (T blocks fill 109 MB of the scratch)
    x = make_inputs("prefill_shard", seed=0)
    o_n, h_n = run(x, True, _lib.CP_OFF)
    o_w, h_w = run(x, False, _lib.CP_OFF)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    y, hs = slice_units(x, 2, 5)
    r = oracle.fwd(y["q"], y["k"], y["v"], y["g"], y["beta"], y["scale"], y["initial_state"])
    eo, eh = rel(host(o_n)[2:3, :, hs], r["o"]), rel(host(h_n)[2:3, hs], r["final_state"])
    print("prefill shard (b=2, hq=5): o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= 2e-2 and eh <= 2e-2
    del o_n, h_n, o_w, h_w
    # 2: packed sequences (one empty) under the exact split, smaller
    x = make_inputs(dict(lens=[700, 0, 129, 300], Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), seed=31)
    o_n, h_n = run(x, True, _lib.CP_EXACT, 3)
    o_w, h_w = run(x, False, _lib.CP_EXACT, 3)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"],
                   cu_seqlens=x["cu_seqlens"])
    eo, eh = rel(host(o_n), r["o"]), rel(host(h_n), r["final_state"])
    print("packed, exact split: o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= tol(x) and eh <= tol(x)
    # 3: a short fp32 problem, smaller still
    x = make_inputs(dict(B=1, T=77, Hq=1, Hv=2, K=64, V=64, dtype="fp32", h0=True), seed=32)
    o_n, h_n = run(x, True, _lib.CP_AUTO)
    o_w, h_w = run(x, False, _lib.CP_AUTO)
    assert torch.equal(o_n, o_w) and torch.equal(h_n, h_w)
    r = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["initial_state"])
    eo, eh = rel(host(o_n), r["o"]), rel(host(h_n), r["final_state"])
    print("fp32: o %.3g final %.3g" % (eo, eh), flush=True)
    assert eo <= tol(x) and eh <= tol(x)
