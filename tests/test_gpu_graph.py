"""gdr_fwd and gdr_fwd_noalloc captured into a HIP graph (through torch's graph
capture) and replayed, against the same calls made eagerly.

The library launches its kernels on the caller's stream and records nothing
else on it when no timing events are passed, so a caller can capture a call.
Each graph is replayed three times; before every replay the test refills the
outputs with NaN and, for the second and third, writes new values into v, runs
the eager call on the new inputs into separate outputs and synchronises.  Every
replay must reproduce the eager result of the same inputs bit for bit (the
same kernels on the same data).  Cases: packed sequences under the exact
sequence split (several kernels per stage: a fill, transition and state scans,
the carry) and a plain batch in fp32.
"""
import ctypes

import pytest
import torch

from gdr_inputs import make_inputs
from gpu_helpers import gpu_inputs

pytestmark = pytest.mark.gpu


def make_args(d, o, ht, x, cp_mode, seg):
    from gated_delta_rule_85_amd import _lib
    B, T, Hq, K = d["q"].shape
    Hv, V = d["v"].shape[2], d["v"].shape[3]
    cu = d["cu_seqlens"]
    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V = B, T, Hq, Hv, K, V
    a.n_seq = B if cu is None else cu.numel() - 1
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
    return a


def call(a, noalloc, ws):
    from gated_delta_rule_85_amd import _lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        rc = _lib.lib.gdr_fwd_noalloc(ctypes.byref(a), stream)
    else:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        rc = _lib.lib.gdr_fwd(ctypes.byref(a), stream)
    assert rc == 0, _lib.strerror(rc)


def outputs(d):
    B, T, Hq, K = d["q"].shape
    Hv, V = d["v"].shape[2], d["v"].shape[3]
    n_seq = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    return (torch.full((B, T, Hv, V), float("nan"), device="cuda"),
            torch.full((n_seq, Hv, K, V), float("nan"), device="cuda"))


CASES = [
    ("packed_exact_split", dict(lens=[700, 0, 129, 300], Hq=2, Hv=4, K=128, V=128, dtype="bf16", h0=True), "exact", 3),
    ("batch_fp32", dict(B=2, T=200, Hq=2, Hv=4, K=64, V=64, dtype="fp32", h0=True), "off", 0),
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("name,spec,mode,seg", CASES, ids=[c[0] for c in CASES])
def test_captured_forward_replays_match_eager_calls(name, spec, mode, seg, noalloc):
    from gated_delta_rule_85_amd import _lib
    cp = {"exact": _lib.CP_EXACT, "off": _lib.CP_OFF}[mode]
    x = make_inputs(spec, seed=41)
    d = gpu_inputs(x)
    o_g, h_g = outputs(d)  # the graph's outputs
    o_e, h_e = outputs(d)  # the eager calls' outputs
    a_g = make_args(d, o_g, h_g, x, cp, seg)
    a_e = make_args(d, o_e, h_e, x, cp, seg)
    need = _lib.fwd_workspace(a_g)
    assert need <= _lib.SCRATCH_BYTES
    ws_g = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    # an eager call first (the allocation-free entry point takes its scratch address
    # on its first call on a device, which is not a call a graph can hold)
    call(a_e, noalloc, ws_e)
    torch.cuda.synchronize()
    print("%s (%s): capture" % (name, "noalloc" if noalloc else "workspace"), flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(a_g, noalloc, ws_g)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        if rep > 0:
            # new values, same buffers: v is what the captured kernels read
            d["v"].copy_(torch.randn(d["v"].shape, device="cuda", generator=gen).to(d["v"].dtype))
        o_g.fill_(float("nan"))
        h_g.fill_(float("nan"))
        o_e.fill_(float("nan"))
        h_e.fill_(float("nan"))
        call(a_e, noalloc, ws_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("%s replay %d" % (name, rep), flush=True)
        assert not torch.isnan(h_e).any()
        assert torch.equal(o_g, o_e), (name, rep, (o_g - o_e).abs().nan_to_num(1e30).max().item())
        assert torch.equal(h_g, h_e), (name, rep)
    del graph
