#!/usr/bin/env python3
"""Throughput of the gated delta rule chunked-prefill forward on one MI355X.

One step is one gdr_fwd call (gdr_chunk_prep + the fused scan/output kernel)
over the full-width prefill shard: B=4, T=4096, H_q=16, H_v=32, K=V=128,
bf16 q/k/v, fp32 g/beta/initial and final state, fp32 o (inference forward:
the A and g_cum tensors a backward would need are not written).  Inputs are seeded
synthetic tensors already resident in HBM; W untimed warm-up steps, then K
timed steps between stream synchronisations.  Each step records HIP events
around each kernel on the library's stream; the dominant kernel's average
duration gives the roofline entry.  The fp64 CPU oracle is timed on a bounded
sample of the same workload for the cpu_baseline entry.

Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunked-prefill fwd tokens/s + % of bf16 MFMA peak, H_v=32 K=V=128 T=4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
F_TRI = 139264                  # algorithmic flop per token per v head (C=64, K=V=128)
STAGES = ("gdr_chunk_prep", "gdr_scan_output", "gdr_wu")


TBLOCK = 17408  # bytes of one (chunk, v head) T block: T hi/lo planes + gate scalars


def algorithmic_bytes(cfg, out_bytes=4):
    """Bytes each kernel must move once per launch in this design (every
    tensor it reads or writes counted once; q/k shared by the v heads of a
    group; one T block per chunk and v head between the two kernels)."""
    B, T, Hq, Hv, K, V = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hv"], cfg["K"], cfg["V"]
    e = 2 if cfg["dtype"] == "bf16" else 4
    tok = B * T
    qk = tok * Hq * K * e
    vv = tok * Hv * V * e
    gate = tok * Hv * 4
    blocks = B * ((T + 63) // 64) * Hv * TBLOCK
    state = B * Hv * K * V * 4
    o = tok * Hv * V * out_bytes
    prep = qk + 2 * gate + blocks                  # k, g, beta -> T blocks
    scan = 2 * qk + vv + blocks + o + (2 * state if cfg.get("h0") else state)
    return {"gdr_chunk_prep": prep, "gdr_scan_output": scan}


def source_hash():
    h = hashlib.sha256()
    for f in ("gdr_scan.hip", "gdr_prep.hip", "gdr_device.hpp"):
        with open(os.path.join(ROOT, "gated_delta_rule_85_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None.  The summary's last
    line is a JSON object with source_hash and bytes_per_launch."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.loads(f.read().strip().splitlines()[-1])
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(x, seconds):
    """Time the fp64 oracle on whole sequences of the workload until about
    `seconds` of CPU time have been spent."""
    import numpy as np

    import oracle
    B = x["q"].shape[0]
    T = x["q"].shape[1]
    done = 0
    elapsed = 0.0
    threads = 0
    for b in range(B):
        sl = {n: np.ascontiguousarray(x[n][b:b + 1], dtype=np.float64)
              for n in ("q", "k", "v", "g", "beta")}
        h0 = None if x["initial_state"] is None else \
            np.ascontiguousarray(x["initial_state"][b:b + 1], dtype=np.float64)
        t0 = time.perf_counter()
        oracle.fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], x["scale"], h0)
        elapsed += time.perf_counter() - t0
        threads = oracle.last_threads()
        done += 1
        if elapsed >= seconds:
            break
    return {"value": done * T / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d sequences (all %d v heads, T=%d) in %.1f s" %
                      (done, B, x["v"].shape[2], T, elapsed)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_shard")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this operator has no multi-GPU path here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from gated_delta_rule_85_amd import _lib
    from gdr_inputs import make_inputs

    x = make_inputs(args.workload, seed=0)
    cfg = x["cfg"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    put = lambda a, t=torch.float32: None if a is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)
    q, k, v = put(x["q"], dt), put(x["k"], dt), put(x["v"], dt)
    g, beta, h0 = put(x["g"]), put(x["beta"]), put(x["initial_state"])
    cu = put(x["cu_seqlens"], torch.int32)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    n_seq = B if cu is None else cu.numel() - 1
    o = torch.empty((B, T, Hv, V), dtype=torch.float32, device=dev)
    ht = torch.empty((n_seq, Hv, K, V), dtype=torch.float32, device=dev)

    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, n_seq
    a.dtype = _lib.BF16 if dt == torch.bfloat16 else _lib.F32
    a.out_dtype = _lib.F32
    a.scale = float(x["scale"])
    a.cp_mode = _lib.CP_AUTO
    a.q, a.k, a.v, a.g, a.beta = q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr()
    a.initial_state = None if h0 is None else h0.data_ptr()
    a.cu_seqlens = None if cu is None else cu.data_ptr()
    # inference forward: o and the final state (the backward's A and g_cum are not written)
    a.o, a.final_state = o.data_ptr(), ht.data_ptr()
    nbytes = _lib.fwd_workspace(a)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes

    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    nev = 2 * _lib.FWD_STAGES
    ev_arrays = []
    for _ in range(args.steps):
        arr = (ctypes.c_void_p * nev)()
        for i in range(nev):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = e.value
        ev_arrays.append(arr)

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    a.events = None
    for _ in range(args.warmup):
        _lib.fwd(a, sh)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        a.events = ctypes.addressof(ev_arrays[i])
        _lib.fwd(a, sh)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps

    stage_ms = {}
    f = ctypes.c_float()
    for s, name in enumerate(STAGES):
        tot = 0.0
        for arr in ev_arrays:
            if hip.hipEventElapsedTime(ctypes.byref(f), arr[2 * s], arr[2 * s + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            tot += f.value
        stage_ms[name] = tot / args.steps
    for arr in ev_arrays:
        for i in range(nev):
            hip.hipEventDestroy(arr[i])

    tokens = B * T
    value = tokens / (ms * 1e-3)
    tflops = F_TRI * tokens * Hv / (ms * 1e-3) / 1e12
    ab = algorithmic_bytes(dict(cfg, B=B, T=T), out_bytes=4)
    dom = max(ab, key=lambda kname: stage_ms[kname])
    achieved = ab[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(dom, args.workload)
    rec = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": "%s: B=%d T=%d H_q=%d H_v=%d K=%d V=%d, %s q/k/v, fp32 g/beta/state/o"
                               % (args.workload, B, T, Hq, Hv, K, V, x["dtype"]),
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "tflops_algorithmic": tflops,
        "mfma_bf16_peak_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
        "kernel_ms": stage_ms,
        "wall_ms_per_step": t_wall * 1e3 / args.steps,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": ab[dom]},
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
