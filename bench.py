#!/usr/bin/env python3
"""Throughput of the gated delta rule chunked-prefill forward on one MI355X.

One step is one gdr_fwd call (gdr_chunk_prep + the fused scan/output kernel)
over the full-width prefill shard: B=4, T=4096, H_q=16, H_v=32, K=V=128,
bf16 q/k/v, fp32 g/beta/initial and final state, fp32 o (inference forward:
the A and g_cum tensors a backward would need are not written).  Inputs are seeded
synthetic tensors already resident in HBM; W untimed warm-up steps,
breakdown passes (K steps per stage, handing the library only that stage's
two HIP events: kernel_ms and the dominant kernel; one more pass with every
event: breakdown_step_ms), then K timed steps between stream
synchronisations, in which only the dominant kernel's two events are handed
over.  The library binds a stage's events to its kernel launches.  The start
event is taken when the stream reaches the stage's first launch, so a stage's
time also holds the gap before that kernel starts (about 2-5 microseconds on
MI355X; rocprofv3's kernel statistics give the kernels' own durations); a
stage that launches nothing records both on the stream, which costs it a few
microseconds.  The dominant kernel's average
duration over the timed steps gives the roofline entry.  The fp64 CPU oracle is timed on a bounded
sample of the same workload for the cpu_baseline entry.

``--workload training`` instead times one training step of the operator:
gdr_fwd (exact scan, handing the backward its chunk-start states and T blocks)
followed by gdr_bwd (dq, dk, dv in bf16; dbeta, dg, dh0 in fp32) at B=8,
T=4096, H_q=32, H_v=64, K=V=128, with upstream gradients do and dht
(``--recompute-states``: the forward writes g_cum and A instead, from which the
backward rebuilds the T blocks and recomputes the states).

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


TBLOCK = 13312  # bytes of one (chunk, v head) forward T block: T hi/lo planes (rows 0-31 at half width) + scalars


def minimal_bytes_per_token_head(cfg, out_bytes=None):
    """Least HBM bytes the forward must move per token and v head: q and k read
    once (each shared by the H_v/H_q v heads of its group), v, g and beta read, o
    written in the input dtype (out_bytes: another output width), and the initial
    and final states amortised over the sequence.  808 B at K=V=128, G=2, T=4096,
    bf16 with an initial state."""
    Hq, Hv, K, V = cfg["Hq"], cfg["Hv"], cfg["K"], cfg["V"]
    tokens = cfg["B"] * cfg["T"]
    n_seq = cfg.get("n_seq", cfg["B"])
    e = 2 if cfg["dtype"] == "bf16" else 4
    eo = e if out_bytes is None else out_bytes
    G = Hv // Hq
    states = (2 if cfg.get("h0") else 1) * K * V * 4 * n_seq / tokens
    return 2 * K * e / G + V * e + 8 + V * eo + states


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


BWD_STAGES = ("gdr_bwd_tblocks", "gdr_bwd_states", "gdr_bwd_scan", "gdr_bwd_local")
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix


def bwd_algorithmic_flops(cfg):
    """Flops each backward kernel must do per launch: the dense products of
    the chunked adjoint at C=64 (counted once per (chunk, v head); K K^T once
    per (chunk, q/k head)), not what the tiling recomputes."""
    B, T, Hq, Hv, K, V = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hv"], cfg["K"], cfg["V"]
    C = 64
    units = B * ((T + C - 1) // C) * Hv
    cc_k, cc_v, ckv = 2 * C * C * K, 2 * C * C * V, 2 * C * K * V
    # reverse scan: P, K dh', P^T dO, T^T dU, Q^T(e dO), K^T(b e dX)
    scan = units * (cc_k + ckv + 2 * cc_v + 2 * ckv)
    # local: P, Kh, Qh, K dh', T X, P^T dO, T^T dU, dO U^T, dU X^T, three K x V
    # products into dq/dk, T^T dT T^T, and (dP*Gam) K, (dP*Gam)^T Q, dS K
    local = units * (cc_k + 3 * ckv + 5 * cc_v + 3 * ckv + 2 * 2 * C ** 3 + 3 * cc_k) \
        + B * ((T + C - 1) // C) * Hq * cc_k
    states = units * (2 * ckv + cc_v)  # K h, T X, K^T U
    return {"gdr_bwd_scan": scan, "gdr_bwd_local": local, "gdr_bwd_states": states}


# sources of the forward kernels and of the backward's chunk-local kernel: a
# traffic summary counts only if taken on these
FWD_SOURCES = ("gdr_scan.hip", "gdr_prep.hip", "gdr_device.hpp", "gdr_layout.hpp", "gdr_lds.hpp",
               "gdr_kernels.hpp")
BWD_LOCAL_SOURCES = ("gdr_bwd_mfma.hip", "gdr_bwd_ops.hpp", "gdr_device.hpp", "gdr_layout.hpp",
                     "gdr_lds.hpp", "gdr_kernels.hpp")


def source_hash(files=FWD_SOURCES):
    """Hash of the code of the given kernel sources: line comments and blank
    lines are dropped (the sources hold no block comments and no "//" inside
    a string), so a change to the comments alone keeps the hash."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_delta_rule_85_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
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
    files = BWD_LOCAL_SOURCES if kernel == "gdr_bwd_local" else FWD_SOURCES
    if t.get("source_hash") != source_hash(files):
        return None
    return t.get("bytes_per_launch")


def cpu_single_core(x, train=False):
    """The oracle on one host core over the first sequence's first 4 v heads
    (and their q/k heads), in tokens/s for the whole workload's head count."""
    import numpy as np

    import oracle
    Hq, Hv = x["q"].shape[2], x["v"].shape[2]
    G = Hv // Hq
    hv = min(4, Hv)
    hq = max(1, hv // G)
    sl = {n: np.ascontiguousarray(x[n][0:1, :, :hq if n in ("q", "k") else hv], dtype=np.float64)
          for n in ("q", "k", "v", "g", "beta")}
    h0 = None if x["initial_state"] is None else \
        np.ascontiguousarray(x["initial_state"][0:1, :hv], dtype=np.float64)
    T = x["q"].shape[1]
    t0 = time.perf_counter()
    oracle.fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], x["scale"], h0, nthreads=1)
    if train:
        oracle.bwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], x["do"][0:1, :, :hv],
                   x["scale"], initial_state=h0, dht=x["dht"][0:1, :hv], nthreads=1)
    el = time.perf_counter() - t0
    return {"value": T * hv / Hv / el, "unit": "tokens/s", "cores": 1,
            "sample": "1 sequence (T=%d), %d of %d v heads, in %.1f s" % (T, hv, Hv, el)}


def cpu_baseline(x, seconds, train=False):
    """Time the fp64 oracle (forward, plus backward when `train`) on whole
    sequences of the workload, taken in turn and again from the first once all
    are done, until about `seconds` of CPU time have been spent."""
    import numpy as np

    import oracle
    B = x["q"].shape[0]
    T = x["q"].shape[1]
    done = 0
    elapsed = 0.0
    threads = 0
    for i in range(64 * B):
        b = i % B
        sl = {n: np.ascontiguousarray(x[n][b:b + 1], dtype=np.float64)
              for n in ("q", "k", "v", "g", "beta")}
        h0 = None if x["initial_state"] is None else \
            np.ascontiguousarray(x["initial_state"][b:b + 1], dtype=np.float64)
        t0 = time.perf_counter()
        oracle.fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], x["scale"], h0)
        if train:
            oracle.bwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], x["do"][b:b + 1],
                       x["scale"], initial_state=h0, dht=x["dht"][b:b + 1])
        elapsed += time.perf_counter() - t0
        threads = oracle.last_threads()
        done += 1
        if elapsed >= seconds:
            break
    return {"value": done * T / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d sequence runs over the workload's %d sequences (all %d v heads, "
                      "T=%d)%s in %.1f s" %
                      (done, B, x["v"].shape[2], T, ", forward + backward" if train else "",
                       elapsed)}


class Events:
    """HIP events handed to the library's timing hooks, one array per step.
    With `keep`, only those entries hold events; the others are NULL, which
    the library skips."""

    def __init__(self, steps, n, keep=None):
        self.hip = hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = n
        self.arrays = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * n)()
            for i in range(n):
                if keep is not None and i not in keep:
                    continue
                e = ctypes.c_void_p()
                if hip.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = e.value
            self.arrays.append(arr)

    def ptr(self, step):
        return ctypes.addressof(self.arrays[step])

    def stage_ms(self, names, only=None):
        """Average duration of stage s (events 2s, 2s+1) over the steps."""
        f = ctypes.c_float()
        out = {}
        for s, name in enumerate(names):
            if only is not None and name != only:
                continue
            tot = 0.0
            for arr in self.arrays:
                if self.hip.hipEventElapsedTime(ctypes.byref(f), arr[2 * s], arr[2 * s + 1]) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                tot += f.value
            out[name] = tot / len(self.arrays)
        return out

    def close(self):
        for arr in self.arrays:
            for i in range(self.n):
                if arr[i]:
                    self.hip.hipEventDestroy(arr[i])


CP_MODES = ("off", "warmup", "exact", "auto", "auto_exact", "auto_pages")


def cp_sweep(steps=40, warmup=5):
    """Forward time of every sequence-split mode over the family's head counts
    (H_v = 64 .. 8, H_q = H_v / 2, the README's TP1..TP8) at three batch x length
    mixes of 16,384 tokens (bf16, K = V = 128, initial state, fp32 o).  Inputs are
    drawn on the device with the recipe's distributions (unit-norm q, k; g =
    -softplus(N(0,1))/2; beta = sigmoid(N(0,1))).  Each mode: median of `steps`
    HIP-event-timed gdr_fwd calls after `warmup`, buffers allocated beforehand.
    Prints one JSON line per (mix, H_v)."""
    import torch

    from gated_delta_rule_85_amd import _lib
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    modes = {"off": _lib.CP_OFF, "warmup": _lib.CP_WARMUP, "exact": _lib.CP_EXACT, "auto": _lib.CP_AUTO,
             "auto_exact": _lib.CP_AUTO_EXACT, "auto_pages": _lib.CP_AUTO_PAGES}
    for B, T in ((4, 4096), (1, 16384), (16, 1024)):
        for Hv in (64, 48, 32, 24, 16, 8):
            Hq, K, V = Hv // 2, 128, 128
            rn = lambda *shape: torch.randn(*shape, device=dev, generator=gen)
            q = torch.nn.functional.normalize(rn(B, T, Hq, K), dim=-1).to(torch.bfloat16)
            k = torch.nn.functional.normalize(rn(B, T, Hq, K), dim=-1).to(torch.bfloat16)
            v = rn(B, T, Hv, V).to(torch.bfloat16)
            g = -0.5 * torch.nn.functional.softplus(rn(B, T, Hv))
            beta = torch.sigmoid(rn(B, T, Hv))
            h0 = 0.1 * rn(B, Hv, K, V)
            o = torch.empty(B, T, Hv, V, device=dev)
            ht = torch.empty(B, Hv, K, V, device=dev)
            row = {"B": B, "T": T, "H_v": Hv}
            args = {}
            for name, mode in modes.items():
                a = _lib.FwdArgs()
                a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, B
                a.dtype, a.out_dtype, a.scale, a.cp_mode = _lib.BF16, _lib.F32, K ** -0.5, mode
                a.q, a.k, a.v, a.g, a.beta = q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr()
                a.initial_state, a.o, a.final_state = h0.data_ptr(), o.data_ptr(), ht.data_ptr()
                n = _lib.fwd_workspace(a)
                ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
                a.workspace, a.workspace_bytes = ws.data_ptr(), n
                args[name] = (a, ws)
                for _ in range(warmup):
                    _lib.fwd(a, stream.cuda_stream)
            # the modes take turns, `rounds` times, so that clock changes hit them alike
            ts = {name: [] for name in modes}
            rounds = 4
            for _ in range(rounds):
                for name in modes:
                    a = args[name][0]
                    for _ in range(max(1, steps // rounds)):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        _lib.fwd(a, stream.cuda_stream)
                        e1.record(stream)
                        e1.synchronize()
                        ts[name].append(e0.elapsed_time(e1))
            for name in modes:
                row[name] = sorted(ts[name])[len(ts[name]) // 2]
            del args
            best = min(row[m] for m in ("off", "warmup", "exact"))
            row["auto_vs_best"] = row["auto"] / best
            print(json.dumps(row), flush=True)
            del q, k, v, g, beta, h0, o, ht
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 100; 20 for the training step)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10; 3)")
    ap.add_argument("--workload", default="prefill_shard")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cold", type=int, default=10,
                    help="extra steps timed after a 1 GiB cache scrub (median reported)")
    ap.add_argument("--cp", choices=("auto", "off", "warmup", "exact", "auto_exact", "auto_pages"), default="auto",
                    help="sequence split of the forward (training: always off)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--recompute-states", action="store_true",
                    help="training: the backward recomputes the chunk-start states")
    ap.add_argument("--cp-sweep", action="store_true",
                    help="instead of the bench line: forward time of every split mode over the "
                         "family's head counts (one JSON line per shape)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this operator has no multi-GPU path here "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.cp_sweep:
        cp_sweep()
        return

    import numpy as np
    import torch

    from gated_delta_rule_85_amd import _lib
    from gdr_inputs import make_inputs

    x = make_inputs(args.workload, seed=0)
    cfg = x["cfg"]
    train = bool(cfg.get("grads"))
    steps = args.steps if args.steps is not None else (20 if train else 100)
    warmup = args.warmup if args.warmup is not None else (3 if train else 10)
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
    keep = []  # device buffers that must outlive the timed loop

    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, n_seq
    a.dtype = _lib.BF16 if dt == torch.bfloat16 else _lib.F32
    a.out_dtype = _lib.F32
    a.scale = float(x["scale"])
    a.cp_mode = _lib.CP_OFF if train else {"auto": _lib.CP_AUTO, "off": _lib.CP_OFF,
                                            "warmup": _lib.CP_WARMUP, "exact": _lib.CP_EXACT,
                                            "auto_exact": _lib.CP_AUTO_EXACT,
                                            "auto_pages": _lib.CP_AUTO_PAGES}[args.cp]
    a.q, a.k, a.v, a.g, a.beta = q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr()
    a.initial_state = None if h0 is None else h0.data_ptr()
    a.cu_seqlens = None if cu is None else cu.data_ptr()
    a.o, a.final_state = o.data_ptr(), ht.data_ptr()
    if train:  # the forward keeps what the backward reads
        if args.recompute_states or dt != torch.bfloat16:  # T blocks rebuilt from g_cum and A
            g_cum = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
            A = torch.empty((B, T, Hv, 64), dtype=torch.float32, device=dev)
            keep += [g_cum, A]
            a.g_cum, a.A = g_cum.data_ptr(), A.data_ptr()
        if not args.recompute_states:  # chunk-start states and T blocks handed over
            n_chunks = B * ((T + 63) // 64) if cu is None else (T + 63) // 64 + n_seq  # bound
            hb = torch.empty((n_chunks, Hv, 4 * K * V), dtype=torch.uint8, device=dev)
            tb = torch.empty(max(_lib.tblocks_bytes(a), 1), dtype=torch.uint8, device=dev)
            keep += [hb, tb]
            a.h_bwd, a.tblk_bwd = hb.data_ptr(), tb.data_ptr()
    nbytes = _lib.fwd_workspace(a)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes

    bw = None
    if train:
        do, dht = put(x["do"], dt), put(x["dht"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        db = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
        dg = torch.empty_like(db)
        dh0 = torch.empty((n_seq, Hv, K, V), dtype=torch.float32, device=dev)
        keep += [do, dht, dq, dk, dv, db, dg, dh0]
        bw = _lib.BwdArgs()
        bw.B, bw.T, bw.H_q, bw.H_v, bw.K, bw.V, bw.n_seq = B, T, Hq, Hv, K, V, n_seq
        bw.dtype = bw.grad_dtype = a.dtype
        bw.scale = a.scale
        bw.q, bw.k, bw.v, bw.beta = a.q, a.k, a.v, a.beta
        bw.g_cum, bw.A = a.g_cum, a.A
        bw.dout, bw.dht, bw.initial_state, bw.cu_seqlens = do.data_ptr(), dht.data_ptr(), \
            a.initial_state, a.cu_seqlens
        bw.dq, bw.dk, bw.dv, bw.dbeta, bw.dg = dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), \
            db.data_ptr(), dg.data_ptr()
        bw.dh0 = dh0.data_ptr()
        bw.h_bwd, bw.tblk_bwd = a.h_bwd, a.tblk_bwd
        nb = _lib.bwd_workspace(bw)
        wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
        keep.append(wsb)
        bw.workspace, bw.workspace_bytes = wsb.data_ptr(), nb

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = {"f": None, "b": None}

    def step(i=None):
        a.events = None if i is None or evs["f"] is None else evs["f"].ptr(i)
        _lib.fwd(a, sh)
        if bw is not None:
            bw.events = None if i is None or evs["b"] is None else evs["b"].ptr(i)
            _lib.bwd(bw, sh)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # stage breakdown (not part of the timed region).  Each stage is timed in a pass
    # of its own, of as many steps as the timed region, that hands over only that
    # stage's two events: a stage that launches no kernel records its events as
    # markers on the stream, which would slow the stages next to it.  One more pass
    # hands over every event, for the median step.
    nbk = steps
    stage_ms = {}
    for key, names, n_ev in (("f", STAGES, _lib.FWD_STAGES),) + ((("b", BWD_STAGES, _lib.BWD_STAGES),) if train else ()):
        for s_i, name in enumerate(names):
            ev = Events(nbk, 2 * n_ev, keep={2 * s_i, 2 * s_i + 1})
            evs["f"], evs["b"] = (ev, None) if key == "f" else (None, ev)
            for i in range(nbk):
                step(i)
            torch.cuda.synchronize()
            stage_ms[name] = ev.stage_ms(names, only=name)[name]
            ev.close()
    evs["f"] = Events(nbk, 2 * _lib.FWD_STAGES)
    evs["b"] = Events(nbk, 2 * _lib.BWD_STAGES) if train else None
    for i in range(nbk):
        step(i)
    torch.cuda.synchronize()
    f = ctypes.c_float()
    per_step = []
    for i in range(nbk):
        first = evs["f"].arrays[i][0]
        last = (evs["b"] if train else evs["f"]).arrays[i][-1]
        if evs["f"].hip.hipEventElapsedTime(ctypes.byref(f), first, last) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        per_step.append(f.value)
    median_ms = sorted(per_step)[len(per_step) // 2]
    evs["f"].close()
    if train:
        evs["b"].close()
    model = bwd_algorithmic_flops(dict(cfg, B=B, T=T)) if train else \
        algorithmic_bytes(dict(cfg, B=B, T=T), out_bytes=4)
    dom = max(model, key=lambda kname: stage_ms[kname])

    # timed region: K steps; only the dominant kernel's two events are recorded
    # (on the library's stream), for the roofline
    in_bwd = dom in BWD_STAGES
    si = (BWD_STAGES if in_bwd else STAGES).index(dom)
    ev_dom = Events(steps, 2 * (_lib.BWD_STAGES if in_bwd else _lib.FWD_STAGES), keep={2 * si, 2 * si + 1})
    evs["f"], evs["b"] = (None, ev_dom) if in_bwd else (ev_dom, None)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / steps
    dom_ms = ev_dom.stage_ms(BWD_STAGES if in_bwd else STAGES, only=dom)[dom]
    ev_dom.close()
    evs["f"] = evs["b"] = None

    # cold: every step after a 1 GiB write that evicts L2 and the MALL (not part of value)
    cold = []
    if args.cold:
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        for _ in range(args.cold):
            scrub.fill_(1.0)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del scrub

    tokens = B * T
    value = tokens / (ms * 1e-3)
    tflops = F_TRI * tokens * Hv / (ms * 1e-3) / 1e12
    wl = "%s: B=%d T=%d H_q=%d H_v=%d K=%d V=%d, %s q/k/v, fp32 g/beta/state/o" % (
        args.workload, B, T, Hq, Hv, K, V, x["dtype"])
    if cu is not None:
        wl += ", %d packed sequences (%d tokens)" % (n_seq, int(x["cu_seqlens"][-1]))
    if not train and args.cp != "auto":
        wl += ", sequence split %s" % args.cp
    rec = {
        "metric": METRIC if not train else
        "GDN chunked fwd+bwd (training step) tokens/s, H_v=%d K=V=%d T=%d" % (Hv, K, T),
        "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": wl + ((", fwd (exact) + bwd, bf16 dq/dk/dv, states "
                                      + ("recomputed" if args.recompute_states else "and T blocks from the forward"))
                                     if train else ""),
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "kernel_ms": stage_ms,
        "breakdown_step_ms": median_ms,  # median step of a pass that records every stage's events
        "wall_ms_per_step": t_wall * 1e3 / steps,
    }
    if cold:
        rec["cold_step_ms"] = sorted(cold)[len(cold) // 2]
    if not train:
        # the path's minimal bytes (per token and v head, times the launch's tokens and
        # v heads) over the dominant kernel's measured duration, against HBM peak; the
        # same bytes over the whole step; this design's own bytes per kernel beside them
        bpt = minimal_bytes_per_token_head(dict(cfg, B=B, T=T, n_seq=n_seq))
        bmin = bpt * tokens * Hv
        achieved = bmin / (dom_ms * 1e-3) / 1e9
        design = model[dom] / (dom_ms * 1e-3) / 1e9
        rec["tflops_algorithmic"] = tflops
        rec["mfma_bf16_peak_frac"] = tflops / MFMA_BF16_PEAK_TFLOPS
        rec["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": achieved,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "traffic": measured_traffic(dom, args.workload),
                           "algorithmic_bytes": bmin, "bytes_per_token_head": bpt,
                           "step_frac": bmin / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "frac_fp32_o": minimal_bytes_per_token_head(dict(cfg, B=B, T=T, n_seq=n_seq), 4)
                           * tokens * Hv
                           / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "design_bytes": model[dom], "design_frac": design / HBM_PEAK_GBS}
    else:
        af = model
        achieved = af[dom] / (dom_ms * 1e-3) / 1e12
        # bf16 inputs: the backward's products run on bf16 MFMA (split fp32 operands);
        # fp32 inputs: on fp32 MFMA (v_mfma_f32_16x16x4_f32)
        peak = MFMA_BF16_PEAK_TFLOPS if dt == torch.bfloat16 else FP32_MFMA_PEAK_TFLOPS
        rec["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": achieved,
                           "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                           "traffic": measured_traffic(dom, args.workload), "algorithmic_flops": af[dom]}
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds, train)
        rec["cpu_single_core"] = cpu_single_core(x, train)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
