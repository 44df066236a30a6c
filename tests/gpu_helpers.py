"""Shared helpers of the GPU parity tests (inputs to the device, error metric)."""
import math

import numpy as np
import torch


def rel(a, b):
    """max |a - b| / rms(b), the operator's parity metric."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(math.sqrt(float(np.mean(b * b))), 1e-300))


def dev(x, dtype=torch.float32):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    """fp64 host copy of a device tensor (numpy arrays pass through as fp64)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_inputs(x):
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    d = dict(q=dev(x["q"], dt), k=dev(x["k"], dt), v=dev(x["v"], dt), g=dev(x["g"]),
             beta=dev(x["beta"]), initial_state=dev(x["initial_state"]))
    d["cu_seqlens"] = None if x["cu_seqlens"] is None else dev(x["cu_seqlens"], torch.int32)
    return d


def run_fwd(x, **kw):
    from gated_delta_rule_85_amd import chunk_gated_delta_rule_fwd
    d = gpu_inputs(x)
    out = chunk_gated_delta_rule_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], x["scale"],
                                     d["initial_state"], d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return out


def tol(x):
    """Tolerance of the parity metric: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs."""
    return 2e-2 if x["dtype"] == "bf16" else 1e-4


def slice_units(x, b, hq):
    """The sub-problem of batch b and q/k head hq with its v heads (exact: units
    of the recurrence are independent)."""
    Hq, Hv = x["q"].shape[2], x["v"].shape[2]
    G = Hv // Hq
    hs = slice(hq * G, (hq + 1) * G)
    y = dict(x)
    y["q"] = x["q"][b:b + 1, :, hq:hq + 1]
    y["k"] = x["k"][b:b + 1, :, hq:hq + 1]
    y["v"] = x["v"][b:b + 1, :, hs]
    y["g"] = x["g"][b:b + 1, :, hs]
    y["beta"] = x["beta"][b:b + 1, :, hs]
    y["initial_state"] = None if x["initial_state"] is None else x["initial_state"][b:b + 1, hs]
    return y, hs
