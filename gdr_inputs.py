"""Seeded synthetic inputs for the gated delta rule operator.

Shared by the tests, the bench and smoke(): the oracle and the HIP path both
receive exactly these arrays.  This module holds no arithmetic of the method
itself, only the input distributions:

  q, k ~ N(0,1), then divided by their L2 norm over the head dimension;
  v ~ N(0,1);  g = -0.5 * softplus(N(0,1)) (a per-token log-decay <= 0);
  beta = sigmoid(N(0,1));  initial state ~ 0.1 * N(0,1);
  upstream gradients: do ~ N(0,1), dht ~ 0.1 * N(0,1).

The pages measure on the head counts of the Qwen3.5/3.6 family (PyPI README,
"Benchmark": h in {64, 48, 32, 24, 16, 8} for TP1..TP8) over varying batch
lengths and print no data, so these synthetic tensors stand in for that
workload.  Draw order from one numpy PCG64 generator: [varlen lengths], q, k,
v, g_raw, beta_raw, [h0], [do], [dht].  bf16 tensors are rounded to nearest
even and returned as float32 arrays holding the exact bf16 values.
"""
import math

import numpy as np

# name -> shape/dtype recipe.  "lens" means packed variable-length sequences.
WORKLOADS = {
    "tiny_fp32": dict(B=1, T=256, Hq=2, Hv=2, K=64, V=64, dtype="fp32", h0=False),
    "prefill_shard": dict(B=4, T=4096, Hq=16, Hv=32, K=128, V=128, dtype="bf16", h0=True),
    "small_head_long": dict(B=1, T=32768, Hq=4, Hv=8, K=128, V=128, dtype="bf16", h0=False),
    "varlen": dict(nseq=16, len_lo=128, len_hi=16384, max_padded=65536, Hq=16, Hv=32,
                   K=128, V=128, dtype="bf16", h0=False),
    "training": dict(B=8, T=4096, Hq=32, Hv=64, K=128, V=128, dtype="bf16", h0=True,
                     grads=True),
}
WORKLOAD_ORDER = ["tiny_fp32", "prefill_shard", "small_head_long", "varlen", "training"]


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _l2norm(x):
    return (x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))).astype(
        np.float32)


def _softplus(x):
    x = x.astype(np.float64)
    return np.where(x > 20, x, np.log1p(np.exp(np.minimum(x, 20))))


def varlen_lengths(rng, nseq, lo, hi, max_padded, chunk=64):
    """Lengths floor(exp(U(ln lo, ln hi))); redrawn until the chunk-padded total fits."""
    while True:
        lens = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=nseq))).astype(
            np.int64)
        if int(np.sum((lens + chunk - 1) // chunk * chunk)) <= max_padded:
            return lens


def make_inputs(shape, seed=0, grads=None, h0=None):
    """Draw one problem.  ``shape`` is a WORKLOADS key or a dict with the same keys
    (B, T or nseq/lens, Hq, Hv, K, V, dtype).  Returns a dict of numpy arrays:
    q, k [B,T,Hq,K]; v [B,T,Hv,V]; g, beta [B,T,Hv]; initial_state
    [N,Hv,K,V] or None; cu_seqlens int32 or None; do, dht when grads; plus
    scale = 1/sqrt(K) and the recipe."""
    cfg = dict(WORKLOADS[shape]) if isinstance(shape, str) else dict(shape)
    rng = np.random.default_rng(seed)
    cu = None
    if "lens" in cfg or "nseq" in cfg:
        lens = np.asarray(cfg["lens"], np.int64) if "lens" in cfg else varlen_lengths(
            rng, cfg["nseq"], cfg["len_lo"], cfg["len_hi"], cfg["max_padded"])
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T, nstate = 1, int(cu[-1]), len(lens)
    else:
        B, T = cfg["B"], cfg["T"]
        nstate = B
    Hq, Hv, K, V = cfg["Hq"], cfg["Hv"], cfg["K"], cfg["V"]
    bf16 = cfg.get("dtype", "bf16") == "bf16"
    f32 = np.float32
    q = _l2norm(rng.standard_normal((B, T, Hq, K), dtype=f32))
    k = _l2norm(rng.standard_normal((B, T, Hq, K), dtype=f32))
    v = rng.standard_normal((B, T, Hv, V), dtype=f32)
    g = (-0.5 * _softplus(rng.standard_normal((B, T, Hv), dtype=f32))).astype(f32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv), dtype=f32).astype(
        np.float64)))).astype(f32)
    use_h0 = cfg.get("h0", False) if h0 is None else h0
    hinit = (0.1 * rng.standard_normal((nstate, Hv, K, V), dtype=f32)).astype(f32) \
        if use_h0 else None
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    out = dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=hinit, cu_seqlens=cu,
               scale=1.0 / math.sqrt(K), dtype="bf16" if bf16 else "fp32", cfg=cfg)
    want_grads = cfg.get("grads", False) if grads is None else grads
    if want_grads:
        do = rng.standard_normal((B, T, Hv, V), dtype=f32)
        out["do"] = round_bf16(do) if bf16 else do
        out["dht"] = (0.1 * rng.standard_normal((nstate, Hv, K, V), dtype=f32)).astype(f32)
    return out
