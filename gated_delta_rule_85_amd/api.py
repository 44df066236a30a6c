"""PyTorch-facing API of the gfx950 gated delta rule operator.

Names and argument order follow the FlashQLA README ("Usage": the high-level
``chunk_gated_delta_rule`` and the low-level ``chunk_gated_delta_rule_fwd`` /
``chunk_gated_delta_rule_bwd``).  PyTorch only allocates device memory and
supplies the current stream; every step runs in libgdr's HIP kernels.

Output dtype.  ``o`` is returned in float32 by default: for bf16 inputs the
operator accumulates in fp32 and a bf16 ``o`` would add a rounding of up to
2^-8 |o| per element (``output_dtype=torch.bfloat16`` selects it).
"""
import math
from typing import NamedTuple

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.BF16, torch.float32: _lib.F32}
_CP = {"auto": _lib.CP_AUTO, "off": _lib.CP_OFF, "warmup": _lib.CP_WARMUP, "exact": _lib.CP_EXACT,
       "auto_exact": _lib.CP_AUTO_EXACT, "auto_pages": _lib.CP_AUTO_PAGES}


class SavedForBackward(NamedTuple):
    """What the forward hands the backward (``return_h_bwd``): the chunk-start
    states in the backward's layout (uint8 [NT,H_v,4KV]: fp32 [K][V] for fp32
    inputs, bf16 hi then lo planes of h^T for bf16 inputs) and the T blocks
    (uint8, one 13,312-byte block per chunk and v head for bf16 inputs: the
    forward's own, which it writes there; 17,408 bytes with full rows for fp32)."""
    states: torch.Tensor
    tblocks: torch.Tensor


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(q, k, v, g, beta, cu_seqlens):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [B,T,H_q,K] and v [B,T,H_v,V]")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bfloat16 or float32")
    B, T, Hv = v.shape[0], v.shape[1], v.shape[2]
    if (g is not None and g.shape != (B, T, Hv)) or beta.shape != (B, T, Hv):
        raise ValueError("g and beta must be [B,T,H_v]")
    if not q.is_cuda:
        raise ValueError("inputs must be on the GPU")
    if cu_seqlens is not None and (B != 1 or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise ValueError("cu_seqlens must be int32 [N+1] with B == 1")
    if cu_seqlens is not None and not cu_seqlens.is_cuda:
        # offsets on the host are checked here; on the device the library clamps them
        # (reading them here would synchronise the stream)
        check_offsets(cu_seqlens, T)


def check_offsets(cu_seqlens, T):
    """Raise ValueError unless the host offsets start at 0, never decrease and end
    at T (the packed token count)."""
    c = torch.as_tensor(cu_seqlens).to(torch.int64)
    if c.dim() != 1 or c.numel() < 2 or int(c[0]) != 0 or int(c[-1]) != T or bool((c[1:] < c[:-1]).any()):
        raise ValueError("cu_seqlens must start at 0, never decrease and end at T")


def _c(t, dtype=None):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.contiguous()


def num_chunks(T, B=1, cu_seqlens=None):
    """Chunk-start state count of the forward's h (with device cu_seqlens this reads
    them back, a host synchronisation)."""
    if cu_seqlens is None:
        return B * ((T + _lib.CHUNK - 1) // _lib.CHUNK)
    lens = (cu_seqlens[1:] - cu_seqlens[:-1]).to("cpu", torch.int64)
    return int(((lens + _lib.CHUNK - 1) // _lib.CHUNK).sum())


def chunk_bound(T, B=1, n_seq=None):
    """Upper bound on the chunk count without reading cu_seqlens: B ceil(T/64), or
    ceil(T/64) + n_seq for n_seq packed sequences (the bound the library uses)."""
    nct = (T + _lib.CHUNK - 1) // _lib.CHUNK
    return B * nct if n_seq is None else nct + n_seq


def chunk_gated_delta_rule_fwd(q, k, v, g, beta, scale=None, initial_state=None,
                               cu_seqlens=None, output_final_state=True, *,
                               output_dtype=torch.float32, return_h=True, cp_mode="auto",
                               cp_segment_chunks=0, cp_warmup_chunks=0, return_wu=False,
                               return_h_bwd=False, return_ga=True):
    """Low-level forward.  Returns ``(g_cum, A, o, h, final_state)``.

    g_cum [B,T,H_v] fp32 is the in-chunk cumulative log-gate; A [B,T,H_v,64]
    fp32 holds, per token, its row of T = (I + A_strict)^{-1} for its chunk;
    h [1,NT,H_v,K,V] fp32 the chunk-start states (None unless return_h);
    final_state [N,H_v,K,V] fp32 (None unless output_final_state).  With
    ``return_wu`` also returns W, U [B,T,H_v,K|V] fp32.  ``cp_mode``: "auto"
    (split where the device model predicts a gain; each segment warms up over a
    window chosen from its gates, or from the sequence start where they do not
    decay: exact to fp32 rounding for any gates), "auto_exact" (the device model,
    exact carry), "auto_pages" (the pages' trigger with a fixed warm-up window),
    "off" (no split), "warmup" (split with a fixed warm-up window of
    ``cp_warmup_chunks``) or "exact" (split with the exact carry).

    ``return_h_bwd`` replaces h by a :class:`SavedForBackward` (the chunk-start
    states in the backward's layout and the T blocks); passed to
    :func:`chunk_gated_delta_rule_bwd` as ``h_bwd`` it saves the backward's
    recompute of the states and rebuild of the T blocks (a ``states`` or
    ``tblocks`` of None there has that part recomputed: the T blocks from g_cum
    and A).  The states are then
    exact: "auto" splits as "auto_exact" and "warmup" is refused.  With
    ``return_ga=False`` g_cum and A are not written (None): a bf16 backward
    given ``h_bwd`` does not read them.
    """
    if return_h_bwd and cp_mode in ("warmup", "auto_pages"):
        raise ValueError("return_h_bwd needs exact states: not with a fixed warm-up window")
    _check(q, k, v, g, beta, cu_seqlens)
    q, k, v = _c(q), _c(k), _c(v)
    g, beta = _c(g, torch.float32), _c(beta, torch.float32)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    h0 = _c(initial_state, torch.float32)
    if h0 is not None and h0.shape != (n_seq, Hv, K, V):
        raise ValueError("initial_state must be [N,H_v,K,V]")
    cu = None if cu_seqlens is None else _c(cu_seqlens).to(dev)
    o = torch.empty((B, T, Hv, V), dtype=output_dtype, device=dev)
    g_cum = A = None
    if return_ga:
        g_cum = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
        A = torch.empty((B, T, Hv, _lib.CHUNK), dtype=torch.float32, device=dev)
    ht = torch.empty((n_seq, Hv, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    h = None
    if return_h and not return_h_bwd:
        # the exact chunk count: from host offsets as given, else read back (a sync)
        h = torch.empty((1 if cu is not None else B, num_chunks(T, 1, cu_seqlens) if cu is not None
                         else num_chunks(T), Hv, K, V), dtype=torch.float32, device=dev)
    if return_h_bwd:
        # sized by the bound, so the training path never reads the offsets back
        h = torch.empty((chunk_bound(T, B, n_seq if cu is not None else None), Hv, 4 * K * V),
                        dtype=torch.uint8, device=dev)
    w = u = None
    if return_wu:
        w = torch.empty((B, T, Hv, K), dtype=torch.float32, device=dev)
        u = torch.empty((B, T, Hv, V), dtype=torch.float32, device=dev)
    a = _lib.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, n_seq
    a.dtype = _DT[q.dtype]
    a.out_dtype = _DT[output_dtype]
    a.scale = float(scale)
    a.cp_mode = _CP[cp_mode]
    a.cp_segment_chunks = int(cp_segment_chunks)
    a.cp_warmup_chunks = int(cp_warmup_chunks)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.initial_state, a.cu_seqlens = _ptr(h0), _ptr(cu)
    a.o, a.final_state, a.g_cum, a.A = _ptr(o), _ptr(ht), _ptr(g_cum), _ptr(A)
    if return_h_bwd:
        tb = torch.empty(max(_lib.tblocks_bytes(a), 1), dtype=torch.uint8, device=dev)
        h = SavedForBackward(h, tb)
        a.h_bwd, a.tblk_bwd = _ptr(h.states), _ptr(tb)
    else:
        a.h = _ptr(h)
    a.w_out, a.u_out = _ptr(w), _ptr(u)
    nbytes = _lib.fwd_workspace(a)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
    _lib.fwd(a, torch.cuda.current_stream(dev).cuda_stream)
    if return_wu:
        return g_cum, A, o, h, ht, w, u
    return g_cum, A, o, h, ht


def chunk_gated_delta_rule_bwd(q, k, v, g, beta, A, do, dht=None, scale=None, initial_state=None,
                               cu_seqlens=None, *, grad_dtype=None, cp_mode="auto", cp_segment_chunks=0,
                               h_bwd=None):
    """Low-level backward.  ``g`` is the forward's g_cum, ``A`` its A.
    Returns ``(dq, dk, dv, db, dg, dh0)``; dh0 is None without initial_state.
    dq, dk, dv come in ``grad_dtype`` (default: the dtype of q), db, dg, dh0 in
    float32.  The gradients are accumulated in fp32; a bf16 dq/dk/dv adds one
    rounding of up to 2^-9 |x| per element.  ``cp_mode``: "auto" (split the
    recurrences of long sequences of few heads), "off" or "exact"; the split is
    always exact here.  ``h_bwd``: the forward's :class:`SavedForBackward`
    (``return_h_bwd``) for the same inputs; without it the chunk-start states
    are recomputed and the T blocks rebuilt from ``g`` and ``A``, which with it
    and bf16 inputs may be None."""
    if cp_mode not in ("auto", "auto_exact", "off", "exact"):
        raise ValueError("cp_mode of the backward: 'auto', 'auto_exact', 'off' or 'exact'")
    _check(q, k, v, g, beta, cu_seqlens)
    if (g is None or A is None) and (h_bwd is None or h_bwd.tblocks is None or q.dtype != torch.bfloat16):
        raise ValueError("g_cum and A are needed unless h_bwd (with T blocks) is given with bf16 inputs")
    q, k, v, do = _c(q), _c(k), _c(v), _c(do, q.dtype)
    g, beta, A = _c(g, torch.float32), _c(beta, torch.float32), _c(A, torch.float32)
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    n_seq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = q.device
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    h0 = _c(initial_state, torch.float32)
    dht = _c(dht, torch.float32)
    cu = None if cu_seqlens is None else _c(cu_seqlens).to(dev)
    if h_bwd is not None:
        nt = chunk_bound(T, B, n_seq if cu is not None else None)
        st = h_bwd.states
        if st is not None and (st.dtype != torch.uint8 or st.shape != (nt, Hv, 4 * K * V)
                               or not st.is_contiguous()):
            raise ValueError("h_bwd.states must be the forward's uint8 [NT,H_v,4KV] states")
    gdt = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty(q.shape, dtype=gdt, device=dev)
    dk = torch.empty(k.shape, dtype=gdt, device=dev)
    dv = torch.empty(v.shape, dtype=gdt, device=dev)
    db = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    dg = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    dh0 = torch.empty((n_seq, Hv, K, V), dtype=torch.float32, device=dev) if h0 is not None else None
    a = _lib.BwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = B, T, Hq, Hv, K, V, n_seq
    a.dtype = _DT[q.dtype]
    a.grad_dtype = _DT[gdt]
    a.cp_mode = _CP[cp_mode]
    a.cp_segment_chunks = int(cp_segment_chunks)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g_cum, a.beta, a.A = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A)
    a.dout, a.dht, a.initial_state, a.cu_seqlens = _ptr(do), _ptr(dht), _ptr(h0), _ptr(cu)
    if h_bwd is not None:
        a.h_bwd, a.tblk_bwd = _ptr(h_bwd.states), _ptr(h_bwd.tblocks)
        if h_bwd.tblocks is not None:  # None: rebuilt from g and A
            fa = _lib.FwdArgs()
            fa.B, fa.T, fa.H_q, fa.H_v, fa.K, fa.V, fa.n_seq = B, T, Hq, Hv, K, V, n_seq
            fa.dtype, fa.out_dtype = a.dtype, _lib.F32
            fa.cu_seqlens = a.cu_seqlens
            if h_bwd.tblocks.dtype != torch.uint8 or h_bwd.tblocks.numel() < _lib.tblocks_bytes(fa) \
                    or not h_bwd.tblocks.is_contiguous():
                raise ValueError("h_bwd.tblocks must be the forward's T blocks")
    a.dq, a.dk, a.dv, a.dbeta, a.dg, a.dh0 = _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db), _ptr(dg), _ptr(dh0)
    nbytes = _lib.bwd_workspace(a)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
    _lib.bwd(a, torch.cuda.current_stream(dev).cuda_stream)
    return dq, dk, dv, db, dg, dh0


class _ChunkGDR(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                output_dtype, cp_mode, save_states):
        # the backward differentiates the exact recurrence: when training, a split
        # (where the device model predicts a gain) is the exact one
        train = any(ctx.needs_input_grad)
        if train:
            cp_mode = "off" if cp_mode == "off" else "auto_exact"
        saved = train and save_states
        # a bf16 backward given the forward's T blocks reads neither g_cum nor A
        g_cum, A, o, hb, ht = chunk_gated_delta_rule_fwd(
            q, k, v, g, beta, scale, initial_state, cu_seqlens, output_final_state=True,
            output_dtype=output_dtype, return_h=False, cp_mode=cp_mode,
            return_h_bwd=saved, return_ga=not (saved and q.dtype == torch.bfloat16))
        hs, tb = hb if saved else (None, None)
        ctx.save_for_backward(q, k, v, g_cum, beta, A, initial_state, cu_seqlens, hs, tb)
        ctx.scale = scale
        ctx.g_dtype = g.dtype
        return o, (ht if output_final_state else None)

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g_cum, beta, A, h0, cu, hs, tb = ctx.saved_tensors
        dq, dk, dv, db, dg, dh0 = chunk_gated_delta_rule_bwd(
            q, k, v, g_cum, beta, A, do, dht, ctx.scale, h0, cu,
            h_bwd=None if hs is None else SavedForBackward(hs, tb))
        return (dq, dk, dv, dg.to(ctx.g_dtype), db.to(beta.dtype), None, dh0, None, None, None,
                None, None)


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None,
                           output_final_state=False, cu_seqlens=None, *,
                           output_dtype=torch.float32, cp_mode="auto", save_states=True):
    """High-level differentiable API.  Returns ``(o, final_state)``.

    Without gradients the forward may split long sequences (``cp_mode``);
    when any input requires a gradient a split is the exact one, as in the
    backward.  ``save_states``: when training, keep the forward's chunk-start
    states (4 K V bytes per chunk and v head) and T blocks for the backward
    instead of recomputing them there (for bf16 inputs g_cum and A are then
    not kept)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o, ht = _ChunkGDR.apply(q, k, v, g, beta, scale, initial_state, output_final_state,
                            cu_seqlens, output_dtype, cp_mode, save_states)
    return o, ht
