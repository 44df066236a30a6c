"""Double-precision CPU oracle for the gated delta rule — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It never imports the HIP package and the
HIP package never imports it; both take their inputs from ``gdr_inputs``.

Sources.  The FlashQLA pages name the operator and its interface (PyPI README,
"Usage": ``chunk_gated_delta_rule(q, k, v, g, beta, scale, initial_state,
output_final_state, cu_seqlens)`` with q, k ``[B,T,H_q,K]``, v ``[B,T,H_v,V]``,
g, beta ``[B,T,H_v]``, state ``[B,H_v,K,V]``; the low-level
``chunk_gated_delta_rule_fwd`` returns ``g, A, o, h, final_state`` and the
backward returns ``dq, dk, dv, db, dg, dh0``).  They do not print the
recurrence; the oracle uses the gated delta rule
``S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T``,
``o_t = scale S_t q_t`` with the state stored as ``h = S^T`` (K x V).

Functions:
  fwd         token recurrence, exact (C, OpenMP over (sequence, v-head) units)
  fwd_split   sequence-split forward with a zero-state warm-up window per
              segment (the pages' AutoCP "sliding window warmup")
  bwd         reverse-mode gradients of the token recurrence (C)
  chunk_form  the chunked evaluation in the order the pages list its steps
              (efeozkan blog, "2. Hardware-Friendly Algebraic Reformulation":
              A matrix, W and U, V correction, output O), numpy fp64; it
              supplies the per-chunk intermediates for per-kernel parity
  token_recurrence_np   a small pure-numpy twin of ``fwd`` for tiny inputs

Pins (tests/test_oracle_*.py): exact rational brute force in the V x K form,
a dense transition-product formula, closed forms (pure decay, orthogonal keys
= gated linear attention, first order in beta, the delta rule's overwrite
property), chunked-form equivalence, invariants, warm-up error bounds, and
finite differences / exact dot-product identities for the backward.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
CHUNK = 64


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        i64, f64 = ctypes.c_int64, ctypes.c_double
        p = ctypes.c_void_p
        common = [i64, p, i64, i64, i64, i64, i64, p, p, p, p, p, f64, p]
        lib.gdr_oracle_fwd.argtypes = common + [p, p, p, ctypes.c_int]
        lib.gdr_oracle_fwd.restype = ctypes.c_int
        lib.gdr_oracle_fwd_split.argtypes = common + [p, p, p, i64, i64, ctypes.c_int]
        lib.gdr_oracle_fwd_split.restype = ctypes.c_int
        lib.gdr_oracle_bwd.argtypes = common + [p, p, p, p, p, p, p, p, ctypes.c_int]
        lib.gdr_oracle_bwd.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _layout(q, v, cu_seqlens):
    """Packed-token view: (Ttot, seq_off[int64], B, T)."""
    B, T = q.shape[0], q.shape[1]
    if cu_seqlens is None:
        off = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        off = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return B * T, off, B, T


def num_chunks(off, chunk=CHUNK):
    lens = np.diff(off)
    return int(np.sum((lens + chunk - 1) // chunk))


def last_threads():
    return _LAST_THREADS[0]


_LAST_THREADS = [0]


def fwd(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None, chunk=CHUNK,
        want_h=False, nthreads=0):
    """Exact forward.  Returns dict(o, final_state, h, g_cum) in float64.

    o ``[B,T,H_v,V]``; final_state ``[N,H_v,K,V]``; h (chunk-start states)
    ``[B,NT,H_v,K,V]`` (``[1,NT_total,...]`` with cu_seqlens); g_cum the
    in-chunk running sum of g (README: the forward returns g).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    h0 = _f64(initial_state)
    Ttot, off, B, T = _layout(q, v, cu_seqlens)
    Hq, K = q.shape[2], q.shape[3]
    Hv, V = v.shape[2], v.shape[3]
    nseq = len(off) - 1
    o = np.zeros((Ttot, Hv, V), np.float64)
    hT = np.zeros((nseq, Hv, K, V), np.float64)
    nch = num_chunks(off, chunk)
    hc = np.zeros((nch, Hv, K, V), np.float64) if want_h else None
    _LAST_THREADS[0] = _lib().gdr_oracle_fwd(
        nseq, _ptr(off), Hq, Hv, K, V, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        float(scale), _ptr(h0), _ptr(o), _ptr(hT), _ptr(hc), int(nthreads))
    out = dict(o=o.reshape(B, T, Hv, V), final_state=hT,
               g_cum=chunk_cumsum(g, off, chunk).reshape(B, T, Hv))
    if want_h:
        out["h"] = hc.reshape(B, nch // B, Hv, K, V)
    return out


def fwd_split(q, k, v, g, beta, scale, seg_chunks, warm_chunks, initial_state=None,
              cu_seqlens=None, chunk=CHUNK, want_h=False, nthreads=0):
    """Sequence-split forward with warm-up; same return as ``fwd``."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    h0 = _f64(initial_state)
    Ttot, off, B, T = _layout(q, v, cu_seqlens)
    Hq, K = q.shape[2], q.shape[3]
    Hv, V = v.shape[2], v.shape[3]
    nseq = len(off) - 1
    o = np.zeros((Ttot, Hv, V), np.float64)
    hT = np.zeros((nseq, Hv, K, V), np.float64)
    nch = num_chunks(off, chunk)
    hc = np.zeros((nch, Hv, K, V), np.float64) if want_h else None
    _LAST_THREADS[0] = _lib().gdr_oracle_fwd_split(
        nseq, _ptr(off), Hq, Hv, K, V, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        float(scale), _ptr(h0), _ptr(o), _ptr(hT), _ptr(hc), int(seg_chunks),
        int(warm_chunks), int(nthreads))
    out = dict(o=o.reshape(B, T, Hv, V), final_state=hT)
    if want_h:
        out["h"] = hc.reshape(B, nch // B, Hv, K, V)
    return out


def bwd(q, k, v, g, beta, do, scale, initial_state=None, dht=None, cu_seqlens=None,
        chunk=CHUNK, nthreads=0):
    """Gradients of <do, o> + <dht, final_state>.  Returns dict(dq, dk, dv, dbeta, dg, dh0)."""
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    h0, dht = _f64(initial_state), _f64(dht)
    Ttot, off, B, T = _layout(q, v, cu_seqlens)
    Hq, K = q.shape[2], q.shape[3]
    Hv, V = v.shape[2], v.shape[3]
    nseq = len(off) - 1
    dq = np.zeros((Ttot, Hq, K), np.float64)
    dk = np.zeros((Ttot, Hq, K), np.float64)
    dv = np.zeros((Ttot, Hv, V), np.float64)
    db = np.zeros((Ttot, Hv), np.float64)
    dg = np.zeros((Ttot, Hv), np.float64)
    dh0 = np.zeros((nseq, Hv, K, V), np.float64)
    _LAST_THREADS[0] = _lib().gdr_oracle_bwd(
        nseq, _ptr(off), Hq, Hv, K, V, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        float(scale), _ptr(h0), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(db),
        _ptr(dg), _ptr(dh0), int(nthreads))
    return dict(dq=dq.reshape(B, T, Hq, K), dk=dk.reshape(B, T, Hq, K),
                dv=dv.reshape(B, T, Hv, V), dbeta=db.reshape(B, T, Hv),
                dg=dg.reshape(B, T, Hv), dh0=dh0)


def chunk_cumsum(g, off, chunk=CHUNK):
    """In-chunk running sum of g (float64), restarting at every chunk and
    sequence start.  g is [.., H] with a packed token axis of length off[-1]."""
    g = np.asarray(g, np.float64).reshape(int(off[-1]), -1)
    out = np.zeros_like(g)
    for j in range(len(off) - 1):
        for c0 in range(int(off[j]), int(off[j + 1]), chunk):
            c1 = min(c0 + chunk, int(off[j + 1]))
            out[c0:c1] = np.cumsum(g[c0:c1], axis=0)
    return out


def token_recurrence_np(q, k, v, g, beta, scale, initial_state=None):
    """Pure-numpy twin of ``fwd`` for tiny single-sequence inputs [B,T,H,..]."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, Hq, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    G = Hv // Hq
    o = np.zeros((B, T, Hv, V))
    hT = np.zeros((B, Hv, K, V))
    for b in range(B):
        for hv in range(Hv):
            hq = hv // G
            h = np.zeros((K, V)) if initial_state is None else \
                np.asarray(initial_state, np.float64)[b, hv].copy()
            for t in range(T):
                h = np.exp(g[b, t, hv]) * h
                u = beta[b, t, hv] * (v[b, t, hv] - h.T @ k[b, t, hq])
                h = h + np.outer(k[b, t, hq], u)
                o[b, t, hv] = scale * (h.T @ q[b, t, hq])
            hT[b, hv] = h
    return o, hT


def chunk_form(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None, chunk=CHUNK):
    """Chunked evaluation in float64, chunk by chunk, for one (sequence, v-head)
    unit at a time.  For a chunk of n tokens with start state h (K x V):

      gam  = running sum of g inside the chunk            (in-chunk log-gate)
      A    = strictly lower part of diag(beta) (K K^T) * exp(gam_r - gam_i)
      T    = (I + A)^{-1}
      W    = T diag(beta * exp(gam)) K ;  U = T diag(beta) V
      Ut   = U - W h                                      (V correction)
      O    = scale (diag(exp(gam)) Q h + (lower-incl-diag of Q K^T * exp(gam_r - gam_i)) Ut)
      h'   = exp(gam_last) h + (diag(exp(gam_last - gam)) K)^T Ut

    Returns dict with per-token arrays gam [B,T,Hv], T_rows [B,T,Hv,C]
    (row r of the chunk's T, zero-padded), W [B,T,Hv,K], U [B,T,Hv,V], the
    chunk-start states h [B,NT,Hv,K,V], o [B,T,Hv,V] and final_state.
    """
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    Ttot, off, B, T = _layout(q, v, cu_seqlens)
    Hq, K = q.shape[2], q.shape[3]
    Hv, V = v.shape[2], v.shape[3]
    G = Hv // Hq
    qf, kf = q.reshape(Ttot, Hq, K), k.reshape(Ttot, Hq, K)
    vf, gf, bf = v.reshape(Ttot, Hv, V), g.reshape(Ttot, Hv), beta.reshape(Ttot, Hv)
    nseq = len(off) - 1
    nch = num_chunks(off, chunk)
    gam = np.zeros((Ttot, Hv))
    Trows = np.zeros((Ttot, Hv, chunk))
    Wf = np.zeros((Ttot, Hv, K))
    Uf = np.zeros((Ttot, Hv, V))
    hc = np.zeros((nch, Hv, K, V))
    o = np.zeros((Ttot, Hv, V))
    hT = np.zeros((nseq, Hv, K, V))
    h0 = None if initial_state is None else np.asarray(initial_state, np.float64)
    cb = 0
    for j in range(nseq):
        t0, t1 = int(off[j]), int(off[j + 1])
        for hv in range(Hv):
            hq = hv // G
            h = np.zeros((K, V)) if h0 is None else h0[j, hv].copy()
            for c, s in enumerate(range(t0, t1, chunk)):
                e_ = min(s + chunk, t1)
                n = e_ - s
                Kc, Qc, Vc = kf[s:e_, hq], qf[s:e_, hq], vf[s:e_, hv]
                bc = bf[s:e_, hv]
                gm = np.cumsum(gf[s:e_, hv])
                Gam = np.exp(gm[:, None] - gm[None, :])
                A = np.tril(bc[:, None] * (Kc @ Kc.T) * Gam, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                W = Tm @ ((bc * np.exp(gm))[:, None] * Kc)
                U = Tm @ (bc[:, None] * Vc)
                hc[cb + c, hv] = h
                Ut = U - W @ h
                P = np.tril(Qc @ Kc.T * Gam)
                o[s:e_, hv] = scale * (np.exp(gm)[:, None] * (Qc @ h) + P @ Ut)
                h = np.exp(gm[-1]) * h + (np.exp(gm[-1] - gm)[:, None] * Kc).T @ Ut
                gam[s:e_, hv] = gm
                Trows[s:e_, hv, :n] = Tm
                Wf[s:e_, hv] = W
                Uf[s:e_, hv] = U
            hT[j, hv] = h
        cb += (t1 - t0 + chunk - 1) // chunk
    return dict(gam=gam.reshape(B, T, Hv), T_rows=Trows.reshape(B, T, Hv, chunk),
                W=Wf.reshape(B, T, Hv, K), U=Uf.reshape(B, T, Hv, V),
                h=hc.reshape(B, nch // B, Hv, K, V), o=o.reshape(B, T, Hv, V), final_state=hT)
