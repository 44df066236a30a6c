"""The C ABI of libgdr without a GPU: exports, struct layout, host-side errors.

Only calls that return before any HIP work are made here (version, error
strings, workspace sizing, argument validation).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def L():
    from gated_delta_rule_85_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdr_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"gdr_fwd", "gdr_bwd", "gdr_fwd_workspace", "gdr_bwd_workspace", "gdr_strerror",
            "gdr_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L.lib, n), n


def test_version_and_strings(L):
    assert L.abi_version() == L.ABI_VERSION
    assert L.strerror(0) == "ok"
    assert L.strerror(-3) == "workspace too small"
    assert L.strerror(12345) == "unknown error"


def _struct_offsets_from_c(tmp_path, struct, fields):
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gdr.h"', "int main(void){"]
    lines.append('printf("size %%zu\\n", sizeof(%s));' % struct)
    for f in fields:
        lines.append('printf("%s %%zu\\n", offsetof(%s, %s));' % (f, struct, f))
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                    "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {k: int(v) for k, v in (l.split() for l in out.splitlines())}


@pytest.mark.parametrize("which", ["fwd", "bwd"])
def test_ctypes_layout_matches_header(L, tmp_path, which):
    st = L.FwdArgs if which == "fwd" else L.BwdArgs
    names = [f[0] for f in st._fields_]
    c = _struct_offsets_from_c(tmp_path, "gdr_%s_args" % which, names)
    assert c["size"] == ctypes.sizeof(st)
    for n in names:
        assert c[n] == getattr(st, n).offset, n


def fwd_args(L, **kw):
    a = L.FwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = 1, 256, 2, 4, 128, 128, 0
    a.dtype, a.out_dtype, a.scale = L.BF16, L.F32, 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def rc_ws(L, a):
    n = ctypes.c_size_t(0)
    return L.lib.gdr_fwd_workspace(ctypes.byref(a), ctypes.byref(n)), n.value


TBLOCK = 17408      # one (chunk, v head) T block with full rows (fp32 inputs): T + gate scalars
TBLOCK_FWD = 13312  # bf16 inputs, forward and backward: hi/lo planes, rows 0-31 at half width


def test_workspace_sizes(L):
    # T=256: 4 chunks x 4 v heads of T blocks
    rc, n = rc_ws(L, fwd_args(L))
    assert rc == 0 and n == 4 * 4 * TBLOCK_FWD
    rc, n = rc_ws(L, fwd_args(L, g_cum=16, A=16))
    assert rc == 0 and n == 4 * 4 * TBLOCK_FWD
    # packed sequences: chunk offsets and clamped bounds (2 (n_seq + 1) int32, the
    # table 256-byte aligned) + blocks for up to ceil(T/64) + n_seq chunks
    rc, n = rc_ws(L, fwd_args(L, cu_seqlens=16, n_seq=3))
    assert rc == 0 and n == 256 + (4 + 3) * 4 * TBLOCK_FWD
    rc, n = rc_ws(L, fwd_args(L, dtype=L.F32, K=64, V=64))
    assert rc == 0 and n == 4 * 4 * TBLOCK  # fp32: full rows
    # up to 8192 packed sequences also get their longest-first order: (3 n_seq + 2)
    # int32 entries; beyond that only the offsets and bounds
    rc, n = rc_ws(L, fwd_args(L, cu_seqlens=16, n_seq=100))
    assert rc == 0 and n == 1280 + (4 + 100) * 4 * TBLOCK_FWD
    rc, n = rc_ws(L, fwd_args(L, cu_seqlens=16, n_seq=9000))
    assert rc == 0 and n == 72192 + (4 + 9000) * 4 * TBLOCK_FWD


@pytest.mark.parametrize("kw,code", [
    (dict(H_v=3), -1),             # H_v % H_q != 0
    (dict(K=96), -2),              # unsupported head dim
    (dict(V=32), -2),
    (dict(dtype=7), -2),
    (dict(out_dtype=9), -2),
    (dict(B=0), -1),
    (dict(T=-1), -1),
    (dict(cu_seqlens=16, n_seq=0), -1),
    (dict(cu_seqlens=16, n_seq=2, B=2), -1),
    (dict(cp_mode=6), -1),
    (dict(cp_mode=-1), -1),
    (dict(cp_segment_chunks=-1), -1),
])
def test_validation_errors(L, kw, code):
    rc, _ = rc_ws(L, fwd_args(L, **kw))
    assert rc == code
    assert L.lib.gdr_fwd(ctypes.byref(fwd_args(L, **kw)), None) == code


def test_segment_count_is_bounded(L):
    """A caller's segment length of one chunk over many units would overflow the
    scan grid and the exact split's workspace size; the plan refuses it."""
    many = dict(T=1 << 20, H_q=1, H_v=1 << 17, cp_segment_chunks=1)  # 16,384 segments x 2^17 units
    for mode in (L.CP_EXACT, L.CP_WARMUP):
        rc, _ = rc_ws(L, fwd_args(L, cp_mode=mode, **many))
        assert rc == L.EINVAL
    n = ctypes.c_size_t(0)
    assert L.lib.gdr_bwd_workspace(ctypes.byref(bwd_args(L, cp_mode=L.CP_EXACT, **many)), ctypes.byref(n)) == L.EINVAL
    # the same shape unsplit, or with segments of 64 chunks, plans normally
    assert rc_ws(L, fwd_args(L, cp_mode=L.CP_OFF, **many))[0] == 0
    assert rc_ws(L, fwd_args(L, cp_mode=L.CP_EXACT, **dict(many, cp_segment_chunks=64)))[0] == 0


def test_chunk_grid_is_bounded(L):
    """Prep and the chunk-local backward launch one workgroup of 256 threads per
    (chunk, q/k head) in a one-dimensional grid of at most 2^32 work-items; the plan
    refuses shapes past it instead of launching a wrapped grid."""
    big = dict(B=1, T=1 << 27, H_v=8)  # 2^21 chunks
    n = ctypes.c_size_t(0)
    assert rc_ws(L, fwd_args(L, H_q=8, **big))[0] == L.EINVAL  # 2^24 workgroups
    assert L.lib.gdr_bwd_workspace(ctypes.byref(bwd_args(L, H_q=8, **big)), ctypes.byref(n)) == L.EINVAL
    assert rc_ws(L, fwd_args(L, H_q=4, cp_mode=L.CP_OFF, **big))[0] == 0
    assert L.lib.gdr_bwd_workspace(ctypes.byref(bwd_args(L, H_q=4, cp_mode=L.CP_OFF, **big)), ctypes.byref(n)) == 0


def test_fwd_host_errors_before_any_launch(L):
    a = fwd_args(L)  # all pointers null
    assert L.lib.gdr_fwd(ctypes.byref(a), None) == L.EINVAL
    a = fwd_args(L, q=16, k=16, v=16, g=16, beta=16, o=16)
    assert L.lib.gdr_fwd(ctypes.byref(a), None) == L.EWORKSPACE
    a = fwd_args(L, q=16, k=16, v=16, g=16, beta=16, o=24, workspace=4096, workspace_bytes=1 << 30)
    assert L.lib.gdr_fwd(ctypes.byref(a), None) == L.EINVAL  # misaligned o
    with pytest.raises(L.GdrError):
        L.fwd_workspace(fwd_args(L, K=48))


def test_forward_states_for_the_backward(L):
    """h_bwd (the chunk-start states in the backward's layout) must be exact: with it
    AUTO plans as AUTO_EXACT; with h or the warm-up split it is refused."""
    long = dict(T=4096, H_q=1, H_v=1)
    rc, n_auto = rc_ws(L, fwd_args(L, **long))
    rc2, n_exact = rc_ws(L, fwd_args(L, cp_mode=L.CP_AUTO_EXACT, **long))
    rc3, n_hb = rc_ws(L, fwd_args(L, h_bwd=16, **long))
    assert rc == rc2 == rc3 == 0
    assert n_hb == n_exact > n_auto  # the exact split's transitions and states
    assert rc_ws(L, fwd_args(L, h_bwd=16, h=16))[0] == L.EINVAL
    assert rc_ws(L, fwd_args(L, h_bwd=16, cp_mode=L.CP_WARMUP))[0] == L.EINVAL
    assert rc_ws(L, fwd_args(L, h_bwd=16, cp_mode=L.CP_AUTO_PAGES))[0] == L.EINVAL
    a = fwd_args(L, q=16, k=16, v=16, g=16, beta=16, o=16, h_bwd=24, workspace=4096,
                 workspace_bytes=1 << 30)
    assert L.lib.gdr_fwd(ctypes.byref(a), None) == L.EINVAL  # misaligned h_bwd


def test_forward_tblocks_for_the_backward(L):
    """tblk_bwd: a caller buffer of gdr_tblocks_bytes() that the backward takes instead
    of rebuilding its T blocks.  For bf16 inputs the forward writes its own blocks there
    (the backward reads the same layout), so they leave the workspace; for fp32 inputs
    it writes a second copy in the backward's layout."""
    assert L.tblocks_bytes(fwd_args(L)) == 4 * 4 * TBLOCK_FWD
    assert L.tblocks_bytes(fwd_args(L, cu_seqlens=16, n_seq=3)) == (4 + 3) * 4 * TBLOCK_FWD
    assert L.tblocks_bytes(fwd_args(L, T=0)) == 0
    assert L.tblocks_bytes(fwd_args(L, dtype=L.F32, K=64, V=64)) == 4 * 4 * TBLOCK
    assert rc_ws(L, fwd_args(L, tblk_bwd=16)) == (0, 0)
    assert rc_ws(L, fwd_args(L, tblk_bwd=16, cu_seqlens=16, n_seq=3)) == (0, 256)
    f32 = dict(dtype=L.F32, K=64, V=64)
    assert rc_ws(L, fwd_args(L, tblk_bwd=16, **f32)) == rc_ws(L, fwd_args(L, **f32))
    a = fwd_args(L, q=16, k=16, v=16, g=16, beta=16, o=16, tblk_bwd=40, workspace=4096,
                 workspace_bytes=1 << 30)
    assert L.lib.gdr_fwd(ctypes.byref(a), None) == L.EINVAL  # misaligned tblk_bwd
    per = 2 * 4 * 128 * 128
    assert L.bwd_workspace(bwd_args(L, tblk_bwd=16)) == 4 * 4 * per
    assert L.bwd_workspace(bwd_args(L, tblk_bwd=16, h_bwd=16)) == 4 * 4 * per // 2
    # with the forward's T blocks a bf16 backward needs neither g_cum nor A (it gets as
    # far as the workspace check); fp32 kernels still read them
    noga = dict(q=16, k=16, v=16, beta=16, dout=16, dq=16, dk=16, dv=16, dbeta=16, dg=16)
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, **noga)), None) == L.EINVAL
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, tblk_bwd=16, **noga)), None) == L.EWORKSPACE
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, tblk_bwd=16, dtype=L.F32, **noga)), None) == L.EINVAL


def bwd_args(L, **kw):
    a = L.BwdArgs()
    a.B, a.T, a.H_q, a.H_v, a.K, a.V, a.n_seq = 1, 256, 2, 4, 128, 128, 0
    a.dtype, a.scale = L.BF16, 0.088
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_bwd_workspace_sizes(L):
    # T blocks + chunk-start states + chunk-end state gradients, per (chunk, v head)
    per = TBLOCK_FWD + 2 * 4 * 128 * 128
    assert L.bwd_workspace(bwd_args(L)) == 4 * 4 * per
    assert L.bwd_workspace(bwd_args(L, cu_seqlens=16, n_seq=3)) == 256 + (4 + 3) * 4 * per
    assert L.bwd_workspace(bwd_args(L, T=0)) == 0
    # exact sequence split forced: the device model (256 compute units without a device,
    # 8 workgroups per segment index, 8-chunk overhead) puts the 4 chunks in 4 segments;
    # per (sequence, v head, segment) a K x K transition and four K x V states, and a
    # zero row
    seg = 4 * 4 * 128 * 4
    split = 4 * 4 * per + seg * 128 + 4 * seg * 128 + 512
    assert L.bwd_workspace(bwd_args(L, cp_mode=L.CP_EXACT)) == split
    # the forward's states (h_bwd) replace the workspace's chunk-start states
    states = 4 * 4 * 4 * 128 * 128
    assert L.bwd_workspace(bwd_args(L, h_bwd=16)) == 4 * 4 * per - states
    assert L.bwd_workspace(bwd_args(L, h_bwd=16, cp_mode=L.CP_EXACT)) == split - states


@pytest.mark.parametrize("kw,code", [
    (dict(H_v=3), -1), (dict(K=96), -2), (dict(dtype=7), -2), (dict(grad_dtype=9), -2),
    (dict(B=0), -1),
    (dict(cu_seqlens=16, n_seq=2, B=2), -1),
    (dict(cp_mode=2), -1),                  # no warm-up split in the backward
    (dict(cp_segment_chunks=-3), -1),
])
def test_bwd_validation_errors(L, kw, code):
    n = ctypes.c_size_t(0)
    assert L.lib.gdr_bwd_workspace(ctypes.byref(bwd_args(L, **kw)), ctypes.byref(n)) == code
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, **kw)), None) == code


def test_bwd_host_errors_before_any_launch(L):
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L)), None) == L.EINVAL  # null pointers
    full = dict(q=16, k=16, v=16, g_cum=16, beta=16, A=16, dout=16, dq=16, dk=16, dv=16,
                dbeta=16, dg=16)
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, **full)), None) == L.EWORKSPACE
    bad = dict(full, dq=24, workspace=4096, workspace_bytes=1 << 34)
    assert L.lib.gdr_bwd(ctypes.byref(bwd_args(L, **bad)), None) == L.EINVAL


def test_host_offsets_are_validated(L):
    """Packed-sequence offsets given on the host are checked by the binding before
    anything reaches the device: 0 first, never decreasing, T last."""
    import torch
    from gated_delta_rule_85_amd.api import check_offsets
    check_offsets(torch.tensor([0, 5, 5, 9], dtype=torch.int32), 9)
    for bad in ([1, 5, 9], [0, 5, 4, 9], [0, 5, 10], [0, 5, 8], [0]):
        with pytest.raises(ValueError):
            check_offsets(torch.tensor(bad, dtype=torch.int32), 9)


def test_noalloc_host_errors_before_any_launch(L):
    """gdr_fwd_noalloc validates like gdr_fwd, ignores the workspace fields, and
    refuses a problem whose scratch exceeds GDR_SCRATCH_BYTES with GDR_ESCRATCH,
    all before looking up its buffer or launching anything."""
    assert L.lib.gdr_fwd_noalloc(ctypes.byref(fwd_args(L)), None) == L.EINVAL
    assert L.lib.gdr_fwd_noalloc(ctypes.byref(fwd_args(L, K=96)), None) == L.ENOTSUP
    big = fwd_args(L, B=8, T=4096, H_q=32, H_v=64, q=16, k=16, v=16, g=16, beta=16, o=16)
    assert rc_ws(L, big)[1] > L.SCRATCH_BYTES
    assert L.lib.gdr_fwd_noalloc(ctypes.byref(big), None) == L.ESCRATCH
    assert L.strerror(L.ESCRATCH).startswith("problem needs more")
