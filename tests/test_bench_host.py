"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic models its roofline entries use."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_prefill_shard():
    """Per chunk-head (K = V = 128, bf16, G = 2, fp32 o): the scan reads q and k (8 KB
    each, shared by the 2 v heads), v 16 KB and the 13 KB T block and writes o 32 KB;
    plus the initial and final states.  Prep reads k and the gates and writes the T block."""
    cfg = dict(B=4, T=4096, Hq=16, Hv=32, K=128, V=128, dtype="bf16", h0=True)
    ab = bench.algorithmic_bytes(cfg, out_bytes=4)
    chunk_heads = 4 * 64 * 32
    state = 4 * 32 * 128 * 128 * 4
    per = 8192 + 8192 + 16384 + bench.TBLOCK + 32768
    assert ab["gdr_scan_output"] == chunk_heads * per + 2 * state
    assert ab["gdr_chunk_prep"] == chunk_heads * (8192 + 2 * 64 * 4 + bench.TBLOCK)


def test_backward_flop_model_is_positive_and_scales_with_tokens():
    cfg = dict(B=1, T=4096, Hq=2, Hv=4, K=128, V=128)
    one = bench.bwd_algorithmic_flops(cfg)
    two = bench.bwd_algorithmic_flops(dict(cfg, B=2))
    for k in one:
        assert one[k] > 0 and two[k] == 2 * one[k]


def test_minimal_bytes_of_the_prefill_shard():
    """The path's least bytes per token and v head at K = V = 128, G = 2, bf16, T = 4096
    with an initial state: q and k 128 each (shared by 2 v heads), v 256, g and beta 8,
    o 256 in bf16 (512 in fp32), the two states amortised 32."""
    cfg = dict(B=4, T=4096, Hq=16, Hv=32, K=128, V=128, dtype="bf16", h0=True)
    assert bench.minimal_bytes_per_token_head(cfg) == 808
    assert bench.minimal_bytes_per_token_head(cfg, out_bytes=4) == 1064
    # packed sequences: the states of every sequence over the packed tokens
    assert bench.minimal_bytes_per_token_head(dict(cfg, B=1, T=16384, n_seq=4)) == 808
