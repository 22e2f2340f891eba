"""The benchmark's algorithmic counts, checked on the CPU against brute-force
enumeration of the attended (query, key) pairs and against the closed form of
the Llama-3.1 chunk; and the one-GPU contract of its command line."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _keys(p, window):
    """Keys a query at position p attends, one by one."""
    return [j for j in range(p + 1) if window <= 0 or j > p - window]


def test_decode_bytes_match_enumeration():
    for window in (0, 5, 64, 100):
        m = W.ModelShape("t", 8, 2, 64, 1e4, window=window, max_position=512)
        pos = [0, 3, 63, 64, 127, 300, 511]
        elems = sum(len(_keys(p, window)) for p in pos) * m.n_kv_heads * m.head_dim
        pages = sum(len({j // 64 for j in _keys(p, window)}) for p in pos)
        want = elems * 2 * 2 + len(pos) * m.n_q_heads * m.head_dim * 2 * 2 + pages * 4
        assert bench.decode_bytes(m, np.array(pos)) == want, window


def test_prefill_flops_match_enumeration():
    for window in (0, 7, 100):
        m = W.ModelShape("t", 4, 2, 32, 1e4, window=window, max_position=512)
        pos = np.concatenate([np.arange(0, 70), np.arange(200, 260)])
        pairs = sum(len(_keys(int(p), window)) for p in pos)
        assert bench.prefill_flops(m, pos) == 4.0 * m.head_dim * m.n_q_heads * pairs


def test_llama31_chunk_flops_closed_form():
    """8192 queries at 57344..65535 over every earlier key: 4*D*Hq * sum(p+1)."""
    m = W.ModelShape("llama31", 32, 8, 128, 5e5, max_position=65536)
    pos = np.arange(57344, 65536)
    total = (57345 + 65536) * 8192 // 2
    assert bench.prefill_flops(m, pos) == 4.0 * 128 * 32 * total == 8246404317184.0


def test_write_bytes_are_rows_read_and_written():
    m = W.ModelShape("qwen3", 32, 8, 128, 1e6, qk_norm_eps=1e-6, max_position=40960)
    assert bench.write_bytes(m, 2176) == 2176 * (32 + 2 * 8) * 128 * 2 * 2


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
