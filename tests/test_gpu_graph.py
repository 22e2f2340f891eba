"""The entries under HIP graph capture: step_paged (write, prefill, decode
and merge) and the in-pass `packed` entry (index preparation, write to
scratch pages, prefill) are captured once and replayed several times, with
eager work and synchronisations between replays; every replay must equal the
eager result bit for bit."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W

from parity import device_pools, handle_for, to_np_bits, torch_i32

pytestmark = pytest.mark.gpu


def _step_setup():
    m = W.ModelShape("graph-step", 8, 2, 128, 1e6, qk_norm_eps=1e-6, max_position=2048)
    rows_pp = 32
    rng = np.random.default_rng(21)
    n_rows = 10
    table = rng.permutation(n_rows * rows_pp).astype(np.int32).reshape(n_rows, rows_pp)
    wl = W.Workload("graph-step", m, n_rows * rows_pp, table)
    kp, vp = device_pools(wl)
    # two prompts of 96 tokens on rows 0-1, eight decode rows 2-9
    pos = np.concatenate([np.arange(96), np.arange(40, 136), rng.integers(200, 2047, 8)]).astype(np.int32)
    rows = np.concatenate([np.zeros(96), np.ones(96), np.arange(2, 10)]).astype(np.int32)
    return m, wl, kp, vp, pos, rows


def test_step_paged_replays_equal_eager():
    m, wl, kp, vp, pos, rows = _step_setup()
    h = handle_for(m)
    T, P = len(pos), 192
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    qkv = wl.qkv("graph", T, "cuda")
    parts = (qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:])
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    tp, tr, tt = torch_i32(pos), torch_i32(rows), torch_i32(wl.table)
    ws = h.workspace(h.step_workspace_bytes(P, 2, T - P))
    q_out = torch.empty(T, hq * D, dtype=torch.int16, device="cuda")
    out = torch.empty_like(q_out)
    k0, v0 = kp.clone(), vp.clone()

    def run():
        h.step_paged(*parts, tp, tr, tt, kp, vp, n_prompt=P, n_segments=2, q_gain=gains[0], k_gain=gains[1],
                     q_out=q_out, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    want_out, want_k, want_v = out.clone(), kp.clone(), vp.clone()

    kp.copy_(k0)
    vp.copy_(v0)
    out.zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm the capture stream, as torch advises
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        kp.copy_(k0)
        vp.copy_(v0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {i}: outputs differ from the eager call"
        assert torch.equal(kp, want_k) and torch.equal(vp, want_v), f"replay {i}: pools differ"
        _ = (torch.randn(1 << 16, device="cuda") * 2).sum().item()   # eager work between replays


def test_packed_replays_equal_eager():
    m = W.ModelShape("graph-packed", 4, 4, 96, 1e4, window=100, max_position=1024)
    wl = W.Workload("graph-packed", m, 1, np.zeros((1, 1), np.int32))
    h = handle_for(m)
    lens = [150, 70]
    pos = np.concatenate([np.arange(300, 300 + lens[0]), np.arange(lens[1])]).astype(np.int32)
    seg = np.concatenate([np.zeros(lens[0]), np.ones(lens[1])]).astype(np.int32)
    T = len(pos)
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    qkv = wl.qkv("graph", T, "cuda")
    parts = (qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:])
    tp, tsg = torch_i32(pos), torch_i32(seg)
    ws = h.workspace(h.inpass_workspace_bytes(T, 2))
    out = torch.empty(T, hq * D, dtype=torch.int16, device="cuda")

    def run():
        h.packed(*parts, tp, tsg, n_segments=2, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    want = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        out.zero_()
        ws.fill_(7)                          # stale scratch must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}: outputs differ from the eager call"
