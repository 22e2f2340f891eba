"""step_paged's one-pass launch (the prompts' prefill tiles and the decode
rows' chunks in one kernel) against the same call through separate prefill
and decode launches (a handle created with DAP_FUSED_STEP=0), on the seeded
random shapes of test_gpu_random (head_dim 64/96/128, 1/2/4 query heads per
kv head, windows, QK-norm, llama3) and the Qwen3-shaped step: q_out, the
outputs and the written pools must agree bit for bit (each query row sees
its pages in the same order with the same arithmetic either way), and the
one-pass kernel must be the one that ran."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W

from parity import device_pools, handle_for, torch_i32
from test_gpu_random import _draw

pytestmark = pytest.mark.gpu


def _run(wl, h, ppos, pseg, dpos, drow, n_segments):
    m = wl.model
    kp, vp = device_pools(wl)
    pos = np.concatenate([ppos, dpos]).astype(np.int32)
    rows = np.concatenate([pseg, drow]).astype(np.int32)
    qkv = W.normal_matrix(wl.key("qkv"), len(pos), m.qkv_width, "cuda")
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda")) if m.qk_norm_eps else (None, None)
    h.set_profiling(True)
    h.profile_read(reset=True)
    q_out, out = h.step_paged(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                              torch_i32(pos), torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=len(ppos),
                              n_segments=n_segments, q_gain=gains[0], k_gain=gains[1])
    torch.cuda.synchronize()
    prof = h.profile_read(reset=True)
    h.set_profiling(False)
    return q_out, out, kp, vp, {k: v[1] for k, v in prof.items()}


def _compare(wl, ppos, pseg, dpos, drow, n_segments, monkeypatch, what):
    one = handle_for(wl.model)
    monkeypatch.setenv("DAP_FUSED_STEP", "0")
    sep = handle_for(wl.model)
    monkeypatch.delenv("DAP_FUSED_STEP")
    a = _run(wl, one, ppos, pseg, dpos, drow, n_segments)
    b = _run(wl, sep, ppos, pseg, dpos, drow, n_segments)
    assert a[4]["step"] == 1 and a[4]["prefill"] == 0 and a[4]["decode"] == 0, f"{what}: one-pass not taken: {a[4]}"
    assert b[4]["step"] == 0 and b[4]["prefill"] == 1 and b[4]["decode"] == 1, f"{what}: {b[4]}"
    for x, y, name in zip(a[:4], b[:4], ("q_out", "out", "K pool", "V pool")):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{what}: {name} differs"


@pytest.mark.parametrize("seed", range(8))
def test_one_pass_step_equals_separate_launches(seed, monkeypatch):
    wl, ppos, pseg, dpos, drow = _draw(seed)
    _compare(wl, ppos, pseg, dpos, drow, int(pseg.max()) + 1, monkeypatch, f"seed {seed}")


def test_one_pass_qwen3_step_equals_separate_launches(monkeypatch):
    wl = W.qwen3()
    _compare(wl, wl.pre_positions, wl.pre_segments, wl.dec_positions, wl.dec_rows, 8, monkeypatch, "qwen3 step")
