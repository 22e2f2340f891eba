"""Seeded random shapes through one step_paged call each, against the oracle.

Every seed draws a model (head_dim 64/96/128, 1-8 kv heads, 1, 2 or 4 query
heads per kv head, a window or none, QK-norm or none, llama3 rope or not)
and 3-6 rows, each with a random page permutation, a pre-filled prefix of
random length, a prompt chunk of random length after it and a decode token
after that; a further row only decodes. The call writes every token, runs
the packed prefill on the prompts and the decode on the step tokens; the
pools must hold the oracle's K/V for every written slot (bit for bit up to
the rounding reading) and every output must match the oracle's attention
over the written pools."""
import zlib

import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, pages

from parity import OraclePool, check_bits, check_close, device_pools, handle_for, oracle_front, to_np_bits, torch_i32

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 96, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    window = int(rng.choice([0, 0, 1, 37, 200, 1000]))
    llama3 = (8.0, 1.0, 4.0, 8192.0) if rng.random() < 0.3 else None
    eps = 1e-6 if rng.random() < 0.4 else None
    theta = float(rng.choice([1e4, 5e5, 1e6]))
    model = W.ModelShape(f"rand-{seed}", hkv * g, hkv, D, theta, window=window, llama3=llama3, qk_norm_eps=eps,
                         max_position=2048)
    n_rows = int(rng.integers(3, 7))
    ppr = model.max_position // 64
    perm = np.random.default_rng(zlib.crc32(model.name.encode())).permutation(n_rows * ppr).astype(np.int32)
    wl = W.Workload(model.name, model, n_rows * ppr, perm.reshape(n_rows, ppr))
    ppos, pseg, dpos, drow = [], [], [], []
    for r in range(n_rows - 1):
        start = int(rng.integers(0, 900))
        n = int(rng.integers(1, 300))
        ppos.append(np.arange(start, start + n))
        pseg.append(np.full(n, r))
        dpos.append(start + n)
        drow.append(r)
    dpos.append(int(rng.integers(0, model.max_position)))       # a row that only decodes
    drow.append(n_rows - 1)
    return wl, np.concatenate(ppos), np.concatenate(pseg), np.array(dpos), np.array(drow)


@pytest.mark.parametrize("seed", range(8))
def test_random_step_matches_oracle(seed):
    wl, ppos, pseg, dpos, drow = _draw(seed)
    m = wl.model
    kp, vp = device_pools(wl)
    pos = np.concatenate([ppos, dpos]).astype(np.int32)
    rows = np.concatenate([pseg, drow]).astype(np.int32)
    T, P = len(pos), len(ppos)
    qkv = W.normal_matrix(wl.key("qkv"), T, m.qkv_width, "cuda")
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda")) if m.qk_norm_eps else (None, None)
    h = handle_for(m)
    q_out, out = h.step_paged(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                              torch_i32(pos), torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=P,
                              n_segments=int(pseg.max()) + 1, q_gain=gains[0], k_gain=gains[1])
    torch.cuda.synchronize()
    g_np = (to_np_bits(gains[0]), to_np_bits(gains[1])) if m.qk_norm_eps else None
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), pos, g_np)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, f"seed {seed} q_out")
    slots = pages.slot_of(wl.table, rows, pos)
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, f"seed {seed} K pages")
    assert np.array_equal(to_np_bits(vg), v_bits), f"seed {seed}: V pages must be a bit copy"
    op = OraclePool(wl, "cuda")
    op.prefetch(wl.table.ravel())
    op.write(slots, k_bits, v_bits)
    ref = attention.paged(bf16.to_f64(q_bits), pos, rows, wl.table, op.read_page, m.window)
    check_close(to_np_bits(out), ref, f"seed {seed} ({hq}/{hkv}/{D} w{m.window} norm {m.qk_norm_eps} "
                                      f"llama3 {m.llama3 is not None})")
