"""The tiny single-layer workload end to end on the GPU: Hq 4, Hkv 2, D 64,
theta 1e4, no window; a 128-token prompt written and prefilled, then 16
decode steps at positions 128..143, each writing its token and attending.
Run over the identity page table (the contiguous cache) and a permuted one;
both must match the oracle, which computes everything from the same qkv."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, pages

from parity import (OraclePool, check_bits, check_close, device_pools, handle_for, oracle_front,
                    to_np_bits, torch_i32)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("permuted", [False, True])
def test_tiny_prefill_then_decode(permuted):
    wl = W.tiny(permuted)
    m = wl.model
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    h = handle_for(m)
    kp, vp = device_pools(wl)
    op = OraclePool(wl, "cuda")
    table = torch_i32(wl.table)

    # prompt: write, then packed prefill
    qkv = W.normal_matrix(wl.key("qkv", "prompt"), 128, m.qkv_width, "cuda")
    pos = wl.pre_positions
    seg = wl.pre_segments
    q_out = h.rope_qknorm_write_pages(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                                      torch_i32(pos), kp, vp, rows=torch_i32(seg), table=table)
    out = h.attn_prefill_packed(q_out, torch_i32(pos), torch_i32(seg), table, kp, vp, n_segments=1)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), pos)
    check_bits(to_np_bits(q_out).reshape(128, hq, D), q_bits, "prompt q_out")
    op.write(pages.slot_of(wl.table, seg, pos), k_bits, v_bits)
    ref = attention.paged(bf16.to_f64(q_bits), pos, seg, wl.table, op.read_page, m.window)
    check_close(to_np_bits(out), ref, "prompt prefill")

    # 16 decode steps
    for step in range(16):
        p = np.array([128 + step], np.int32)
        r = np.zeros(1, np.int32)
        x = W.normal_matrix(wl.key("qkv", "step"), 1, m.qkv_width, "cuda", row0=step)
        qo = h.rope_qknorm_write_pages(x[:, :hq * D], x[:, hq * D:(hq + hkv) * D], x[:, (hq + hkv) * D:],
                                       torch_i32(p), kp, vp, rows=torch_i32(r), table=table)
        o = h.attn_decode_paged(qo, torch_i32(p), table, kp, vp)
        torch.cuda.synchronize()
        _, qb, kb, vb = oracle_front(wl, to_np_bits(x), p)
        op.write(pages.slot_of(wl.table, r, p), kb, vb)
        ref = attention.paged(bf16.to_f64(qb), p, r, wl.table, op.read_page, m.window)
        check_close(to_np_bits(o), ref, f"decode step {step}")
    # the pool now holds positions 0..143: read it back bit for bit
    slots = pages.slot_of(wl.table, np.zeros(144, int), np.arange(144))
    kg, vg = dap.gather_slots(kp, vp, slots)
    ko = np.stack([op.read_page(int(s) // 64)[0][:, int(s) % 64] for s in slots])
    vo = np.stack([op.read_page(int(s) // 64)[1][:, int(s) % 64] for s in slots])
    check_bits(to_np_bits(kg), bf16.from_f64(ko), "K pool after 144 writes")
    assert np.array_equal(to_np_bits(vg), bf16.from_f64(vo))
