"""GPU parity on the five model-shaped workloads at full size, in the launch
configuration the benchmark times (same entries, same shapes).

Every token's written q_out and K are compared bit for bit against the
oracle's rounding (only elements the oracle flags as lying on a bf16
rounding midpoint may differ, by one ulp) and V exactly. Attention outputs
are compared element by element: every decode row (Mistral, Qwen3), every
prompt token (Phi-3, Qwen3) and, for the 8192-token Llama chunk, a
stratified sample that holds a token of each 32-row half of every one of its
128 tiles. Each full-size prefill and decode is run again with the queries
scaled by 4 (the peaky variant: the softmax then concentrates on a few keys,
so a dropped key cannot hide in a near-uniform average)."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, pages

from parity import (OraclePool, check_bits, check_close, device_pools, handle_for, oracle_attention,
                    oracle_front, oracle_rows, to_np_bits, torch_i32)

pytestmark = pytest.mark.gpu


def _split(qkv, m):
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    return qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:]


def _gains(wl):
    if not wl.model.qk_norm_eps:
        return None, None
    g = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    return g, (to_np_bits(g[0]), to_np_bits(g[1]))


def _peaky(q):
    """The same queries scaled by 4 (exact in bf16)."""
    return (q.view(torch.bfloat16).float() * 4).to(torch.bfloat16)


def _check_written(wl, kp, vp, slots, k_bits, v_bits, what):
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, what + " K")
    assert np.array_equal(to_np_bits(vg), v_bits), what + " V must be a bit copy"


def test_phi3_prefill_then_decode_loop():
    wl = W.phi3()
    m = wl.model
    h = handle_for(m)
    kp, vp = device_pools(wl)
    op = OraclePool(wl, "cuda")
    table = torch_i32(wl.table)
    T = wl.n_pre
    qkv = wl.qkv("prompt", T, "cuda")
    pos, seg = torch_i32(wl.pre_positions), torch_i32(wl.pre_segments)
    q_out = h.rope_qknorm_write_pages(*_split(qkv, m), pos, kp, vp, rows=seg, table=table)
    out = h.attn_prefill_packed(q_out, pos, seg, table, kp, vp, n_segments=4)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), wl.pre_positions)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, "prompt q_out")
    slots = pages.slot_of(wl.table, wl.pre_segments, wl.pre_positions)
    _check_written(wl, kp, vp, slots, k_bits, v_bits, "prompt")
    op.write(slots, k_bits, v_bits)
    # every prompt token, and every one again with the queries scaled by 4
    out4 = h.attn_prefill_packed(_peaky(q_out), pos, seg, table, kp, vp, n_segments=4)
    torch.cuda.synchronize()
    qf = bf16.to_f64(q_bits)
    ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], wl.pre_positions, wl.pre_segments)
    check_close(to_np_bits(out), ref, "phi3 prefill (all 4096 tokens)")
    check_close(to_np_bits(out4), ref4, "phi3 prefill peaky (all 4096 tokens)")

    # decode loop: every step writes its active rows' tokens and attends
    steps = W.phi3_decode_schedule()
    sample_steps = {0, 1, 463, 464, 465, 1000, 1463, 1464, 1465, 1975, 1976, 1977, 2400, 2488}
    ws = h.workspace(h.decode_workspace_bytes(4))
    kept = {}
    all_slots, all_tok = [], []
    for t, (rows, positions) in enumerate(steps):
        x = wl.qkv("step", len(rows), "cuda", row0=4 * t)
        tp, tr = torch_i32(positions), torch_i32(rows)
        qo = h.rope_qknorm_write_pages(*_split(x, m), tp, kp, vp, rows=tr, table=table)
        o = h.attn_decode_paged(qo, tp, table, kp, vp, rows=tr, workspace=ws)
        if t in sample_steps:
            o4 = h.attn_decode_paged(_peaky(qo), tp, table, kp, vp, rows=tr, workspace=ws)
            kept[t] = (x.clone(), o.clone(), o4.clone())
        all_tok.append((t, rows, positions))
    torch.cuda.synchronize()
    # the oracle writes every decode token (its own k/v) and checks sampled steps
    for t, rows, positions in all_tok:
        x = wl.qkv("step", len(rows), "cpu", row0=4 * t).numpy().view(np.uint16)
        _, qb, kb, vb = oracle_front(wl, x, positions)
        s = pages.slot_of(wl.table, rows, positions)
        op.write(s, kb, vb)
        if t in kept:
            assert np.array_equal(to_np_bits(kept[t][0]), x)
            qf = bf16.to_f64(qb)
            ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], positions, rows)
            check_close(to_np_bits(kept[t][1]), ref, f"phi3 decode step {t}")
            check_close(to_np_bits(kept[t][2]), ref4, f"phi3 decode step {t}, peaky")
    # read-only measurement call: all four rows at 3000
    q = W.normal_matrix(wl.key("q", "final"), 4, m.n_q_heads * m.head_dim, "cuda")
    p3000 = np.full(4, 3000, np.int32)
    o = h.attn_decode_paged(q, torch_i32(p3000), table, kp, vp, workspace=ws)
    o4 = h.attn_decode_paged(_peaky(q), torch_i32(p3000), table, kp, vp, workspace=ws)
    torch.cuda.synchronize()
    qf = bf16.to_f64(to_np_bits(q)).reshape(4, m.n_q_heads, m.head_dim)
    ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], p3000, np.arange(4))
    check_close(to_np_bits(o), ref, "phi3 decode at 3000")
    check_close(to_np_bits(o4), ref4, "phi3 decode at 3000, peaky")
    # every position 0..3000 of every row, bit for bit against the oracle's pool
    for r in range(4):
        sl = pages.slot_of(wl.table, np.full(3001, r), np.arange(3001))
        kg, vg = dap.gather_slots(kp, vp, sl)
        ko = np.stack([op.read_page(int(s) // 64)[0][:, int(s) % 64] for s in sl])
        vo = np.stack([op.read_page(int(s) // 64)[1][:, int(s) % 64] for s in sl])
        check_bits(to_np_bits(kg), bf16.from_f64(ko), f"row {r} K after the loop")
        assert np.array_equal(to_np_bits(vg), bf16.from_f64(vo))


def test_mistral_decode():
    wl = W.mistral()
    m = wl.model
    h = handle_for(m)
    kp, vp = device_pools(wl)
    table = torch_i32(wl.table)
    R = wl.n_dec
    qkv = wl.qkv("step", R, "cuda")
    pos, rows = torch_i32(wl.dec_positions), torch_i32(wl.dec_rows)
    q_out = h.rope_qknorm_write_pages(*_split(qkv, m), pos, kp, vp, rows=rows, table=table)
    out = h.attn_decode_paged(q_out, pos, table, kp, vp)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), wl.dec_positions)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, "q_out")
    slots = pages.slot_of(wl.table, wl.dec_rows, wl.dec_positions)
    _check_written(wl, kp, vp, slots, k_bits, v_bits, "new token")
    op = OraclePool(wl, "cuda")
    op.write(slots, k_bits, v_bits)
    # every row, and every row again with the queries scaled by 4
    out4 = h.attn_decode_paged(_peaky(q_out), pos, table, kp, vp)
    torch.cuda.synchronize()
    qf = bf16.to_f64(q_bits)
    ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], wl.dec_positions, wl.dec_rows)
    check_close(to_np_bits(out), ref, "mistral decode (all 64 rows)")
    check_close(to_np_bits(out4), ref4, "mistral decode peaky (all 64 rows)")


def test_llama31_chunked_prefill():
    wl = W.llama31()
    m = wl.model
    h = handle_for(m)
    kp, vp = device_pools(wl)
    table = torch_i32(wl.table)
    T = wl.n_pre
    qkv = wl.qkv("chunk", T, "cuda")
    pos, seg = torch_i32(wl.pre_positions), torch_i32(wl.pre_segments)
    q_out = h.rope_qknorm_write_pages(*_split(qkv, m), pos, kp, vp, rows=seg, table=table)
    out = h.attn_prefill_packed(q_out, pos, seg, table, kp, vp, n_segments=1)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), wl.pre_positions)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, "q_out")
    slots = pages.slot_of(wl.table, wl.pre_segments, wl.pre_positions)
    _check_written(wl, kp, vp, slots, k_bits, v_bits, "chunk")
    op = OraclePool(wl, "cuda")
    op.write(slots, k_bits, v_bits)
    # one token from each 32-row half of every 64-token tile (the tile a
    # workgroup takes at head_dim 128 and 4 query heads per kv head), plus
    # both ends of the chunk and of its page and tile edges
    rng = np.random.default_rng(2)
    halves = np.arange(0, T, 32)
    pick = np.unique(np.concatenate([halves + rng.integers(0, 32, halves.size), np.arange(4), np.arange(T - 4, T),
                                     [31, 32, 63, 64, 4095, 4096]]))
    assert pick.size >= 256
    out4 = h.attn_prefill_packed(_peaky(q_out), pos, seg, table, kp, vp, n_segments=1)
    torch.cuda.synchronize()
    qf = bf16.to_f64(q_bits[pick])
    ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], wl.pre_positions[pick], wl.pre_segments[pick])
    check_close(to_np_bits(out)[pick], ref, f"llama31 prefill ({pick.size} tokens, every tile)")
    check_close(to_np_bits(out4)[pick], ref4, f"llama31 prefill peaky ({pick.size} tokens, every tile)")


def test_qwen3_step_paged():
    wl = W.qwen3()
    m = wl.model
    h = handle_for(m)
    kp, vp = device_pools(wl)
    table = torch_i32(wl.table)
    P, R = wl.n_pre, wl.n_dec
    qkv = wl.qkv("step", P + R, "cuda")
    pos = torch_i32(np.concatenate([wl.pre_positions, wl.dec_positions]))
    rows = torch_i32(np.concatenate([wl.pre_segments, wl.dec_rows]))
    (g, g_np) = _gains(wl)
    q_out, out = h.step_paged(*_split(qkv, m), pos, rows, table, kp, vp, n_prompt=P, n_segments=8,
                              q_gain=g[0], k_gain=g[1])
    torch.cuda.synchronize()
    all_pos = np.concatenate([wl.pre_positions, wl.dec_positions])
    all_rows = np.concatenate([wl.pre_segments, wl.dec_rows])
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), all_pos, g_np)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, "q_out")
    slots = pages.slot_of(wl.table, all_rows, all_pos)
    _check_written(wl, kp, vp, slots, k_bits, v_bits, "step")
    op = OraclePool(wl, "cuda")
    op.write(slots, k_bits, v_bits)
    # every prompt token and every decode row, and all of them again with the
    # queries scaled by 4 (through the prefill and decode the step runs)
    q4 = _peaky(q_out)
    o4_pre = h.attn_prefill_packed(q4[:P], pos[:P], rows[:P], table, kp, vp, n_segments=8)
    o4_dec = h.attn_decode_paged(q4[P:], pos[P:], table, kp, vp, rows=rows[P:])
    torch.cuda.synchronize()
    qf = bf16.to_f64(q_bits)
    ref, ref4 = oracle_rows(wl, op, [qf, 4 * qf], all_pos, all_rows)
    check_close(to_np_bits(out)[:P], ref[:P], "qwen3 prefill part (all 2048 tokens)")
    check_close(to_np_bits(out)[P:], ref[P:], "qwen3 decode part (all 128 rows)")
    check_close(to_np_bits(o4_pre), ref4[:P], "qwen3 prefill part peaky (all 2048 tokens)")
    check_close(to_np_bits(o4_dec), ref4[P:], "qwen3 decode part peaky (all 128 rows)")
    # the composition equals the three entries called one after another
    ws_d = h.workspace(h.decode_workspace_bytes(R))
    o_pre = h.attn_prefill_packed(q_out[:P], pos[:P], rows[:P], table, kp, vp, n_segments=8)
    o_dec = h.attn_decode_paged(q_out[P:], pos[P:], table, kp, vp, rows=rows[P:], workspace=ws_d)
    torch.cuda.synchronize()
    assert torch.equal(o_pre.view(torch.int16), out[:P].view(torch.int16))
    assert torch.equal(o_dec.view(torch.int16), out[P:].view(torch.int16))


def test_mistral_contiguous_decode_rows():
    """The Mistral rows through dap_decode_rows on a contiguous cache (the
    identity table), at full size: written token bits and every row."""
    wl = W.mistral_contiguous()
    m = wl.model
    h = handle_for(m)
    kp, vp = device_pools(wl)
    R = wl.n_dec
    max_seq = wl.table.shape[1] * 64
    qkv = wl.qkv("step", R, "cuda")
    out = h.decode_rows(*_split(qkv, m), torch_i32(wl.dec_positions), kp, vp, max_seq=max_seq)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), wl.dec_positions)
    slots = pages.slot_of(wl.table, wl.dec_rows, wl.dec_positions)
    _check_written(wl, kp, vp, slots, k_bits, v_bits, "contiguous new token")
    op = OraclePool(wl, "cuda")
    op.write(slots, k_bits, v_bits)
    ref, = oracle_rows(wl, op, [bf16.to_f64(q_bits)], wl.dec_positions, wl.dec_rows)
    check_close(to_np_bits(out), ref, "contiguous decode (all 64 rows)")


def test_packed_training_forward():
    """8 Llama-3.1-shaped prompts of 4096 tokens through dap_packed at full
    size: sampled query tokens of every prompt (first, last and a spread)
    against the oracle's in-pass attention over the prompt's own keys."""
    wl = W.packed_train()
    m = wl.model
    h = handle_for(m)
    T = wl.n_pre
    qkv = wl.qkv("train", T, "cuda")
    pos, seg = wl.pre_positions, wl.pre_segments
    out = h.packed(*_split(qkv, m), torch_i32(pos), torch_i32(seg), n_segments=8)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), pos)
    qf, kf, vf = bf16.to_f64(q_bits), bf16.to_f64(k_bits), bf16.to_f64(v_bits)
    got = to_np_bits(out)
    rng = np.random.default_rng(3)
    picks, refs = [], []
    for sgi in range(8):
        idx = np.nonzero(seg == sgi)[0]
        idx = idx[np.argsort(pos[idx])]
        K, V = np.swapaxes(kf[idx], 0, 1), np.swapaxes(vf[idx], 0, 1)
        sample = np.unique(np.concatenate([[0, 1, 63, 64, len(idx) - 1], rng.choice(len(idx), 6, replace=False)]))
        for k in sample:
            t = idx[k]
            picks.append(t)
            refs.append(attention.attend_one(qf[t], K, V, int(pos[t]), m.window))
    check_close(got[np.array(picks)], np.stack(refs), "packed training forward (sampled tokens)")
