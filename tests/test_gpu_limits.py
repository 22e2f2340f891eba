"""Largest sizes and degenerate cases through the C ABI: the largest position
a handle accepts, the most rows one decode call takes, the largest head
group, and the cases whose answer is a stored value (one visible key)."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import bf16

from parity import (OraclePool, check_close, device_pools, handle_for, oracle_attention, to_np_bits, torch_i32)

pytestmark = pytest.mark.gpu

MAX_POSITION = 1 << 22


def test_decode_at_the_largest_position_with_the_largest_group():
    """One row at position 4194303 over 65536 pages, 16 query heads per kv head."""
    m = W.ModelShape("lim-maxpos", 16, 1, 64, 1e4, max_position=MAX_POSITION)
    n_pages = MAX_POSITION // 64
    table = np.random.default_rng(11).permutation(n_pages).astype(np.int32).reshape(1, n_pages)
    wl = W.Workload("lim-maxpos", m, n_pages, table)
    kp, vp = device_pools(wl)
    h = handle_for(m, validate=True)
    pos = np.array([MAX_POSITION - 1], np.int32)
    q = W.normal_matrix(wl.key("q"), 1, m.n_q_heads * m.head_dim, "cuda")
    # sharpen the scores so a few keys dominate and a dropped page would show
    q = (q.view(torch.bfloat16).float() * 3.0).to(torch.bfloat16).view(torch.int16)
    out = h.attn_decode_paged(q, torch_i32(pos), torch_i32(table), kp, vp)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    ref = oracle_attention(wl, op, bf16.to_f64(to_np_bits(q)).reshape(1, 16, 64), pos, np.zeros(1, np.int32))
    check_close(to_np_bits(out), ref, "decode at position 4194303")


def test_decode_with_the_most_rows_one_call_takes():
    """65535 rows (the call's limit); a spread of 256 rows against the oracle."""
    m = W.ModelShape("lim-rows", 8, 2, 64, 1e4, max_position=256)
    R, ppr = 65535, 4
    rng = np.random.default_rng(12)
    n_pages = 8192
    table = rng.integers(0, n_pages, size=(R, ppr)).astype(np.int32)      # rows may share pages (read only)
    wl = W.Workload("lim-rows", m, n_pages, table)
    kp, vp = device_pools(wl)
    h = handle_for(m)
    pos = rng.integers(0, 256, size=R).astype(np.int32)
    q = W.normal_matrix(wl.key("q"), R, m.n_q_heads * m.head_dim, "cuda")
    out = h.attn_decode_paged(q, torch_i32(pos), torch_i32(table), kp, vp)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, R - 1], rng.choice(R, 254, replace=False)]))
    op = OraclePool(wl, "cuda")
    qf = bf16.to_f64(to_np_bits(q[torch.as_tensor(pick, device="cuda")])).reshape(len(pick), 8, 64)
    ref = oracle_attention(wl, op, qf, pos[pick], pick.astype(np.int32))
    check_close(to_np_bits(out)[pick], ref, "decode of 65535 rows, sampled")
    with pytest.raises(dap.DapError) as e:
        h.attn_decode_paged(torch.zeros(R + 1, 512, dtype=torch.int16, device="cuda"),
                            torch_i32(np.zeros(R + 1)), torch_i32(table), kp, vp)
    assert e.value.status == dap.UNSUPPORTED


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (8, 2, 128), (4, 4, 96)])
def test_window_of_one_returns_each_token_its_own_value(hq, hkv, d):
    """Window 1: each query sees only its own key, so the output is exactly
    its own V (softmax of one score is 1), bit for bit, in the prefill and
    in the decode."""
    m = W.ModelShape(f"lim-w1-{d}", hq, hkv, d, 1e4, window=1, max_position=512)
    table = np.arange(8, dtype=np.int32).reshape(1, 8)
    wl = W.Workload(m.name, m, 8, table)
    kp, vp = device_pools(wl)
    h = handle_for(m)
    T = 300
    pos = np.arange(100, 100 + T, dtype=np.int32)
    qkv = wl.qkv("w1", T, "cuda")
    D = d
    qo = h.rope_qknorm_write_pages(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                                   torch_i32(pos), kp, vp, rows=torch_i32(np.zeros(T)), table=torch_i32(table))
    out_p = h.attn_prefill_packed(qo, torch_i32(pos), torch_i32(np.zeros(T)), torch_i32(table), kp, vp, n_segments=1)
    out_d = h.attn_decode_paged(qo[-3:], torch_i32(pos[-3:]), torch_i32(table), kp, vp, rows=torch_i32([0, 0, 0]))
    torch.cuda.synchronize()
    v = to_np_bits(qkv[:, (hq + hkv) * D:]).reshape(T, hkv, 1, D)
    want = np.broadcast_to(v, (T, hkv, hq // hkv, D)).reshape(T, hq * D)
    assert np.array_equal(to_np_bits(out_p), want), "prefill with window 1 must return the token's own V"
    assert np.array_equal(to_np_bits(out_d), want[-3:]), "decode with window 1 must return the token's own V"


def test_first_position_returns_the_first_value():
    """A token at position 0 sees one key: the output is that token's V."""
    m = W.ModelShape("lim-p0", 8, 2, 128, 1e4, max_position=256)
    table = np.array([[3, 1, 0, 2]], np.int32)
    wl = W.Workload(m.name, m, 4, table)
    kp, vp = device_pools(wl)
    h = handle_for(m)
    qkv = wl.qkv("p0", 1, "cuda")
    hq, hkv, D = 8, 2, 128
    qo = h.rope_qknorm_write_pages(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                                   torch_i32([0]), kp, vp, rows=torch_i32([0]), table=torch_i32(table))
    out_p = h.attn_prefill_packed(qo, torch_i32([0]), torch_i32([0]), torch_i32(table), kp, vp, n_segments=1)
    out_d = h.attn_decode_paged(qo, torch_i32([0]), torch_i32(table), kp, vp)
    torch.cuda.synchronize()
    v = to_np_bits(qkv[:, (hq + hkv) * D:]).reshape(1, hkv, 1, D)
    want = np.broadcast_to(v, (1, hkv, hq // hkv, D)).reshape(1, hq * D)
    assert np.array_equal(to_np_bits(out_p), want) and np.array_equal(to_np_bits(out_d), want)
