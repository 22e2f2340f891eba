"""Output canaries: every entry writes only the outputs it owns.

Each output (out, and q_out where an entry returns it) is passed as a view
into a larger buffer filled with a canary pattern: rows longer than
Hq * D (ld_out / ld_q_out above the row width) and more rows than the call
has tokens. After the call, every canary element outside the view must be
untouched, and every element inside it must have been written (no canary
survives in a real output)."""
import zlib

import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W

from parity import device_pools, handle_for, torch_i32

pytestmark = pytest.mark.gpu

CANARY = 0x5A5A     # bf16 ~1.5e16: no output of these calls can equal it
PAD_COLS, PAD_ROWS = 72, 5


def _model(window=0, eps=1e-6):
    return W.ModelShape("canary", 16, 4, 128, 1e4, window=window, qk_norm_eps=eps, max_position=1024)


def _buffer(n, width):
    """A canary-filled [n + PAD_ROWS, width + PAD_COLS] buffer and the [n, width] view outputs go to."""
    buf = torch.full((n + PAD_ROWS, width + PAD_COLS), CANARY, dtype=torch.int16, device="cuda")
    return buf, buf[:n, :width]


def _check(buf, n, width, what):
    b = buf.cpu().numpy().view(np.uint16)
    assert np.all(b[:, width:] == CANARY), f"{what}: wrote past the row width"
    assert np.all(b[n:] == CANARY), f"{what}: wrote past the last row"
    assert not np.any(b[:n, :width] == CANARY), f"{what}: left an output element unwritten"


def _split(qkv, m):
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    return qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:]


def _setup(window=0):
    m = _model(window)
    rng = np.random.default_rng(zlib.crc32(b"canary"))
    n_rows, ppr = 4, 16
    wl = W.Workload(f"canary-{window}", m, n_rows * ppr, rng.permutation(n_rows * ppr).astype(np.int32)
                    .reshape(n_rows, ppr))
    kp, vp = device_pools(wl)
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    return m, wl, kp, vp, gains, handle_for(m)


@pytest.mark.parametrize("window", [0, 100])
def test_paged_entries_write_only_their_outputs(window):
    m, wl, kp, vp, (gq, gk), h = _setup(window)
    width = m.n_q_heads * m.head_dim
    table = torch_i32(wl.table)
    # write: 70 prompt tokens on rows 0-1
    pos = np.concatenate([np.arange(30), np.arange(200, 240)]).astype(np.int32)
    seg = np.repeat(np.array([0, 1], np.int32), [30, 40])
    T = len(pos)
    qkv = W.normal_matrix(wl.key("qkv"), T, m.qkv_width, "cuda")
    qbuf, q_out = _buffer(T, width)
    h.rope_qknorm_write_pages(*_split(qkv, m), torch_i32(pos), kp, vp, rows=torch_i32(seg), table=table,
                              q_out=q_out, q_gain=gq, k_gain=gk)
    obuf, out = _buffer(T, width)
    h.attn_prefill_packed(q_out, torch_i32(pos), torch_i32(seg), table, kp, vp, n_segments=2, out=out)
    dpos = np.array([500, 1023, 64], np.int32)
    drow = np.array([2, 3, 1], np.int32)
    dbuf, dout = _buffer(3, width)
    qd = W.normal_matrix(wl.key("qd"), 3, width, "cuda")
    h.attn_decode_paged(qd, torch_i32(dpos), table, kp, vp, rows=torch_i32(drow), out=dout)
    torch.cuda.synchronize()
    _check(qbuf, T, width, "rope_qknorm_write_pages q_out")
    _check(obuf, T, width, "attn_prefill_packed out")
    _check(dbuf, 3, width, "attn_decode_paged out")

    # step_paged, with prompt tokens and without (the decode-step form)
    for n_prompt in (T, 0):
        spos = np.concatenate([pos[:n_prompt], dpos]).astype(np.int32)
        srow = np.concatenate([seg[:n_prompt], drow]).astype(np.int32)
        n = len(spos)
        x = W.normal_matrix(wl.key("qkv", "step", n_prompt), n, m.qkv_width, "cuda")
        sq_buf, sq = _buffer(n, width)
        so_buf, so = _buffer(n, width)
        h.step_paged(*_split(x, m), torch_i32(spos), torch_i32(srow), table, kp, vp, n_prompt=n_prompt,
                     n_segments=2, q_gain=gq, k_gain=gk, q_out=sq, out=so)
        torch.cuda.synchronize()
        _check(sq_buf, n, width, f"step_paged q_out (n_prompt {n_prompt})")
        _check(so_buf, n, width, f"step_paged out (n_prompt {n_prompt})")


def test_cache_and_inpass_entries_write_only_their_outputs():
    m = _model()
    width = m.n_q_heads * m.head_dim
    h = handle_for(m)
    gq = W.uniform_bf16(W.stream_key("canary-gain", "q"), torch.arange(128, device="cuda"), 0.5, 1.5)
    gk = W.uniform_bf16(W.stream_key("canary-gain", "k"), torch.arange(128, device="cuda"), 0.5, 1.5)
    rows, max_seq = 3, 512
    kp, vp = dap.pools(rows * max_seq // 64, m.n_kv_heads, m.head_dim)
    kp.zero_()
    vp.zero_()

    def qkv(n, tag):
        return _split(W.normal_matrix(W.stream_key("canary", tag), n, m.qkv_width, "cuda"), m)

    calls = []
    buf, out = _buffer(rows * 40, width)        # prefill: 40 tokens per row at 0..39
    h.prefill(*qkv(rows * 40, "prefill"), 0, kp, vp, cache_rows=rows, max_seq=max_seq, q_gain=gq, k_gain=gk,
              out=out)
    calls.append((buf, rows * 40, "prefill"))
    buf, out = _buffer(rows, width)
    h.decode(*qkv(rows, "decode"), 40, kp, vp, max_seq=max_seq, q_gain=gq, k_gain=gk, out=out)
    calls.append((buf, rows, "decode"))
    buf, out = _buffer(rows, width)
    h.decode_rows(*qkv(rows, "decode_rows"), torch_i32(np.array([41, 300, 511], np.int32)), kp, vp,
                  max_seq=max_seq, q_gain=gq, k_gain=gk, out=out)
    calls.append((buf, rows, "decode_rows"))
    buf, out = _buffer(2 * 33, width)
    h.prefill_slots(*qkv(2 * 33, "prefill_slots"), torch_i32(np.array([2, 0], np.int32)), kp, vp,
                    cache_rows=rows, max_seq=max_seq, q_gain=gq, k_gain=gk, out=out)
    calls.append((buf, 2 * 33, "prefill_slots"))
    lens = [17, 64, 100]
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    seg = np.repeat(np.arange(3, dtype=np.int32), lens)
    buf, out = _buffer(len(pos), width)
    h.packed(*qkv(len(pos), "packed"), torch_i32(pos), torch_i32(seg), n_segments=3, q_gain=gq, k_gain=gk, out=out)
    calls.append((buf, len(pos), "packed"))
    buf, out = _buffer(2 * 70, width)
    h.forward(*qkv(2 * 70, "forward"), 2, q_gain=gq, k_gain=gk, out=out)
    calls.append((buf, 2 * 70, "forward"))
    torch.cuda.synchronize()
    for buf, n, what in calls:
        _check(buf, n, width, what)
