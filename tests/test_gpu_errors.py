"""Error paths and edge cases through the C ABI on the GPU.

Validate mode checks index arrays on the host before any kernel runs, so
the bad inputs here never reach a kernel there. Without validate mode the
kernels' own bounds checks skip an out-of-range page id; the test checks the
other rows are untouched by it."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16

from parity import OraclePool, check_close, device_pools, handle_for, to_np_bits, torch_i32

pytestmark = pytest.mark.gpu


def _setup(window=0, rows=4, ppr=8, hq=8, hkv=2, d=128):
    m = W.ModelShape(f"err-{window}", hq, hkv, d, 1e4, window=window, max_position=ppr * 64)
    rng = np.random.default_rng(3)
    table = rng.permutation(rows * ppr).astype(np.int32).reshape(rows, ppr)
    wl = W.Workload(m.name, m, rows * ppr, table)
    kp, vp = device_pools(wl)
    return wl, m, kp, vp


def test_validate_mode_accepts_good_inputs_and_rejects_bad_ones():
    wl, m, kp, vp = _setup()
    h = handle_for(m, validate=True)
    q = W.normal_matrix(wl.key("q"), 4, m.n_q_heads * m.head_dim, "cuda")
    pos = torch_i32([10, 200, 511, 64])
    table = torch_i32(wl.table)
    h.attn_decode_paged(q, pos, table, kp, vp)                     # fine
    torch.cuda.synchronize()
    with pytest.raises(dap.DapError) as e:                        # position past max_position
        h.attn_decode_paged(q, torch_i32([10, 200, 512, 64]), table, kp, vp)
    assert e.value.status == dap.BAD_INDEX
    bad = wl.table.copy()
    bad[2, 3] = wl.n_pages                                         # page id out of range
    with pytest.raises(dap.DapError) as e:
        h.attn_decode_paged(q, pos, torch_i32(bad), kp, vp)
    assert e.value.status == dap.BAD_INDEX
    with pytest.raises(dap.DapError) as e:                        # table row out of range
        h.attn_decode_paged(q, pos, table, kp, vp, rows=torch_i32([0, 1, 4, 2]))
    assert e.value.status == dap.BAD_INDEX
    # the write: two tokens on one slot
    qkv = W.normal_matrix(wl.key("qkv"), 2, m.qkv_width, "cuda")
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    parts = (qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:])
    with pytest.raises(dap.DapError) as e:
        h.rope_qknorm_write_pages(*parts, torch_i32([5, 5]), kp, vp, rows=torch_i32([1, 1]), table=table)
    assert e.value.status == dap.BAD_INDEX
    with pytest.raises(dap.DapError) as e:
        h.rope_qknorm_write_pages(*parts, torch_i32([5, 6]), kp, vp, slots=torch_i32([7, 7]))
    assert e.value.status == dap.BAD_INDEX
    # the prefill: more runs of equal segments than n_segments says
    seg = torch_i32([0, 1, 0, 1])
    with pytest.raises(dap.DapError) as e:
        h.attn_prefill_packed(q, torch_i32([0, 0, 1, 1]), seg, table, kp, vp, n_segments=2)
    assert e.value.status == dap.BAD_INDEX
    h.attn_prefill_packed(q, torch_i32([0, 0, 1, 1]), seg, table, kp, vp, n_segments=4)   # fine
    torch.cuda.synchronize()


def test_argument_checks():
    wl, m, kp, vp = _setup()
    h = handle_for(m)
    q = W.normal_matrix(wl.key("q"), 4, m.n_q_heads * m.head_dim, "cuda")
    pos = torch_i32([10, 200, 511, 64])
    table = torch_i32(wl.table)
    with pytest.raises(dap.DapError) as e:                        # workspace too small
        h.attn_decode_paged(q, pos, table, kp, vp, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == dap.WORKSPACE_TOO_SMALL
    with pytest.raises(dap.DapError) as e:                        # out aliases q
        h.attn_decode_paged(q, pos, table, kp, vp, out=q)
    assert e.value.status == dap.INVALID_ARG
    with pytest.raises(dap.DapError) as e:                        # row stride not a multiple of 8
        h.attn_decode_paged(torch.empty(4, 1028, dtype=torch.int16, device="cuda")[:, :1024], pos, table, kp, vp)
    assert e.value.status == dap.INVALID_ARG
    g = handle_for(W.ModelShape("g8", 16, 2, 128, 1e4, max_position=512))   # group 8: decode only
    with pytest.raises(dap.DapError) as e:
        g.attn_prefill_packed(torch.zeros(4, 2048, dtype=torch.int16, device="cuda"), torch_i32([0, 1, 2, 3]),
                              torch_i32([0, 0, 0, 0]), table, kp, vp, n_segments=1)
    assert e.value.status == dap.UNSUPPORTED


def test_binding_refuses_tensors_the_kernels_would_overrun():
    """The C side sees pointers and the sizes the binding derives; tensors
    that are too short, on the host, or shaped for another model are refused
    before any kernel runs."""
    wl, m, kp, vp = _setup()
    h = handle_for(m)
    width = m.n_q_heads * m.head_dim
    q = W.normal_matrix(wl.key("q"), 4, width, "cuda")
    pos = torch_i32([10, 200, 511, 64])
    table = torch_i32(wl.table)
    bad_calls = {
        "q on the host": lambda: h.attn_decode_paged(q.cpu(), pos, table, kp, vp),
        "q with fewer rows than positions": lambda: h.attn_decode_paged(q[:3], pos, table, kp, vp),
        "q narrower than Hq*D": lambda: h.attn_decode_paged(q[:, :width - 8], pos, table, kp, vp),
        "out with fewer rows": lambda: h.attn_decode_paged(q, pos, table, kp, vp, out=torch.empty_like(q)[:2]),
        "pool for another kv head count": lambda: h.attn_decode_paged(q, pos, table, kp.view(-1, 1, kp.shape[-1]),
                                                                      vp.view(-1, 1, vp.shape[-1])),
        "pools of different sizes": lambda: h.attn_decode_paged(q, pos, table, kp, vp[:-1]),
        "segments shorter than the tokens": lambda: h.attn_prefill_packed(q, pos, pos[:2], table, kp, vp,
                                                                         n_segments=4),
        "table on the host": lambda: h.attn_decode_paged(q, pos, table.cpu(), kp, vp),
        "workspace on the host": lambda: h.attn_decode_paged(q, pos, table, kp, vp,
                                                            workspace=torch.zeros(1 << 20, dtype=torch.uint8)),
        "cache pool smaller than rows x max_seq": lambda: h.decode(q, q[:, :m.n_kv_heads * m.head_dim],
                                                                   q[:, :m.n_kv_heads * m.head_dim], 5, kp, vp,
                                                                   max_seq=kp.shape[0] * 64),
    }
    for what, call in bad_calls.items():
        with pytest.raises(dap.DapError) as e:
            call()
        assert e.value.status == dap.INVALID_ARG, what
    torch.cuda.synchronize()


def test_empty_calls_are_no_ops():
    wl, m, kp, vp = _setup()
    h = handle_for(m, validate=True)
    e32 = torch.zeros(0, dtype=torch.int32, device="cuda")
    q = torch.zeros(0, m.n_q_heads * m.head_dim, dtype=torch.int16, device="cuda")
    table = torch_i32(wl.table)
    h.attn_decode_paged(q, e32, table, kp, vp)
    h.attn_prefill_packed(q, e32, e32, table, kp, vp, n_segments=1)
    qkv = torch.zeros(0, m.qkv_width, dtype=torch.int16, device="cuda")
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    h.rope_qknorm_write_pages(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:], e32,
                              kp, vp, rows=e32, table=table)
    torch.cuda.synchronize()


def test_out_of_range_page_is_skipped_and_other_rows_are_untouched():
    wl, m, kp, vp = _setup()
    h = handle_for(m)                      # no validate: the kernels' own bounds checks act
    bad = wl.table.copy()
    bad[1, 2] = 1 << 30
    q = W.normal_matrix(wl.key("q"), 4, m.n_q_heads * m.head_dim, "cuda")
    pos = np.array([300, 300, 300, 300], np.int32)
    out = h.attn_decode_paged(q, torch_i32(pos), torch_i32(bad), kp, vp)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    good_rows = np.array([0, 2, 3])
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(4, m.n_q_heads, m.head_dim)[good_rows],
                          pos[good_rows], good_rows, wl.table, op.read_page, 0)
    check_close(to_np_bits(out)[good_rows], ref, "rows beside the bad page id")


def test_calls_follow_the_current_stream():
    wl, m, kp, vp = _setup()
    h = handle_for(m)
    s = torch.cuda.Stream()
    q = W.normal_matrix(wl.key("q"), 4, m.n_q_heads * m.head_dim, "cuda")
    pos = torch_i32([10, 200, 511, 64])
    table = torch_i32(wl.table)
    ref = h.attn_decode_paged(q, pos, table, kp, vp)
    torch.cuda.synchronize()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q2 = q.clone()                     # produced on s, consumed on s
        out = h.attn_decode_paged(q2, pos, table, kp, vp)
        res = out.clone()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(res, ref)
