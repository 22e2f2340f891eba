"""GPU parity of each entry on small seeded inputs that span several tiles,
ragged tails, page edges, windows and every supported head shape.

Inputs come straight from the generators (bf16 N(0,1) queries, pools of
generated pages), so both sides see identical bits; the oracle is the fp64
definition in oracle/."""
import zlib

import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, core, pages

from parity import (OraclePool, check_bits, check_close, device_pools, handle_for, oracle_front,
                    to_np_bits, torch_i32)

pytestmark = pytest.mark.gpu


def _model(hq, hkv, d, window=0, max_position=4096, theta=1e4, llama3=None, eps=None):
    return W.ModelShape(f"unit-{hq}-{hkv}-{d}-{window}", hq, hkv, d, theta, window=window, llama3=llama3,
                        qk_norm_eps=eps, max_position=max_position)


def _workload(model, n_rows, n_pages_per_row, tag, shared=0):
    """Rows with their own pages from one seeded permutation."""
    rng = np.random.default_rng(zlib.crc32(tag.encode()))
    n_pages = n_rows * n_pages_per_row
    perm = rng.permutation(n_pages).astype(np.int32)
    table = perm.reshape(n_rows, n_pages_per_row)
    return W.Workload(tag, model, n_pages, table)


def _queries(wl, n, scale=1.0, tag="q"):
    q = W.normal_matrix(wl.key(tag), n, wl.model.n_q_heads * wl.model.head_dim, "cuda")
    if scale != 1.0:
        q = (q.view(torch.bfloat16).float() * scale).to(torch.bfloat16).view(torch.int16)
    return q


DECODE_SHAPES = [
    (4, 2, 64, 0), (32, 32, 96, 2047), (32, 8, 128, 0), (8, 1, 128, 0), (16, 1, 64, 100), (4, 4, 96, 0),
]


@pytest.mark.parametrize("hq,hkv,d,window", DECODE_SHAPES)
@pytest.mark.parametrize("peaky", [False, True])
def test_decode_matches_oracle(hq, hkv, d, window, peaky):
    model = _model(hq, hkv, d, window, max_position=4096)
    wl = _workload(model, 6, 64, f"dec-{hq}-{hkv}-{d}-{window}")
    kp, vp = device_pools(wl)
    positions = np.array([0, 63, 64, 1000, 2047, 4095], np.int32)
    q = _queries(wl, 6, 4.0 if peaky else 1.0)
    h = handle_for(model)
    out = h.attn_decode_paged(q, torch_i32(positions), torch_i32(wl.table), kp, vp)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(6, hq, d), positions, np.arange(6), wl.table,
                          op.read_page, window)
    check_close(to_np_bits(out), ref, f"decode {hq}/{hkv}/{d} w{window}")


def _bf16_ulp(x):
    """Spacing of bf16 values at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    x = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(x)).astype(int) - 7)


@pytest.mark.parametrize("peaky", [False, True])
def test_decode_rows_indirection_and_split_invariance(peaky):
    """The same rows decoded with one chunk per row, two, four and sixteen
    for the longest row (the chunk size follows the call's size, so the rows
    are repeated 32, 16, 8, 2 and 1 times), and under other handles'
    chunkings. The merge is exact in real arithmetic and the decode applies
    each weight with 16 significant bits (a bf16 pair), so every chunking
    must agree with the one-chunk result to float32 rounding, and every
    result must lie within one bf16 ulp (plus 2^-20 for float32
    cancellation) of the fp64 oracle."""
    model = _model(32, 8, 128, 0, max_position=65536)
    wl = _workload(model, 8, 128, "dec-rows")
    kp, vp = device_pools(wl)
    rows = np.array([7, 2, 2, 5], np.int32)
    positions = np.array([8191, 4000, 130, 64], np.int32)
    q = _queries(wl, 4, 4.0 if peaky else 1.0)
    h = handle_for(model)
    results = {}
    for rep in (32, 16, 8, 2, 1):       # 1, 2, 4, 16 and 16 chunks for the 128-page row
        n = 4 * rep
        # the chunk size, from the library's workspace query: n rows x Hq x
        # chunks per row (for the longest row, 1024 pages) x (D + 2) floats
        splits = h.decode_workspace_bytes(n) // (n * 32 * 130 * 4)
        chunks = -(-128 // (1024 // splits))
        out = h.attn_decode_paged(q.repeat(rep, 1), torch_i32(np.tile(positions, rep)), torch_i32(wl.table), kp, vp,
                                  rows=torch_i32(np.tile(rows, rep)))
        o = to_np_bits(out).reshape(rep, 4, -1)
        assert all(np.array_equal(o[0], o[i]) for i in range(rep)), "repeated rows differ within one call"
        results[chunks] = o[0]
    assert sorted(results) == [1, 2, 4, 16], sorted(results)
    for max_pos in (8192, 1 << 20):                  # other handles, other chunkings
        h2 = handle_for(_model(32, 8, 128, 0, max_position=max_pos))
        out = h2.attn_decode_paged(q, torch_i32(positions), torch_i32(wl.table), kp, vp, rows=torch_i32(rows))
        results[f"max_position {max_pos}"] = to_np_bits(out)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(4, 32, 128), positions, rows, wl.table,
                          op.read_page, 0).reshape(4, -1)
    check_close(results[1], ref, "decode rows, one chunk")
    one = bf16.to_f64(results[1])
    for k, bits in results.items():
        o = bf16.to_f64(bits)
        diff = np.abs(o - one)
        assert np.all(diff <= _bf16_ulp(np.maximum(np.abs(o), np.abs(one))) + 2.0 ** -20), \
            f"{k} chunks: max difference {diff.max():.3e} from the one-chunk result"
        err = np.abs(o - ref)
        assert np.all(err <= _bf16_ulp(ref) + 2.0 ** -20), \
            f"{k} chunks: max error {err.max():.3e} from the oracle, beyond one bf16 ulp"


PREFILL_SHAPES = [(4, 2, 64, 0), (32, 32, 96, 2047), (32, 8, 128, 0), (8, 8, 128, 40), (8, 2, 96, 0)]


@pytest.mark.parametrize("hq,hkv,d,window", PREFILL_SHAPES)
@pytest.mark.parametrize("peaky", [False, True])
def test_prefill_packed_matches_oracle(hq, hkv, d, window, peaky):
    model = _model(hq, hkv, d, window, max_position=1024)
    wl = _workload(model, 5, 16, f"pre-{hq}-{hkv}-{d}-{window}")
    kp, vp = device_pools(wl)
    # ragged prompts: a single token, sub-tile, exact tile, multi-tile, and a
    # chunk continuing after a prefix at a page-unaligned position
    spec = [(0, 0, 1), (1, 0, 37), (2, 0, 128), (3, 0, 261), (4, 300, 200)]
    pos = np.concatenate([np.arange(s, s + n) for _, s, n in spec]).astype(np.int32)
    seg = np.concatenate([np.full(n, r) for r, _, n in spec]).astype(np.int32)
    T = len(pos)
    q = _queries(wl, T, 4.0 if peaky else 1.0)
    h = handle_for(model)
    out = h.attn_prefill_packed(q, torch_i32(pos), torch_i32(seg), torch_i32(wl.table), kp, vp,
                                n_segments=len(spec))
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(T, hq, d), pos, seg, wl.table, op.read_page, window)
    check_close(to_np_bits(out), ref, f"prefill {hq}/{hkv}/{d} w{window}")


def test_prefill_unsorted_tokens_and_repeated_segments():
    """Tokens of one prompt need not be contiguous or sorted: each token sees
    its own row up to its own position."""
    model = _model(32, 8, 128, 0, max_position=1024)
    wl = _workload(model, 3, 16, "pre-shuffle")
    kp, vp = device_pools(wl)
    rng = np.random.default_rng(5)
    pos = rng.integers(0, 1024, 300).astype(np.int32)
    seg = np.repeat(rng.integers(0, 3, 30), 10).astype(np.int32)
    q = _queries(wl, 300)
    h = handle_for(model)
    out = h.attn_prefill_packed(q, torch_i32(pos), torch_i32(seg), torch_i32(wl.table), kp, vp,
                                n_segments=30)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(300, 32, 128), pos, seg, wl.table, op.read_page, 0)
    check_close(to_np_bits(out), ref, "prefill shuffled")


@pytest.mark.parametrize("n_seg", [64, 65, 5000])
def test_prefill_many_short_segments(n_seg):
    """One-token prompts, each its own row and tile: 64 tiles (sorted in one
    wave's registers), 65 (sorted in LDS) and 5000 (more than the tile pass
    sorts, dispatched in order). Each token attends its own row up to its
    position, over pre-filled pages."""
    model = _model(4, 2, 64, 0, max_position=256)
    wl = _workload(model, n_seg, 4, f"pre-many-{n_seg}")
    kp, vp = device_pools(wl)
    rng = np.random.default_rng(n_seg)
    pos = rng.integers(0, 256, n_seg).astype(np.int32)
    seg = rng.permutation(n_seg).astype(np.int32)
    q = _queries(wl, n_seg)
    h = handle_for(model)
    out = h.attn_prefill_packed(q, torch_i32(pos), torch_i32(seg), torch_i32(wl.table), kp, vp, n_segments=n_seg)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    op.prefetch(wl.table.ravel())
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(n_seg, 4, 64), pos, seg, wl.table, op.read_page, 0)
    check_close(to_np_bits(out), ref, f"prefill {n_seg} one-token segments")


@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 2), (96, 4, 4), (128, 8, 2)])
@pytest.mark.parametrize("n_pages", [1, 2, 3, 4, 5, 6])
def test_prefill_tile_of_n_pages(d, hq, hkv, n_pages):
    """One tile of 64 tokens at positions 64(n-1) .. 64n-1 attends exactly n
    pages: fewer, as many and more pages than the kernel keeps in flight (its
    LDS ring holds 3 pages at head_dim 96 and 4 otherwise), so the pipeline's
    start, steady state and drain are each exercised."""
    model = _model(hq, hkv, d, 0, max_position=512)
    wl = _workload(model, 1, 6, f"pre-npages-{d}-{n_pages}")
    kp, vp = device_pools(wl)
    pos = np.arange(64 * (n_pages - 1), 64 * n_pages, dtype=np.int32)
    seg = np.zeros(64, np.int32)
    q = _queries(wl, 64)
    h = handle_for(model)
    out = h.attn_prefill_packed(q, torch_i32(pos), torch_i32(seg), torch_i32(wl.table), kp, vp, n_segments=1)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    op.prefetch(wl.table.ravel())
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(64, hq, d), pos, seg, wl.table, op.read_page, 0)
    check_close(to_np_bits(out), ref, f"prefill tile of {n_pages} pages, head_dim {d}")


def test_prefill_out_of_range_page_is_skipped_and_other_segments_are_untouched():
    """Without validate mode a page id past the pool is caught by the kernel:
    that page is neither read nor attended, and the segments whose rows are
    sound match the oracle."""
    model = _model(8, 2, 128, 0, max_position=512)
    wl = _workload(model, 3, 4, "pre-bad-page")
    kp, vp = device_pools(wl)
    bad = wl.table.copy()
    bad[1, 1] = 1 << 30
    pos = np.tile(np.arange(100, 200, dtype=np.int32), 3)
    seg = np.repeat(np.arange(3, dtype=np.int32), 100)
    q = _queries(wl, 300)
    h = handle_for(model)
    out = h.attn_prefill_packed(q, torch_i32(pos), torch_i32(seg), torch_i32(bad), kp, vp, n_segments=3)
    torch.cuda.synchronize()
    op = OraclePool(wl, "cuda")
    op.prefetch(wl.table.ravel())
    good = seg != 1
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(300, 8, 128)[good], pos[good], seg[good], wl.table,
                          op.read_page, 0)
    check_close(to_np_bits(out)[good], ref, "segments beside the bad page id")


def test_step_paged_decode_sees_the_prompt_written_in_the_same_call():
    """step_paged writes every token first: a decode token that continues
    its own row's prompt from the same call (and one that continues a prompt
    row at the prompt's last position + 1 in another page) attends the
    prompt's keys and values as the oracle's write-then-attend does."""
    model = _model(8, 2, 64, 0, max_position=1024)
    wl = _workload(model, 3, 16, "step-same-row")
    kp, vp = device_pools(wl)
    # row 0: prompt at 0..99, decode token at 100; row 1: prompt at 40..127
    # (prefix 0..39 pre-filled), decode token at 128 (a new page); row 2:
    # decode only, at 500
    ppos = np.concatenate([np.arange(0, 100), np.arange(40, 128)]).astype(np.int32)
    pseg = np.concatenate([np.zeros(100), np.ones(88)]).astype(np.int32)
    dpos = np.array([100, 128, 500], np.int32)
    drow = np.array([0, 1, 2], np.int32)
    pos = np.concatenate([ppos, dpos])
    rows = np.concatenate([pseg, drow])
    T, P = len(pos), len(ppos)
    qkv = W.normal_matrix(wl.key("qkv"), T, model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    h = handle_for(model)
    q_out, out = h.step_paged(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                              torch_i32(pos), torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=P, n_segments=2)
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), pos, None)
    op = OraclePool(wl, "cuda")
    op.write(pages.slot_of(wl.table, rows, pos), k_bits, v_bits)
    ref = attention.paged(bf16.to_f64(q_bits), pos, rows, wl.table, op.read_page, 0)
    check_close(to_np_bits(out), ref, "step_paged over one call's own writes")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("explicit_slots", [False, True])
def test_step_paged_decode_only(in_place, explicit_slots):
    """A decode step (no prompt tokens) with QK-norm: the decode writes each
    row's token itself; with q_out over q (in place) every token is written
    first instead. Either way q_out and K match the oracle bit for bit, V is
    a bit copy, and the outputs match the oracle over the written pools."""
    model = _model(8, 2, 128, 0, max_position=2048, theta=1e6, eps=1e-6)
    wl = _workload(model, 6, 32, f"step-dec-{in_place}-{explicit_slots}")
    kp, vp = device_pools(wl)
    pos = np.array([5, 63, 64, 700, 1500, 2047], np.int32)
    rows = np.arange(6, dtype=np.int32)
    T = len(pos)
    qkv = W.normal_matrix(wl.key("qkv"), T, model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    slots = pages.slot_of(wl.table, rows, pos)
    h = handle_for(model)
    qkv_bits = to_np_bits(qkv)                 # before the call: in place, q is overwritten
    q = qkv[:, :hq * D]
    q_out, out = h.step_paged(q, qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:], torch_i32(pos),
                              torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=0, n_segments=1,
                              slots=torch_i32(slots) if explicit_slots else None, q_gain=gains[0], k_gain=gains[1],
                              q_out=q if in_place else None)
    torch.cuda.synchronize()
    g_np = (to_np_bits(gains[0]), to_np_bits(gains[1]))
    _, q_bits, k_bits, v_bits = oracle_front(wl, qkv_bits, pos, g_np)
    check_bits(to_np_bits(q_out).reshape(q_bits.shape), q_bits, "decode-step q_out")
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, "decode-step K pages")
    assert np.array_equal(to_np_bits(vg), v_bits), "decode-step V must be a bit copy"
    op = OraclePool(wl, "cuda")
    op.prefetch(wl.table.ravel())
    op.write(slots, k_bits, v_bits)
    ref = attention.paged(bf16.to_f64(q_bits), pos, rows, wl.table, op.read_page, 0)
    check_close(to_np_bits(out), ref, "decode step over its own writes")


def test_step_paged_validate_refuses_two_step_tokens_in_a_row():
    """A decode-only call writes each row's token inside the decode, so it
    takes one token per row: validate mode refuses two in one row. With
    prompt tokens every token is written first, and a step token may even
    precede its row's prompt tokens."""
    model = _model(8, 2, 64, 0, max_position=1024)
    wl = _workload(model, 3, 16, "step-validate")
    kp, vp = device_pools(wl)
    h = handle_for(model, validate=True)
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads

    def call(pos, rows, n_prompt):
        qkv = W.normal_matrix(wl.key("qkv"), len(pos), model.qkv_width, "cuda")
        return h.step_paged(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                            torch_i32(pos), torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=n_prompt,
                            n_segments=2)

    call(np.array([10, 11], np.int32), np.array([1, 2], np.int32), 0)
    call(np.array([10, 20, 30, 15], np.int32), np.array([0, 0, 0, 0], np.int32), 3)
    with pytest.raises(dap.DapError) as e:
        call(np.array([10, 11], np.int32), np.array([1, 1], np.int32), 0)
    assert e.value.status == dap.BAD_INDEX
    torch.cuda.synchronize()


WRITE_MODELS = [
    _model(4, 2, 64, 0, 4096, theta=1e4),
    _model(32, 32, 96, 2047, 4096, theta=1e4),
    _model(32, 8, 128, 0, 65536, theta=5e5, llama3=(8.0, 1.0, 4.0, 8192.0)),
    _model(32, 8, 128, 0, 40960, theta=1e6, eps=1e-6),
]


@pytest.mark.parametrize("model", WRITE_MODELS, ids=lambda m: m.name)
@pytest.mark.parametrize("explicit_slots", [False, True])
def test_write_matches_oracle_bits(model, explicit_slots):
    n_rows = 4
    ppr = model.max_position // 64
    wl = _workload(model, n_rows, ppr, "wr-" + model.name)
    kp, vp = device_pools(wl)
    k_before, v_before = kp.clone(), vp.clone()
    rng = np.random.default_rng(9)
    T = 300
    rows = rng.integers(0, n_rows, T).astype(np.int32)
    # distinct (row, position) pairs, positions across the whole range
    flat = rng.choice(n_rows * model.max_position, T, replace=False)
    rows, positions = (flat // model.max_position).astype(np.int32), (flat % model.max_position).astype(np.int32)
    qkv = W.normal_matrix(wl.key("qkv"), T, model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    gains = None
    if model.qk_norm_eps:
        gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    slots = pages.slot_of(wl.table, rows, positions)
    h = handle_for(model)
    q_out = h.rope_qknorm_write_pages(
        qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:], torch_i32(positions), kp, vp,
        rows=None if explicit_slots else torch_i32(rows),
        slots=torch_i32(slots) if explicit_slots else None,
        table=None if explicit_slots else torch_i32(wl.table),
        q_gain=gains[0] if gains else None, k_gain=gains[1] if gains else None)
    torch.cuda.synchronize()
    g_np = (to_np_bits(gains[0]), to_np_bits(gains[1])) if gains else None
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), positions, g_np)
    check_bits(to_np_bits(q_out).reshape(T, hq, D), q_bits, "q_out")
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, "K pages")
    assert np.array_equal(to_np_bits(vg), v_bits), "V pages must be a bit copy"
    # nothing else in the pools changed
    s = torch.as_tensor(slots, device="cuda")
    kb, vb = dap.pool_logical(k_before, v_before)
    ka, va = dap.pool_logical(kp, vp)
    kb[s // 64, :, s % 64, :] = ka[s // 64, :, s % 64, :]
    vb[s // 64, :, s % 64, :] = va[s // 64, :, s % 64, :]
    assert torch.equal(kb.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(vb.view(torch.int16), va.view(torch.int16))


@pytest.mark.parametrize("d,n_tokens", [(64, 161), (96, 161), (128, 161), (128, 4100)])
def test_write_runs_of_slots(d, n_tokens):
    """Prompt-shaped writes: a run from an 8-aligned position with a partial
    last group of 8, then a run from a misaligned position, in the same V
    tiles (groups of 8 slots that form one aligned run are stored whole, the
    others element by element); both write forms (per token below 4096
    tokens, per wave from 4096 up). Pools must match the oracle bit for bit
    and nothing else may change."""
    model = _model(16, 4, d, 0, max_position=8192, theta=1e4)
    wl = _workload(model, 2, 128, f"wr-runs-{d}-{n_tokens}")
    kp, vp = device_pools(wl)
    k_before, v_before = kp.clone(), vp.clone()
    n0 = n_tokens - 61
    rows = np.concatenate([np.zeros(n0), np.ones(61)]).astype(np.int32)
    positions = np.concatenate([np.arange(64, 64 + n0), np.arange(37, 98)]).astype(np.int32)
    qkv = W.normal_matrix(wl.key("qkv"), n_tokens, model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    h = handle_for(model)
    q_out = h.rope_qknorm_write_pages(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                                      torch_i32(positions), kp, vp, rows=torch_i32(rows), table=torch_i32(wl.table))
    torch.cuda.synchronize()
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), positions, None)
    check_bits(to_np_bits(q_out).reshape(n_tokens, hq, D), q_bits, "q_out")
    slots = pages.slot_of(wl.table, rows, positions)
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, "K pages")
    assert np.array_equal(to_np_bits(vg), v_bits), "V pages must be a bit copy"
    s = torch.as_tensor(slots, device="cuda")
    kb, vb = dap.pool_logical(k_before, v_before)
    ka, va = dap.pool_logical(kp, vp)
    kb[s // 64, :, s % 64, :] = ka[s // 64, :, s % 64, :]
    vb[s // 64, :, s % 64, :] = va[s // 64, :, s % 64, :]
    assert torch.equal(kb.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(vb.view(torch.int16), va.view(torch.int16))


def test_write_in_place_q():
    model = _model(32, 8, 128, 0, 512, theta=1e6, eps=1e-6)
    wl = _workload(model, 2, 8, "wr-inplace")
    kp, vp = device_pools(wl)
    T = 64
    positions = np.arange(100, 164, dtype=np.int32)
    rows = np.zeros(T, np.int32)
    qkv = W.normal_matrix(wl.key("qkv"), T, model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    gains = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    _, q_bits, _, _ = oracle_front(wl, to_np_bits(qkv), positions, (to_np_bits(gains[0]), to_np_bits(gains[1])))
    h = handle_for(model)
    qv = qkv[:, :hq * D]
    h.rope_qknorm_write_pages(qv, qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:], torch_i32(positions),
                              kp, vp, rows=torch_i32(rows), table=torch_i32(wl.table), q_out=qv,
                              q_gain=gains[0], k_gain=gains[1])
    torch.cuda.synchronize()
    check_bits(to_np_bits(qv).reshape(T, hq, D), q_bits, "in-place q_out")


def test_inv_freq_table_matches_oracle():
    for model in WRITE_MODELS:
        h = handle_for(model)
        from parity import oracle_freqs
        assert np.allclose(h.inv_freq().numpy(), oracle_freqs(model), rtol=1e-15, atol=0)


def test_decode_workspace_reused_across_row_counts():
    """One workspace serves calls with different row counts: each call must
    match a call on a fresh workspace bit for bit."""
    model = _model(32, 32, 96, 2047, max_position=4096)
    wl = _workload(model, 4, 64, "dec-ws-reuse")
    kp, vp = device_pools(wl)
    h = handle_for(model)
    table = torch_i32(wl.table)
    ws = h.workspace(h.decode_workspace_bytes(4))
    q = _queries(wl, 4)
    keep = []
    for n in (4, 1, 2, 4, 3, 1, 4):
        pos = torch_i32(np.array([3000, 2100, 700, 4000][:n], np.int32))
        rows = torch_i32(np.arange(n)[::-1].copy())
        a = h.attn_decode_paged(q[:n], pos, table, kp, vp, rows=rows, workspace=ws)
        b = h.attn_decode_paged(q[:n], pos, table, kp, vp, rows=rows)          # fresh zeroed workspace
        keep.append((a, b, pos, rows))
    torch.cuda.synchronize()
    for a, b, _, _ in keep:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
