"""The contiguous-cache entries (decode, decode_rows, prefill, prefill_slots)
and the in-pass entries (packed, forward) through the C ABI, against the
oracle: the pages' dense-cache and no-cache entries, realised over an
identity page table and over scratch pages."""
import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, pages

from parity import (OraclePool, check_bits, check_close, device_pools, handle_for, oracle_attention, oracle_front,
                    to_np_bits, torch_i32)

pytestmark = pytest.mark.gpu

MODELS = {
    "gqa2-d64": W.ModelShape("ent-gqa2", 4, 2, 64, 1e4, max_position=1024),
    "mha-d96-window": W.ModelShape("ent-win", 4, 4, 96, 1e4, window=100, max_position=1024),
    "gqa4-d128-qknorm": W.ModelShape("ent-qkn", 8, 2, 128, 1e6, qk_norm_eps=1e-6, max_position=1024),
}


def _cache(model, rows, max_seq, tag):
    """A contiguous cache of `rows` rows: pools with the identity table."""
    ppr = max_seq // 64
    table = np.arange(rows * ppr, dtype=np.int32).reshape(rows, ppr)
    wl = W.Workload(tag, model, rows * ppr, table)
    kp, vp = device_pools(wl)
    return wl, kp, vp


def _split(qkv, m):
    D, hq, hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    return qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:]


def _gains(wl):
    if not wl.model.qk_norm_eps:
        return None, None, None
    g = (wl.gains("q", "cuda"), wl.gains("k", "cuda"))
    return g[0], g[1], (to_np_bits(g[0]), to_np_bits(g[1]))


def _check_cache_call(wl, kp, vp, qkv, out, positions, rows, g_np, what):
    """Oracle: write every token into the generated pools, then paged
    attention over the identity table; also the written slots' bits."""
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), positions, g_np)
    slots = pages.slot_of(wl.table, rows, positions)
    op = OraclePool(wl)
    op.write(slots, k_bits, v_bits)
    ref = oracle_attention(wl, op, bf16.to_f64(q_bits), positions, rows)
    check_close(to_np_bits(out), ref, what)
    kg, vg = dap.gather_slots(kp, vp, slots)
    check_bits(to_np_bits(kg), k_bits, what + " K pages")
    assert np.array_equal(to_np_bits(vg), v_bits), what + ": V pages must be a bit copy"


@pytest.mark.parametrize("name", list(MODELS))
def test_decode_rows_and_decode(name):
    m = MODELS[name]
    R, MS = 3, 1024
    wl, kp, vp = _cache(m, R, MS, "dr-" + name)
    h = handle_for(m)
    qg, kg, g_np = _gains(wl)
    pos = np.array([5, 700, 1023], np.int32)
    qkv = wl.qkv("dr", R, "cuda")
    out = h.decode_rows(*_split(qkv, m), torch_i32(pos), kp, vp, max_seq=MS, q_gain=qg, k_gain=kg)
    torch.cuda.synchronize()
    _check_cache_call(wl, kp, vp, qkv, out, pos, np.arange(R), g_np, f"decode_rows {name}")
    # decode: every row at one position, on a fresh cache
    wl2, kp2, vp2 = _cache(m, R, MS, "d-" + name)
    qkv2 = wl2.qkv("d", R, "cuda")
    out2 = h.decode(*_split(qkv2, m), 640, kp2, vp2, max_seq=MS, q_gain=qg, k_gain=kg)
    torch.cuda.synchronize()
    _check_cache_call(wl2, kp2, vp2, qkv2, out2, np.full(R, 640, np.int32), np.arange(R), g_np, f"decode {name}")


@pytest.mark.parametrize("name", list(MODELS))
def test_prefill_span_over_an_earlier_prefix(name):
    m = MODELS[name]
    R, MS, S, pos = 2, 1024, 150, 300
    wl, kp, vp = _cache(m, R, MS, "pf-" + name)
    h = handle_for(m)
    qg, kg, g_np = _gains(wl)
    qkv = wl.qkv("pf", R * S, "cuda")
    out = h.prefill(*_split(qkv, m), pos, kp, vp, cache_rows=R, max_seq=MS, q_gain=qg, k_gain=kg)
    torch.cuda.synchronize()
    positions = np.tile(np.arange(pos, pos + S, dtype=np.int32), R)
    rows = np.repeat(np.arange(R, dtype=np.int32), S)
    _check_cache_call(wl, kp, vp, qkv, out, positions, rows, g_np, f"prefill {name}")


@pytest.mark.parametrize("name", list(MODELS))
def test_prefill_slots_sees_only_the_prompt(name):
    m = MODELS[name]
    R, MS, S = 3, 1024, 130
    slots = np.array([2, 0], np.int32)
    wl, kp, vp = _cache(m, R, MS, "ps-" + name)
    h = handle_for(m)
    qg, kg, g_np = _gains(wl)
    qkv = wl.qkv("ps", len(slots) * S, "cuda")
    out = h.prefill_slots(*_split(qkv, m), torch_i32(slots), kp, vp, cache_rows=R, max_seq=MS, q_gain=qg,
                          k_gain=kg)
    torch.cuda.synchronize()
    positions = np.tile(np.arange(S, dtype=np.int32), len(slots))
    rows = np.repeat(slots, S)
    _check_cache_call(wl, kp, vp, qkv, out, positions, rows, g_np, f"prefill_slots {name}")
    # the same outputs from the no-cache definition: attention among the prompt's own tokens
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), positions, g_np)
    ref = attention.packed_inpass(bf16.to_f64(q_bits), bf16.to_f64(k_bits), bf16.to_f64(v_bits), positions, rows,
                                  m.window)
    check_close(to_np_bits(out), ref, f"prefill_slots {name} vs in-pass")


def _inpass_ref(wl, qkv, positions, segments, g_np):
    _, q_bits, k_bits, v_bits = oracle_front(wl, to_np_bits(qkv), positions, g_np)
    return attention.packed_inpass(bf16.to_f64(q_bits), bf16.to_f64(k_bits), bf16.to_f64(v_bits), positions,
                                   segments, wl.model.window)


@pytest.mark.parametrize("name", list(MODELS))
def test_packed_segments_at_their_own_positions(name):
    m = MODELS[name]
    wl = W.Workload("pk-" + name, m, 1, np.zeros((1, 1), np.int32))
    h = handle_for(m, validate=True)
    qg, kg, g_np = _gains(wl)
    # three prompts packed end to end, starting mid-page, at 0, and far out
    spans = [(100, 230), (0, 64), (900, 1000)]
    positions = np.concatenate([np.arange(a, b, dtype=np.int32) for a, b in spans])
    segments = np.concatenate([np.full(b - a, s, np.int32) for s, (a, b) in enumerate(spans)])
    qkv = wl.qkv("pk", len(positions), "cuda")
    out = h.packed(*_split(qkv, m), torch_i32(positions), torch_i32(segments), n_segments=3, q_gain=qg, k_gain=kg)
    torch.cuda.synchronize()
    check_close(to_np_bits(out), _inpass_ref(wl, qkv, positions, segments, g_np), f"packed {name}")


def test_packed_many_segments_across_workgroups():
    """300 segments of 1-40 tokens at scattered starting positions: segment
    bounds gathered by several preparation workgroups, most waves spanning
    more than one segment, segments straddling wave and workgroup edges."""
    m = MODELS["gqa2-d64"]
    wl = W.Workload("pk-many", m, 1, np.zeros((1, 1), np.int32))
    h = handle_for(m, validate=True)
    rng = np.random.default_rng(20250)
    lens = rng.integers(1, 41, size=300)
    starts = rng.integers(0, 1024 - 40, size=300)
    positions = np.concatenate([np.arange(a, a + n, dtype=np.int32) for a, n in zip(starts, lens)])
    segments = np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(lens)])
    assert len(positions) > 4 * 1024          # more than four preparation workgroups of tokens
    qkv = wl.qkv("many", len(positions), "cuda")
    out = h.packed(*_split(qkv, m), torch_i32(positions), torch_i32(segments), n_segments=300)
    torch.cuda.synchronize()
    check_close(to_np_bits(out), _inpass_ref(wl, qkv, positions, segments, None), "packed, 300 segments")


@pytest.mark.parametrize("seed", range(6))
def test_random_packed_matches_oracle(seed):
    """Seeded random in-pass calls: head_dim 64/96/128, 1-8 kv heads, 1, 2 or
    4 query heads per kv head, a window or none, QK-norm or none, llama3
    rope or not; 1-20 segments of 1-200 tokens packed in a shuffled id order
    at scattered first positions, three segment ids left empty."""
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 96, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    window = int(rng.choice([0, 0, 1, 37, 200]))
    llama3 = (8.0, 1.0, 4.0, 8192.0) if rng.random() < 0.3 else None
    eps = 1e-6 if rng.random() < 0.4 else None
    theta = float(rng.choice([1e4, 5e5, 1e6]))
    m = W.ModelShape(f"pk-rand-{seed}", hkv * g, hkv, D, theta, window=window, llama3=llama3, qk_norm_eps=eps,
                     max_position=2048)
    wl = W.Workload(m.name, m, 1, np.zeros((1, 1), np.int32))
    n_seg = int(rng.integers(1, 21))
    ids = rng.permutation(n_seg + 3)[:n_seg]            # three ids stay empty
    lens = rng.integers(1, 201, size=n_seg)
    starts = rng.integers(0, 2048 - 200, size=n_seg)
    positions = np.concatenate([np.arange(a, a + n, dtype=np.int32) for a, n in zip(starts, lens)])
    segments = np.concatenate([np.full(n, sid, np.int32) for sid, n in zip(ids, lens)])
    h = handle_for(m, validate=True)
    qg, kg, g_np = _gains(wl)
    qkv = wl.qkv("rand", len(positions), "cuda")
    out = h.packed(*_split(qkv, m), torch_i32(positions), torch_i32(segments), n_segments=n_seg + 3, q_gain=qg,
                   k_gain=kg)
    torch.cuda.synchronize()
    check_close(to_np_bits(out), _inpass_ref(wl, qkv, positions, segments, g_np),
                f"packed seed {seed} ({hkv * g}/{hkv}/{D} w{window} norm {eps} llama3 {llama3 is not None}, "
                f"{n_seg} segments)")


def test_packed_equals_prompts_alone_and_reuses_its_workspace():
    m = MODELS["gqa4-d128-qknorm"]
    wl = W.Workload("pk-alone", m, 1, np.zeros((1, 1), np.int32))
    h = handle_for(m)
    qg, kg, g_np = _gains(wl)
    lens = [70, 200, 33]
    positions = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    segments = np.concatenate([np.full(n, s, np.int32) for s, n in enumerate(lens)])
    qkv = wl.qkv("alone", len(positions), "cuda")
    ws = h.workspace(h.inpass_workspace_bytes(len(positions), 3))
    both = h.packed(*_split(qkv, m), torch_i32(positions), torch_i32(segments), n_segments=3, q_gain=qg, k_gain=kg,
                    workspace=ws)
    start = 0
    for n in lens:          # each prompt alone, through the same workspace
        sub = qkv[start:start + n]
        alone = h.packed(*_split(sub, m), torch_i32(np.arange(n)), torch_i32(np.zeros(n)), n_segments=1, q_gain=qg,
                         k_gain=kg, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(alone, both[start:start + n]), "packing changed a prompt's outputs"
        start += n


@pytest.mark.parametrize("name", list(MODELS))
def test_forward_whole_sequences(name):
    m = MODELS[name]
    wl = W.Workload("fw-" + name, m, 1, np.zeros((1, 1), np.int32))
    h = handle_for(m)
    qg, kg, g_np = _gains(wl)
    B, S = 2, 150
    qkv = wl.qkv("fw", B * S, "cuda")
    out = h.forward(*_split(qkv, m), B, q_gain=qg, k_gain=kg)
    torch.cuda.synchronize()
    positions = np.tile(np.arange(S, dtype=np.int32), B)
    segments = np.repeat(np.arange(B, dtype=np.int32), S)
    check_close(to_np_bits(out), _inpass_ref(wl, qkv, positions, segments, g_np), f"forward {name}")


def test_entry_argument_and_validate_errors():
    m = MODELS["gqa2-d64"]
    R, MS = 2, 256
    wl, kp, vp = _cache(m, R, MS, "ent-err")
    h = handle_for(m, validate=True)
    qkv = wl.qkv("err", 2 * 10, "cuda")
    with pytest.raises(dap.DapError) as e:                    # position past max_seq
        h.decode(*_split(qkv[:R], m), MS, kp, vp, max_seq=MS)
    assert e.value.status == dap.INVALID_ARG
    with pytest.raises(dap.DapError) as e:                    # max_seq not a multiple of 64
        h.decode(*_split(qkv[:R], m), 3, kp, vp, max_seq=100)
    assert e.value.status == dap.INVALID_ARG
    with pytest.raises(dap.DapError) as e:                    # two prompts into one cache row
        h.prefill_slots(*_split(qkv, m), torch_i32([1, 1]), kp, vp, cache_rows=R, max_seq=MS)
    assert e.value.status == dap.BAD_INDEX
    with pytest.raises(dap.DapError) as e:                    # a gap in a segment's positions
        pos = np.concatenate([np.arange(5), np.arange(6, 11)]).astype(np.int32)
        h.packed(*_split(qkv[:10], m), torch_i32(pos), torch_i32(np.zeros(10)), n_segments=1)
    assert e.value.status == dap.BAD_INDEX
    with pytest.raises(dap.DapError) as e:                    # a segment split over two runs
        seg = np.array([0] * 5 + [1] * 5 + [0] * 5 + [1] * 5, np.int32)
        pos = np.concatenate([np.arange(5), np.arange(5), np.arange(5, 10), np.arange(5, 10)]).astype(np.int32)
        h.packed(*_split(qkv, m), torch_i32(pos), torch_i32(seg), n_segments=2)
    assert e.value.status == dap.BAD_INDEX
    with pytest.raises(dap.DapError) as e:                    # more than 4096 segments
        h.packed(*_split(qkv[:10], m), torch_i32(np.arange(10)), torch_i32(np.zeros(10)), n_segments=5000)
    assert e.value.status == dap.UNSUPPORTED
    torch.cuda.synchronize()
