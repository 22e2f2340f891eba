"""Stale slots and mask edges on the GPU.

A slot that a query does not attend keeps "what an earlier request left
there" ("Phi-3 Mini 4K Instruct" files, src/attention.linnet: the comment on
prefill_slots, nothing needs clearing because decoding never reads past its
own position; the `seen` mask of decode_rows). The kernels still load whole
pages, so these tests fill every slot outside the attended set J with NaN,
+Inf or -Inf, in both pools (the tail of each row's last page, the slots
before a window's first key in its page, and every other slot of every page
a call touches), and check that each output is finite, bit-identical to the
same call over cleanly filled pools, and equal to the oracle (which reads
only J).

The edge probe sets q = 0, so every key in J has the same weight and the
output is the mean of V over J exactly; it spikes V at both ends of J
(j = max(0, p - W + 1) and j = p) and, with the opposite sign, just outside
them. A key wrongly dropped or wrongly kept moves the output by the spike
over |J|, far beyond the tolerance."""
import zlib

import numpy as np
import pytest
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, pages

from parity import OraclePool, check_close, device_pools, handle_for, to_np_bits, torch_i32

pytestmark = pytest.mark.gpu

POISON = {"nan": 0x7FC0, "inf": 0x7F80, "-inf": 0xFF80}


def _model(hq, hkv, d, window=0, max_position=4096, eps=None):
    return W.ModelShape(f"poison-{hq}-{hkv}-{d}-{window}", hq, hkv, d, 1e4, window=window, qk_norm_eps=eps,
                        max_position=max_position)


def _workload(model, n_rows, ppr, tag):
    rng = np.random.default_rng(zlib.crc32(tag.encode()))
    perm = rng.permutation(n_rows * ppr).astype(np.int32)
    return W.Workload(tag, model, n_rows * ppr, perm.reshape(n_rows, ppr))


def _attended(wl, rows, positions):
    """Pool slots of every key some query attends: J(p) of each (row, position)."""
    win = wl.model.window
    keep = set()
    for r, p in zip(rows, positions):
        lo = max(0, int(p) - win + 1) if win > 0 else 0
        js = np.arange(lo, int(p) + 1)
        keep.update(pages.slot_of(wl.table, np.full(js.size, r), js).tolist())
    return keep


def _pools_with(wl, keep, value):
    """Pools holding the generated pages on the slots in ``keep`` and
    ``value`` (a bf16 bit pattern) on every other slot of every page."""
    m = wl.model
    ids = np.arange(wl.n_pages)
    k = wl.pages("k", ids, "cuda").clone()
    v = wl.pages("v", ids, "cuda").clone()
    mask = torch.ones(wl.n_pages * 64, dtype=torch.bool, device="cuda")
    mask[torch.as_tensor(sorted(keep), dtype=torch.long, device="cuda")] = False
    mask = mask.view(wl.n_pages, 1, 64, 1).expand(-1, m.n_kv_heads, -1, m.head_dim)
    bits = torch.tensor(value, dtype=torch.int32).to(torch.int16).item()
    k[mask] = bits
    v[mask] = bits
    kp, vp = dap.pools(wl.n_pages, m.n_kv_heads, m.head_dim)
    dap.store_pages(kp, vp, ids, k, v)
    return kp, vp


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what + ": differs from the run over clean pools"


DECODE_CASES = [(32, 8, 128, 0), (32, 32, 96, 2047), (4, 2, 64, 100), (16, 1, 64, 0)]


@pytest.mark.parametrize("hq,hkv,d,window", DECODE_CASES)
@pytest.mark.parametrize("poison", list(POISON))
def test_decode_ignores_stale_slots(hq, hkv, d, window, poison):
    model = _model(hq, hkv, d, window)
    wl = _workload(model, 8, 64, f"poison-dec-{hq}-{hkv}-{d}-{window}")
    # page-aligned, page-final and mid-page positions; long rows span several chunks
    positions = np.array([0, 63, 64, 130, 1000, 2047, 3001, 4095], np.int32)
    rows = np.arange(8, dtype=np.int32)
    keep = _attended(wl, rows, positions)
    q = W.normal_matrix(wl.key("q"), 8, hq * d, "cuda")
    h = handle_for(model)
    args = (torch_i32(positions), torch_i32(wl.table))
    kp, vp = _pools_with(wl, keep, POISON[poison])
    out = h.attn_decode_paged(q, *args, kp, vp)
    kc, vc = device_pools(wl)
    clean = h.attn_decode_paged(q, *args, kc, vc)
    torch.cuda.synchronize()
    assert torch.isfinite(out.view(torch.bfloat16).float()).all(), "non-finite decode output"
    _same_bits(out, clean, f"decode {poison}")
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(8, hq, d), positions, rows, wl.table, op.read_page,
                          window)
    check_close(to_np_bits(out), ref, f"decode over {poison} stale slots")


PREFILL_CASES = [(32, 8, 128, 0), (32, 32, 96, 2047), (8, 8, 128, 40), (4, 2, 64, 100), (8, 2, 96, 0)]


@pytest.mark.parametrize("hq,hkv,d,window", PREFILL_CASES)
@pytest.mark.parametrize("poison", ["nan", "inf"])
def test_prefill_ignores_stale_slots(hq, hkv, d, window, poison):
    model = _model(hq, hkv, d, window, max_position=4096)
    wl = _workload(model, 5, 64, f"poison-pre-{hq}-{hkv}-{d}-{window}")
    # prompts from position 0, chunks after unaligned prefixes, one long
    # chunk whose window starts inside a page
    spec = [(0, 0, 1), (1, 0, 37), (2, 5, 128), (3, 300, 261), (4, 2100, 700)]
    pos = np.concatenate([np.arange(s, s + n) for _, s, n in spec]).astype(np.int32)
    seg = np.concatenate([np.full(n, r) for r, _, n in spec]).astype(np.int32)
    T = len(pos)
    keep = _attended(wl, seg, pos)
    q = W.normal_matrix(wl.key("q"), T, hq * d, "cuda")
    h = handle_for(model)
    args = (torch_i32(pos), torch_i32(seg), torch_i32(wl.table))
    kp, vp = _pools_with(wl, keep, POISON[poison])
    out = h.attn_prefill_packed(q, *args, kp, vp, n_segments=len(spec))
    kc, vc = device_pools(wl)
    clean = h.attn_prefill_packed(q, *args, kc, vc, n_segments=len(spec))
    torch.cuda.synchronize()
    assert torch.isfinite(out.view(torch.bfloat16).float()).all(), "non-finite prefill output"
    _same_bits(out, clean, f"prefill {poison}")
    op = OraclePool(wl, "cuda")
    ref = attention.paged(bf16.to_f64(to_np_bits(q)).reshape(T, hq, d), pos, seg, wl.table, op.read_page, window)
    check_close(to_np_bits(out), ref, f"prefill over {poison} stale slots")


@pytest.mark.parametrize("n_prompt_rows", [3, 0])
@pytest.mark.parametrize("window", [0, 300])
def test_step_paged_ignores_stale_slots(n_prompt_rows, window):
    """Prompts (chunks after prefixes) and decode rows in one step_paged call
    over pools whose only clean slots are the keys the call attends; with no
    prompt rows the call takes the decode-step form (the decode writes its
    own tokens)."""
    model = _model(16, 4, 128, window, max_position=2048, eps=1e-6)
    wl = _workload(model, 6, 32, f"poison-step-{n_prompt_rows}-{window}")
    ppos, pseg = [], []
    starts = [0, 70, 500][:n_prompt_rows]
    lens = [100, 129, 300][:n_prompt_rows]
    for r, (s, n) in enumerate(zip(starts, lens)):
        ppos.append(np.arange(s, s + n))
        pseg.append(np.full(n, r))
    dpos = np.array([640, 1999, 77], np.int32)
    drow = np.array([3, 4, 5], np.int32)
    pos = np.concatenate(ppos + [dpos]).astype(np.int32)
    rows = np.concatenate(pseg + [drow]).astype(np.int32)
    P = int(sum(lens))
    keep = _attended(wl, rows, pos)
    qkv = W.normal_matrix(wl.key("qkv"), len(pos), model.qkv_width, "cuda")
    D, hq, hkv = model.head_dim, model.n_q_heads, model.n_kv_heads
    gq, gk = wl.gains("q", "cuda"), wl.gains("k", "cuda")
    h = handle_for(model)
    outs = []
    for kp, vp in (_pools_with(wl, keep, POISON["nan"]), device_pools(wl)):
        _, out = h.step_paged(qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:],
                              torch_i32(pos), torch_i32(rows), torch_i32(wl.table), kp, vp, n_prompt=P,
                              n_segments=max(n_prompt_rows, 1), q_gain=gq, k_gain=gk)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].view(torch.bfloat16).float()).all(), "non-finite step output"
    _same_bits(outs[0], outs[1], "step_paged")


@pytest.mark.parametrize("entry", ["packed", "forward"])
def test_inpass_entries_ignore_workspace_contents(entry):
    """The no-cache entries put each segment's keys on scratch pages inside
    the caller's workspace; the tail of a segment's last page is never
    written. A workspace full of 0xFF bytes (bf16 NaN, int32 -1) must give
    the same bits as a zeroed one."""
    model = _model(32, 8, 128, 0, max_position=4096)
    wl = _workload(model, 1, 1, f"poison-inpass-{entry}")
    h = handle_for(model)
    D, hq, hkv = 128, 32, 8
    if entry == "packed":
        lens = [1, 63, 65, 200, 129]
        pos = np.concatenate([np.arange(n) + (7 if i % 2 else 0) for i, n in enumerate(lens)]).astype(np.int32)
        seg = np.concatenate([np.full(n, i) for i, n in enumerate(lens)]).astype(np.int32)
        T = len(pos)
        nb = h.inpass_workspace_bytes(T, len(lens))
    else:
        T, n_seqs = 3 * 150, 3
        nb = h.inpass_workspace_bytes(T, n_seqs)
    qkv = W.normal_matrix(wl.key("qkv"), T, model.qkv_width, "cuda")
    parts = (qkv[:, :hq * D], qkv[:, hq * D:(hq + hkv) * D], qkv[:, (hq + hkv) * D:])
    outs = []
    for fill in (0xFF, 0x00):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        if entry == "packed":
            outs.append(h.packed(*parts, torch_i32(pos), torch_i32(seg), n_segments=len(lens), workspace=ws))
        else:
            outs.append(h.forward(*parts, n_seqs, workspace=ws))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].view(torch.bfloat16).float()).all(), f"non-finite {entry} output"
    _same_bits(outs[0], outs[1], entry)


SPIKE = 1000.0      # exactly representable in bf16


def _spiked_pools(wl, rows, positions):
    """Generated pools with V = +SPIKE at both ends of each query's J and
    -SPIKE just outside them (where those positions exist in the row)."""
    m = wl.model
    ids = np.arange(wl.n_pages)
    k = wl.pages("k", ids, "cuda").clone()
    v = wl.pages("v", ids, "cuda").clone()
    vf = v.view(torch.bfloat16)
    n_pos = wl.table.shape[1] * 64
    inside, outside = set(), set()
    for r, p in zip(rows, positions):
        lo = max(0, int(p) - m.window + 1) if m.window > 0 else 0
        inside |= {(int(r), lo), (int(r), int(p))}
        outside |= {(int(r), j) for j in (lo - 1, int(p) + 1) if 0 <= j < n_pos}
    outside -= inside
    for val, where in ((SPIKE, inside), (-SPIKE, outside)):
        for r, j in where:
            s = int(pages.slot_of(wl.table, [r], [j])[0])
            vf[s // 64, :, s % 64, :] = val
    kp, vp = dap.pools(wl.n_pages, m.n_kv_heads, m.head_dim)
    dap.store_pages(kp, vp, ids, k, v)
    return kp, vp, k, v


@pytest.mark.parametrize("hq,hkv,d,window", [(32, 8, 128, 0), (32, 32, 96, 2047), (4, 2, 64, 100)])
def test_spikes_at_the_edges_of_j_with_zero_queries(hq, hkv, d, window):
    model = _model(hq, hkv, d, window)
    wl = _workload(model, 6, 64, f"spike-{hq}-{hkv}-{d}-{window}")
    h = handle_for(model)
    # decode rows, then a prompt per row as the prefill's tokens
    positions = np.array([0, 64, 130, 2046, 2047, 4000], np.int32)
    rows = np.arange(6, dtype=np.int32)
    kp, vp, k, v = _spiked_pools(wl, rows, positions)
    q = torch.zeros(6, hq * d, dtype=torch.int16, device="cuda")
    out = h.attn_decode_paged(q, torch_i32(positions), torch_i32(wl.table), kp, vp)
    pre_pos = np.concatenate([np.arange(p - min(p, 40), p + 1) for p in positions]).astype(np.int32)
    pre_seg = np.concatenate([np.full(min(p, 40) + 1, r) for r, p in zip(rows, positions)]).astype(np.int32)
    qp = torch.zeros(len(pre_pos), hq * d, dtype=torch.int16, device="cuda")
    outp = h.attn_prefill_packed(qp, torch_i32(pre_pos), torch_i32(pre_seg), torch_i32(wl.table), kp, vp,
                                 n_segments=6)
    torch.cuda.synchronize()
    kn, vn = to_np_bits(k), to_np_bits(v)
    read = lambda pg: (bf16.to_f64(kn[pg]), bf16.to_f64(vn[pg]))
    ref = attention.paged(np.zeros((6, hq, d)), positions, rows, wl.table, read, window)
    check_close(to_np_bits(out), ref, "decode with edge spikes, q = 0")
    # the last token of each prompt sees exactly the decode's J: same values
    refp = attention.paged(np.zeros((len(pre_pos), hq, d)), pre_pos, pre_seg, wl.table, read, window)
    check_close(to_np_bits(outp), refp, "prefill with edge spikes, q = 0")
    # every spike inside J moves the mean by SPIKE / |J|: the outputs are far from the unspiked mean
    assert np.all(np.abs(ref).max(axis=(1, 2)) > 0.3)
