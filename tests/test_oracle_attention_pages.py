"""Pins for the oracle's page addressing, K/V write and attention.

The equivalences come from the pages (packed = per-prompt, paged =
contiguous, decode continues prefill, window at or above the sequence
length = plain causal); the brute-force reference is torch's
scaled_dot_product_attention in float64 with an explicit boolean mask, and
the special cases (one key, constant V, q = 0) have closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, bf16, core, pages, rope

PAGE = 64


def _reader(k_pool, v_pool, hkv, d):
    def read_page(page):
        k, v = pages.page_logical(k_pool, v_pool, page, hkv, d)
        return bf16.to_f64(k), bf16.to_f64(v)
    return read_page


def _random_pools(rng, n_pages, hkv, d):
    k = bf16.from_f64(rng.standard_normal((n_pages, hkv, PAGE, d)))
    v = bf16.from_f64(rng.standard_normal((n_pages, hkv, PAGE, d)))
    return pages.pools_from_logical(k, v), (k, v)


# ------------------------------------------------------------- addressing

def test_slot_addressing_by_hand():
    table = np.array([[5, 2, -1], [7, 1, 0]], np.int32)
    # row 0, position 70 -> table[0][1] = page 2, index 6 -> slot 2*64 + 6
    # row 1, position 5  -> table[1][0] = page 7, index 5 -> slot 453
    # row 1, position 191 -> table[1][2] = page 0, index 63 -> slot 63
    assert list(pages.slot_of(table, [0, 1, 1], [70, 5, 191])) == [134, 453, 63]


def test_write_places_bits_and_keeps_everything_else():
    rng = np.random.default_rng(10)
    n_pages, hkv, d = 6, 2, 64
    canary = 0x7FC1
    kp, vp = pages.empty_pools(n_pages, hkv, d, fill=canary)
    slots = np.array([0, 63, 64 * 3 + 17, 64 * 5 + 63, 64 * 2], np.int64)
    kb = rng.integers(0, 0x7F00, (len(slots), hkv, d)).astype(np.uint16)
    vb = rng.integers(0, 0x7F00, (len(slots), hkv, d)).astype(np.uint16)
    kp2, vp2 = pages.write(kp, vp, slots, kb, vb)
    # check with 4-D indexing of the documented layouts
    for t, s in enumerate(slots):
        pg, i = divmod(int(s), PAGE)
        assert np.array_equal(kp2[pg, :, i, :], kb[t])
        assert np.array_equal(vp2[pg, :, :, i], vb[t])
    assert np.count_nonzero(kp2 != canary) <= kb.size
    assert np.count_nonzero(kp2 != kp) == np.count_nonzero(kb != canary)
    assert np.count_nonzero(vp2 != vp) == np.count_nonzero(vb != canary)


def test_pool_layout_round_trip():
    rng = np.random.default_rng(11)
    (kp, vp), (kl, vl) = _random_pools(rng, 4, 3, 96)
    for pg in range(4):
        k, v = pages.page_logical(kp, vp, pg, 3, 96)
        assert np.array_equal(k, kl[pg]) and np.array_equal(v, vl[pg])


# ------------------------------------------------------- attention: brute force

def _sdpa(q, K, V, mask):
    """torch fp64 SDPA: q [Hq, nq, D], K/V [Hq, n, D], mask [nq, n] bool."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=torch.from_numpy(mask)).numpy()


@pytest.mark.parametrize("hq,hkv,d,window", [(4, 2, 64, 0), (4, 1, 96, 5), (2, 2, 128, 3)])
def test_paged_matches_torch_sdpa_brute_force(hq, hkv, d, window):
    rng = np.random.default_rng(12)
    n_pages = 3
    (kp, vp), (kl, vl) = _random_pools(rng, n_pages, hkv, d)
    table = np.array([[2, 0, 1]], np.int32)
    T = 150
    positions = np.arange(T)
    q = rng.standard_normal((T, hq, d))
    out = attention.paged(q, positions, np.zeros(T, np.int64), table,
                          _reader(kp, vp, hkv, d), window)
    # dense logical sequence of the row
    K = np.concatenate([bf16.to_f64(kl[p]) for p in table[0]], axis=1)[:, :T]
    V = np.concatenate([bf16.to_f64(vl[p]) for p in table[0]], axis=1)[:, :T]
    g = hq // hkv
    Kq = np.repeat(K, g, axis=0)
    Vq = np.repeat(V, g, axis=0)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = j <= i
    if window:
        mask &= j > i - window
    ref = _sdpa(np.swapaxes(q, 0, 1).copy(), Kq, Vq, mask)
    assert np.allclose(out, np.swapaxes(ref, 0, 1), rtol=1e-12, atol=1e-12)


def test_one_key_constant_v_and_zero_query():
    rng = np.random.default_rng(13)
    hkv, d = 2, 64
    (kp, vp), (kl, vl) = _random_pools(rng, 2, hkv, d)
    table = np.array([[1, 0]], np.int32)
    rd = _reader(kp, vp, hkv, d)
    q = rng.standard_normal((1, 4, d)) * 5
    # position 0: exactly one key -> output is V_0
    out = attention.paged(q, [0], [0], table, rd)
    v0 = bf16.to_f64(vl[1][:, 0])                      # [Hkv, D]
    assert np.array_equal(out[0], np.repeat(v0, 2, axis=0))
    # q = 0 -> uniform weights -> mean of V over the attended positions
    p, W = 100, 40
    out = attention.paged(np.zeros((1, 4, d)), [p], [0], table, rd, window=W)
    V = np.concatenate([bf16.to_f64(vl[1]), bf16.to_f64(vl[0])], axis=1)
    mean = V[:, p - W + 1: p + 1].mean(axis=1)
    assert np.allclose(out[0], np.repeat(mean, 2, axis=0), rtol=1e-13, atol=1e-15)
    # constant V -> output equals that constant
    vc = np.full_like(vl, bf16.from_f64(np.array([0.375]))[0])
    kp2, vp2 = pages.pools_from_logical(kl, vc)
    out = attention.paged(q, [77], [0], table, _reader(kp2, vp2, hkv, d))
    assert np.allclose(out, 0.375, rtol=1e-14)


def test_mask_edges_by_spike_and_nan_poison():
    rng = np.random.default_rng(14)
    hkv, d = 1, 64
    (kp, vp), (kl, vl) = _random_pools(rng, 4, hkv, d)
    table = np.array([[3, 1, 0, 2]], np.int32)
    p, W = 150, 70
    lo = p - W + 1
    # NaN-poison every position outside [lo, p], including the stale tail of
    # the last page; the output must stay finite and unchanged
    nan = 0x7FC0
    kl2, vl2 = kl.copy(), vl.copy()
    for j in list(range(0, lo)) + list(range(p + 1, 4 * PAGE)):
        pg = table[0][j // PAGE]
        kl2[pg, :, j % PAGE] = nan
        vl2[pg, :, j % PAGE] = nan
    q = rng.standard_normal((1, 2, d))
    clean = attention.paged(q, [p], [0], table, _reader(kp, vp, hkv, d), W)
    poisoned = attention.paged(q, [p], [0], table, _reader(*pages.pools_from_logical(kl2, vl2), hkv, d), W)
    assert np.all(np.isfinite(poisoned)) and np.array_equal(clean, poisoned)
    # spikes at both ends of the window with q = 0: each contributes spike/|J|
    for j in (lo, p):
        vl3 = vl.copy()
        vl3[table[0][j // PAGE], :, j % PAGE] = bf16.from_f64(np.array([1024.0]))[0]
        base = attention.paged(np.zeros((1, 2, d)), [p], [0], table, _reader(kp, vp, hkv, d), W)
        spiked = attention.paged(np.zeros((1, 2, d)), [p], [0], table,
                                 _reader(*pages.pools_from_logical(kl, vl3), hkv, d), W)
        v_old = bf16.to_f64(vl[table[0][j // PAGE], 0, j % PAGE])
        assert np.allclose(spiked - base, (1024.0 - v_old) / W, rtol=1e-10)


# ------------------------------------------------------- the pages' equivalences

def test_window_at_or_above_length_is_plain_causal():
    rng = np.random.default_rng(15)
    (kp, vp), _ = _random_pools(rng, 3, 2, 96)
    table = np.array([[0, 2, 1]], np.int32)
    T = 180
    q = rng.standard_normal((T, 4, 96))
    rd = _reader(kp, vp, 2, 96)
    causal = attention.paged(q, np.arange(T), np.zeros(T, int), table, rd, 0)
    for W in (T, T + 1, 2047):
        assert np.array_equal(attention.paged(q, np.arange(T), np.zeros(T, int), table, rd, W), causal)
    assert not np.allclose(attention.paged(q, np.arange(T), np.zeros(T, int), table, rd, T - 1), causal)


def test_paged_equals_identity_table_equals_contiguous():
    rng = np.random.default_rng(16)
    hkv, d, n = 2, 64, 3
    kl = bf16.from_f64(rng.standard_normal((n, hkv, PAGE, d)))
    vl = bf16.from_f64(rng.standard_normal((n, hkv, PAGE, d)))
    perm = np.array([2, 0, 1])
    # the same logical row stored in permuted physical pages
    kp_id, vp_id = pages.pools_from_logical(kl, vl)
    kl_perm, vl_perm = np.empty_like(kl), np.empty_like(vl)
    kl_perm[perm], vl_perm[perm] = kl, vl
    kp_pm, vp_pm = pages.pools_from_logical(kl_perm, vl_perm)
    T = 192
    q = rng.standard_normal((T, 4, d))
    pos = np.arange(T)
    rows = np.zeros(T, int)
    a = attention.paged(q, pos, rows, np.array([[0, 1, 2]]), _reader(kp_id, vp_id, hkv, d))
    b = attention.paged(q, pos, rows, perm[None, :], _reader(kp_pm, vp_pm, hkv, d))
    cache_k = np.concatenate(list(bf16.to_f64(kl)), axis=1)[None]     # [1, Hkv, 192, D]
    cache_v = np.concatenate(list(bf16.to_f64(vl)), axis=1)[None]
    c = attention.contiguous(q, pos, rows, cache_k, cache_v)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def _tiny_pass(rng, prompts, hq=4, hkv=2, d=64, window=0, gains=False):
    """Packed prompts from position 0 through the full front half + write."""
    P = sum(prompts)
    pos = np.concatenate([np.arange(L) for L in prompts])
    seg = np.concatenate([np.full(L, r) for r, L in enumerate(prompts)])
    n_pg = [-(-L // PAGE) for L in prompts]
    table = np.full((len(prompts), max(n_pg)), -1, np.int32)
    nxt = 0
    order = rng.permutation(sum(n_pg))
    for r, k in enumerate(n_pg):
        table[r, :k] = order[nxt:nxt + k]
        nxt += k
    kp, vp = pages.empty_pools(sum(n_pg), hkv, d, fill=0x7FC0)   # NaN where never written
    qkv = bf16.from_f64(rng.standard_normal((P, (hq + 2 * hkv) * d)))
    f = rope.inv_freq(1e4, d)
    g = (bf16.from_f64(rng.uniform(0.5, 1.5, d)), bf16.from_f64(rng.uniform(0.5, 1.5, d))) if gains else (None, None)
    q, k, vb = core.prepare_tokens(qkv, pos, hq, hkv, d, f, g[0], g[1], 1e-6 if gains else None)
    kp, vp = core.write_tokens(kp, vp, table, seg, pos, None, k, vb)
    return dict(q=q, k=k, vb=vb, pos=pos, seg=seg, table=table, kp=kp, vp=vp, hkv=hkv, d=d)


def test_packed_inpass_equals_paged_equals_per_prompt():
    rng = np.random.default_rng(17)
    c = _tiny_pass(rng, [70, 128, 33], gains=True)
    rd = _reader(c["kp"], c["vp"], c["hkv"], c["d"])
    paged = attention.paged(c["q"], c["pos"], c["seg"], c["table"], rd, window=50)
    # the pages' own-mask definition over the pass's own (rounded) k and v
    k_r = bf16.round_f64(c["k"])
    v_r = bf16.to_f64(c["vb"])
    inpass = attention.packed_inpass(c["q"], k_r, v_r, c["pos"], c["seg"], window=50)
    assert np.allclose(paged, inpass, rtol=1e-12, atol=1e-13)
    # each prompt alone
    start = 0
    for r, L in enumerate([70, 128, 33]):
        sl = slice(start, start + L)
        alone = attention.packed_inpass(c["q"][sl], k_r[sl], v_r[sl], c["pos"][sl],
                                        np.zeros(L, int), window=50)
        assert np.allclose(paged[sl], alone, rtol=1e-12, atol=1e-13)
        start += L


def test_decode_at_pos_equals_last_row_of_prefill():
    rng = np.random.default_rng(18)
    c = _tiny_pass(rng, [130])
    rd = _reader(c["kp"], c["vp"], c["hkv"], c["d"])
    full = attention.paged(c["q"], c["pos"], c["seg"], c["table"], rd)
    for p in (0, 63, 64, 129):
        dec = attention.paged(c["q"][p:p + 1], [p], [0], c["table"], rd)
        assert np.array_equal(dec[0], full[p])
        # prefill of p + 1 tokens: its last row
        pre = attention.paged(c["q"][:p + 1], c["pos"][:p + 1], c["seg"][:p + 1], c["table"], rd)
        assert np.array_equal(pre[-1], dec[0])


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(19)
    hkv, d, g = 2, 64, 4
    kl = bf16.from_f64(rng.standard_normal((2, hkv, PAGE, d)))
    vl = bf16.from_f64(rng.standard_normal((2, hkv, PAGE, d)))
    table = np.array([[1, 0]])
    q = rng.standard_normal((40, hkv * g, d))
    pos = rng.integers(0, 128, 40)
    rows = np.zeros(40, int)
    gqa = attention.paged(q, pos, rows, table, _reader(*pages.pools_from_logical(kl, vl), hkv, d))
    kr, vr = np.repeat(kl, g, axis=1), np.repeat(vl, g, axis=1)
    mha = attention.paged(q, pos, rows, table, _reader(*pages.pools_from_logical(kr, vr), hkv * g, d))
    assert np.allclose(gqa, mha, rtol=1e-13, atol=1e-15)


def test_front_half_v_is_a_bit_copy_and_q_k_follow_norm_then_rope():
    rng = np.random.default_rng(20)
    hq, hkv, d, T = 4, 2, 64, 9
    qkv = bf16.from_f64(rng.standard_normal((T, (hq + 2 * hkv) * d)))
    pos = rng.integers(0, 40000, T)
    f = rope.inv_freq(1e6, d)
    q, k, vb = core.prepare_tokens(qkv, pos, hq, hkv, d, f)
    assert np.array_equal(vb, qkv[:, (hq + hkv) * d:].reshape(T, hkv, d))
    # without a norm, rope at position 0 returns the input exactly
    q0, k0, _ = core.prepare_tokens(qkv, np.zeros(T, int), hq, hkv, d, f)
    assert np.array_equal(q0.reshape(T, -1), bf16.to_f64(qkv[:, :hq * d]))
    assert np.array_equal(k0.reshape(T, -1), bf16.to_f64(qkv[:, hq * d:(hq + hkv) * d]))
    # head h owns columns h*D .. h*D + D - 1 of its slice
    qkv2 = qkv.copy()
    qkv2[:, 2 * d: 3 * d] = bf16.from_f64(np.zeros((T, d)))      # zero q head 2
    q2, _, _ = core.prepare_tokens(qkv2, pos, hq, hkv, d, f)
    assert np.all(q2[:, 2] == 0) and np.array_equal(q2[:, [0, 1, 3]], q[:, [0, 1, 3]])


def test_front_half_norm_then_rope_against_torch_and_transformers():
    """prepare_tokens with distinct non-uniform q/k gains at positions > 0,
    against an independent composition: torch's rms_norm on each head slice
    ("Qwen3-4B", QK-norm paragraph: each head's slice, before rope), then
    transformers' apply_rotary_pos_emb with cos/sin built from theta^(-2i/D).
    Rope-before-norm and swapped gains are shown to disagree, so the check
    can tell the compositions apart."""
    import torch
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb

    rng = np.random.default_rng(21)
    hq, hkv, d, T, theta, eps = 8, 2, 128, 11, 1e6, 1e-6
    qkv = bf16.from_f64(rng.standard_normal((T, (hq + 2 * hkv) * d)) * rng.uniform(0.1, 3.0, (T, 1)))
    pos = rng.integers(1, 40000, T)
    qg = bf16.from_f64(rng.uniform(0.5, 1.5, d))
    kg = bf16.from_f64(rng.uniform(0.5, 1.5, d))
    f = rope.inv_freq(theta, d)
    q, k, _ = core.prepare_tokens(qkv, pos, hq, hkv, d, f, qg, kg, eps)

    x = torch.from_numpy(bf16.to_f64(qkv))
    tq = x[:, :hq * d].reshape(T, hq, d)
    tk = x[:, hq * d:(hq + hkv) * d].reshape(T, hkv, d)
    gq = torch.from_numpy(bf16.to_f64(qg))
    gk = torch.from_numpy(bf16.to_f64(kg))
    inv = 1.0 / theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
    emb = torch.cat([ang, ang], dim=-1)                      # [T, D]
    cos, sin = emb.cos(), emb.sin()

    def compose(a, b, ga, gb, norm_first=True):
        # transformers' layout: [batch, heads, seq, D] with cos/sin [batch, seq, D]
        a4, b4 = a.permute(1, 0, 2)[None], b.permute(1, 0, 2)[None]
        nrm = lambda t, g: torch.nn.functional.rms_norm(t, (d,), weight=g, eps=eps)
        if norm_first:
            a4, b4 = nrm(a4, ga), nrm(b4, gb)
        ra, rb = apply_rotary_pos_emb(a4, b4, cos[None], sin[None])
        if not norm_first:
            ra, rb = nrm(ra, ga), nrm(rb, gb)
        return ra[0].permute(1, 0, 2).numpy(), rb[0].permute(1, 0, 2).numpy()

    ref_q, ref_k = compose(tq, tk, gq, gk)
    # the two frequency formulas may differ in their last bit, which the
    # angle (position up to 40000) scales to ~1e-11
    assert np.allclose(q, ref_q, rtol=1e-9, atol=1e-9)
    assert np.allclose(k, ref_k, rtol=1e-9, atol=1e-9)
    # the plausible mistakes give clearly different values
    wrong_order = compose(tq, tk, gq, gk, norm_first=False)
    swapped = compose(tq, tk, gk, gq)
    for wq, wk in (wrong_order, swapped):
        assert np.max(np.abs(wq - q)) > 1e-2 and np.max(np.abs(wk - k)) > 1e-2


@pytest.mark.parametrize("hq,hkv,d,window", [(4, 2, 64, 0), (8, 8, 96, 37), (32, 8, 128, 300), (16, 1, 64, 1)])
def test_attend_many_matches_torch_sdpa_with_explicit_masks(hq, hkv, d, window):
    """attend_many (a block of one row's queries in one masked product)
    against torch's fp64 scaled_dot_product_attention given each query's
    boolean mask over the row's keys, at unsorted, repeated and page-crossing
    positions."""
    import torch

    rng = np.random.default_rng(hq * 1000 + d + window)
    L = 700
    K = rng.standard_normal((hkv, L, d))
    V = rng.standard_normal((hkv, L, d))
    pos = np.concatenate([rng.integers(0, L, 20), [0, 1, 63, 64, L - 1, L - 1]])
    q = rng.standard_normal((len(pos), hq, d)) * 2.0
    ours = attention.attend_many(q, K, V, pos, window)
    g = hq // hkv
    j = np.arange(L)
    lo = np.maximum(0, pos - window + 1) if window > 0 else np.zeros_like(pos)
    mask = torch.from_numpy((j[None, :] >= lo[:, None]) & (j[None, :] <= pos[:, None]))     # [n, L]
    kt = torch.from_numpy(np.repeat(K, g, axis=0))                                           # [Hq, L, D]
    vt = torch.from_numpy(np.repeat(V, g, axis=0))
    qt = torch.from_numpy(q).transpose(0, 1)                                                 # [Hq, n, D]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None])
    assert np.allclose(ours, ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-13)
    # and it agrees with the one-query form on every query
    one = np.stack([attention.attend_one(q[i], K, V, int(pos[i]), window) for i in range(len(pos))])
    assert np.allclose(ours, one, rtol=1e-12, atol=1e-13)
