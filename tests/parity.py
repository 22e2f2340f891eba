"""Helpers shared by the GPU parity tests: device pools filled from the seeded
generators, an oracle-side view of the same pools (generated pages plus the
oracle's own writes), and the comparison gates.

Nothing here reads a value the HIP path produced into an oracle input: the
oracle side regenerates pages from the generator (which gives identical bits
on CPU and GPU) and overlays the K/V values the oracle itself computed."""
from __future__ import annotations

import math

import numpy as np
import torch

import decoder_attention_paged_amd as dap
import workloads as W
from oracle import attention, bf16, core, pages, rope

ATOL = 2e-2
RTOL = 2e-2
REL_RMS = 1e-2
TIE_TOL = 1e-12
TIE_REPORT = []        # (what, elements, flagged near-ties, differing) per check_bits call


def handle_for(model: W.ModelShape, validate=False) -> dap.Handle:
    return dap.Handle(dap.Model(model.n_q_heads, model.n_kv_heads, model.head_dim, model.rope_theta,
                                window=model.window, max_position=model.max_position,
                                llama3=model.llama3, qk_norm_eps=model.qk_norm_eps), validate=validate)


def oracle_freqs(model: W.ModelShape):
    return rope.inv_freq(model.rope_theta, model.head_dim, model.llama3)


def to_np_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def device_pools(wl: W.Workload, device="cuda", chunk=2048):
    """K/V pools of the workload, every page filled from the generator."""
    m = wl.model
    kp, vp = dap.pools(wl.n_pages, m.n_kv_heads, m.head_dim, device=device)
    for s in range(0, wl.n_pages, chunk):
        ids = np.arange(s, min(s + chunk, wl.n_pages))
        dap.store_pages(kp, vp, ids, wl.pages("k", ids, device), wl.pages("v", ids, device))
    return kp, vp


class OraclePool:
    """The oracle's view of a pool: generated page contents plus overlays of
    the slots the oracle wrote. Pages are generated on ``gen_device`` (the
    generator's bits do not depend on the device) and cached on the host."""

    def __init__(self, wl: W.Workload, gen_device="cpu"):
        self.wl = wl
        self.gen_device = gen_device
        self.overlay = {}          # page -> {index: (k_bits[Hkv, D], v_bits[Hkv, D])}
        self.cache = {}

    def write(self, slots, k_bits: np.ndarray, v_bits: np.ndarray):
        for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
            pg, i = int(s) // 64, int(s) % 64
            self.overlay.setdefault(pg, {})[i] = (k_bits[t], v_bits[t])
            self.cache.pop(pg, None)

    def prefetch(self, page_ids):
        ids = [int(p) for p in page_ids if int(p) not in self.cache]
        for s in range(0, len(ids), 1024):
            part = ids[s:s + 1024]
            k = to_np_bits(self.wl.pages("k", part, self.gen_device))
            v = to_np_bits(self.wl.pages("v", part, self.gen_device))
            for j, pg in enumerate(part):
                self._store(pg, k[j], v[j])

    def _store(self, pg, k, v):
        k, v = k.copy(), v.copy()
        for i, (kb, vb) in self.overlay.get(pg, {}).items():
            k[:, i, :] = kb
            v[:, i, :] = vb
        self.cache[pg] = (bf16.to_f64(k), bf16.to_f64(v))

    def read_page(self, pg):
        if pg not in self.cache:
            self.prefetch([pg])
        return self.cache[pg]


def row_pages(wl: W.Workload, rows, positions):
    """Every page id the given (row, position) queries read (whole ranges)."""
    ids = set()
    win = wl.model.window
    for r, p in zip(rows, positions):
        lo = max(0, p - win + 1) if win > 0 else 0
        for j in range(lo // 64, p // 64 + 1):
            ids.add(int(wl.table[r, j]))
    return sorted(ids)


class RoundedBits(np.ndarray):
    """bf16 bit patterns the oracle rounded from float64, carrying ``tie``: the
    mask of elements whose float64 value lies within 1e-12 of a bf16 rounding
    midpoint (bf16.near_tie). Only the array oracle_front returns carries it;
    slices, reshapes and arithmetic give plain strict arrays (tie None)."""

    def __array_finalize__(self, obj):
        self.tie = None


def _rounded(x):
    r = bf16.from_f64(x).view(RoundedBits)
    r.tie = bf16.near_tie(x, TIE_TOL)
    return r


def oracle_front(wl: W.Workload, qkv_bits: np.ndarray, positions, gains=None):
    """Oracle q (float64), rounded q and k bits (RoundedBits, with their
    near-tie masks), and v bits for tokens."""
    m = wl.model
    qg, kg = (gains if gains is not None else (None, None))
    q, k, vb = core.prepare_tokens(qkv_bits, positions, m.n_q_heads, m.n_kv_heads, m.head_dim,
                                   oracle_freqs(m), qg, kg, m.qk_norm_eps)
    return q, _rounded(q), _rounded(k), vb


def check_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str):
    """Elementwise |gpu - ref| <= ATOL + RTOL |ref| and relative RMS <= REL_RMS."""
    g = bf16.to_f64(gpu_bits).reshape(ref.shape)
    err = np.abs(g - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rel_rms = float(np.sqrt(np.sum((g - ref) ** 2) / max(np.sum(ref ** 2), 1e-300)))
    big = np.abs(ref) >= 1e-3
    max_rel = float(np.max(err[big] / np.abs(ref[big]))) if big.any() else 0.0
    msg = (f"{what}: max abs {err.max():.3e}, max rel(|ref|>=1e-3) {max_rel:.3e}, "
           f"rel rms {rel_rms:.3e}, {int(bad.sum())} of {bad.size} outside tolerance")
    assert np.all(np.isfinite(g)), what + ": non-finite output"
    assert not bad.any(), msg
    assert rel_rms <= REL_RMS, msg
    return msg


def check_bits(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str):
    """Rounded values must equal the oracle's rounding bit for bit. The only
    exception is an element the oracle flagged as lying within 1e-12 of a
    bf16 rounding midpoint (``ref_bits.tie``), where two correct float64
    evaluations may round to adjacent values: it may differ by one ulp. The
    number flagged is recorded in TIE_REPORT and printed at the session's end."""
    a = np.asarray(gpu_bits).astype(np.int64).reshape(-1)
    b = np.asarray(ref_bits).astype(np.int64).reshape(-1)
    assert a.shape == b.shape, f"{what}: {a.shape} values against {b.shape}"
    tie = getattr(ref_bits, "tie", None)
    tie = np.zeros(a.shape, bool) if tie is None else np.asarray(tie).reshape(-1)
    same = a == b
    off = ~same & ~tie
    assert not off.any(), (f"{what}: {int(off.sum())} of {a.size} values differ from the oracle's rounding "
                           f"(first at {int(np.nonzero(off)[0][0])}: {a[off][0]:#06x} vs {b[off][0]:#06x})")
    # adjacent bf16 values of the same sign differ by 1 in the bit pattern
    near = (np.abs(a - b) == 1) & ((a ^ b) & 0x8000 == 0)
    assert np.all(same | near), f"{what}: a flagged near-tie value differs by more than 1 ulp"
    TIE_REPORT.append((what, a.size, int(tie.sum()), int((~same).sum())))
    return int(tie.sum())


def oracle_attention(wl, opool: OraclePool, q_f64, positions, rows):
    opool.prefetch(row_pages(wl, rows, positions))
    return attention.paged(q_f64, positions, rows, wl.table, opool.read_page, wl.model.window)


def oracle_rows(wl: W.Workload, opool: OraclePool, qs, positions, rows, block=32):
    """Oracle attention for one or more query sets (e.g. q and the peaky 4q)
    at the same (row, position) pairs, row by row: each row's pages are
    regenerated (with the oracle's own writes in ``opool``) once for all the
    query sets and dropped before the next row, and its queries run in
    position-sorted blocks of ``block`` tokens through attention.attend_many.
    Memory stays bounded by one row, so every row of the largest pools can be
    checked. Returns a list of outputs, one per query set."""
    qs = [np.asarray(q, dtype=np.float64) for q in qs]
    positions = np.asarray(positions, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    outs = [np.empty_like(q) for q in qs]
    win = wl.model.window
    for r in np.unique(rows):
        idx = np.nonzero(rows == r)[0]
        idx = idx[np.argsort(positions[idx], kind="stable")]
        n = int(positions[idx].max()) + 1
        tmp = OraclePool(wl, opool.gen_device)
        tmp.overlay = opool.overlay
        tmp.prefetch(wl.table[r, :-(-n // 64)])
        K, V = attention.gather_row(wl.table[r], n, tmp.read_page)
        del tmp
        for s0 in range(0, len(idx), block):
            b = idx[s0:s0 + block]
            for q, out in zip(qs, outs):
                out[b] = attention.attend_many(q[b], K, V, positions[b], win)
        del K, V
    return outs


def torch_i32(a, device="cuda"):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)
