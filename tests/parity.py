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


def oracle_front(wl: W.Workload, qkv_bits: np.ndarray, positions, gains=None):
    """Oracle q (float64), rounded q and k bits, and v bits for tokens."""
    m = wl.model
    qg, kg = (gains if gains is not None else (None, None))
    q, k, vb = core.prepare_tokens(qkv_bits, positions, m.n_q_heads, m.n_kv_heads, m.head_dim,
                                   oracle_freqs(m), qg, kg, m.qk_norm_eps)
    return q, bf16.from_f64(q), bf16.from_f64(k), vb


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


def check_bits(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str, min_identical=0.9999):
    """Rounded values: >= 99.99% bit-identical and every one within 1 bf16 ulp."""
    a = gpu_bits.astype(np.int64).reshape(-1)
    b = ref_bits.astype(np.int64).reshape(-1)
    same = a == b
    # adjacent bf16 values of the same sign differ by 1 in the bit pattern
    ulp = np.abs(a - b)
    frac = same.mean() if same.size else 1.0
    assert frac >= min_identical, f"{what}: only {frac:.6f} of values bit-identical"
    assert np.all(same | ((ulp == 1) & ((a ^ b) & 0x8000 == 0))), f"{what}: a value differs by more than 1 ulp"
    return frac


def oracle_attention(wl, opool: OraclePool, q_f64, positions, rows):
    opool.prefetch(row_pages(wl, rows, positions))
    return attention.paged(q_f64, positions, rows, wl.table, opool.read_page, wl.model.window)


def torch_i32(a, device="cuda"):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)
