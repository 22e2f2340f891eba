"""Seeded synthetic inputs for the paged decoder-attention core.

This module is shared input plumbing: both the fp64 oracle's tests and the
HIP path's tests/bench draw their inputs from here, so both see the same
bits. It holds none of the method's arithmetic (no rope, no norm, no
softmax, no page addressing): only random values, index arrays and the five
workload shapes.

Values. Every bf16 value is drawn by a counter-based generator, so any
slice (one page, one token row) can be regenerated on its own, on the CPU or
on the GPU, with identical bits:

  u(key, i) = fmix32( fmix32( lo32(i) XOR k0 ) XOR lo32( hi32(i) + k1 ) )

where fmix32 is the 32-bit finalizer of MurmurHash3 (Appleby, public domain:
x ^= x>>16; x *= 0x85ebca6b; x ^= x>>13; x *= 0xc2b2ae35; x ^= x>>16) and
(k0, k1) come from a BLAKE2b digest of the tensor's name. A standard normal
value is the inverse-CDF quantile table entry ndtri((k + 1/2) / 65536) for
k = u >> 16, rounded to bf16 once when the table is built. Only integer
operations and one table gather run per element, so CPU and GPU agree bit
for bit.

Index arrays (lengths, positions, page permutations) are small and drawn on
the host with numpy's PCG64 seeded from SeedSequence(0).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

SEED = 0
PAGE = 64  # positions per page (the pages' PageSize)

_M32 = 0xFFFFFFFF


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding values in [0, 2**32),
    split into 16-bit halves so no int64 product overflows."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + ((hi * (c & 0xFFFF)) << 16)) & _M32


def _fmix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x85EBCA6B)
    x = x ^ (x >> 13)
    x = _mul32(x, 0xC2B2AE35)
    x = x ^ (x >> 16)
    return x


def stream_key(*names) -> Tuple[int, int]:
    """Two 32-bit keys for a named tensor stream (seed folded in)."""
    h = hashlib.blake2b(("|".join(str(n) for n in (SEED,) + names)).encode(), digest_size=8).digest()
    return int.from_bytes(h[:4], "little"), int.from_bytes(h[4:], "little")


def hash_u32(key: Tuple[int, int], idx: torch.Tensor) -> torch.Tensor:
    """Counter-based 32-bit value for every int64 counter in ``idx``."""
    k0, k1 = key
    lo = idx & _M32
    hi = (idx >> 32) & _M32
    a = _fmix32(lo ^ k0)
    return _fmix32(a ^ ((hi + k1) & _M32))


_TABLE_CACHE = {}


def normal_table(device="cpu") -> torch.Tensor:
    """65536 bf16 quantiles of N(0,1), as int16 bit patterns."""
    dev = torch.device(device)
    if dev not in _TABLE_CACHE:
        if torch.device("cpu") not in _TABLE_CACHE:
            k = torch.arange(65536, dtype=torch.float64)
            q = torch.special.ndtri((k + 0.5) / 65536.0)
            _TABLE_CACHE[torch.device("cpu")] = q.to(torch.float32).to(torch.bfloat16).view(torch.int16)
        _TABLE_CACHE[dev] = _TABLE_CACHE[torch.device("cpu")].to(dev)
    return _TABLE_CACHE[dev]


def normal_bf16(key, idx: torch.Tensor) -> torch.Tensor:
    """bf16 N(0,1) bit patterns (int16) for int64 counters ``idx``."""
    table = normal_table(idx.device)
    return table[hash_u32(key, idx) >> 16]


def uniform_bf16(key, idx: torch.Tensor, lo: float, hi: float) -> torch.Tensor:
    """bf16 U(lo, hi) bit patterns (int16) for int64 counters ``idx``."""
    u = (hash_u32(key, idx).to(torch.float64) + 0.5) / 4294967296.0
    return (lo + (hi - lo) * u).to(torch.float32).to(torch.bfloat16).view(torch.int16)


def normal_matrix(key, rows: int, cols: int, device="cpu", row0: int = 0) -> torch.Tensor:
    """[rows, cols] bf16 N(0,1) bits; element (r, c) uses counter (row0+r)*cols + c."""
    idx = (torch.arange(rows, dtype=torch.int64, device=device)[:, None] + row0) * cols \
        + torch.arange(cols, dtype=torch.int64, device=device)[None, :]
    return normal_bf16(key, idx)


def page_values(key, page_ids, n_kv_heads: int, head_dim: int, device="cpu") -> torch.Tensor:
    """Logical contents of physical pages: [n, n_kv_heads, PAGE, head_dim] bf16 bits.

    Element (page, h, s, d) uses counter ((page*Hkv + h)*PAGE + s)*D + d, so a
    page's contents depend only on its physical id."""
    pid = torch.as_tensor(np.asarray(page_ids, dtype=np.int64), device=device)
    per_page = n_kv_heads * PAGE * head_dim
    idx = pid[:, None] * per_page + torch.arange(per_page, dtype=torch.int64, device=device)[None, :]
    return normal_bf16(key, idx).view(-1, n_kv_heads, PAGE, head_dim)


def bf16_bits_to_float(bits: torch.Tensor) -> torch.Tensor:
    """Reinterpret int16 bf16 bit patterns as a bfloat16 tensor (no rounding)."""
    return bits.view(torch.bfloat16)


# ---------------------------------------------------------------------------
# Model constants and workload shapes.
# ---------------------------------------------------------------------------

@dataclass
class ModelShape:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    window: int = 0                       # 0 = no window
    llama3: Optional[Tuple[float, float, float, float]] = None  # factor, low_ff, high_ff, original
    qk_norm_eps: Optional[float] = None   # None = no QK-norm
    max_position: int = 4096

    @property
    def qkv_width(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


@dataclass
class Workload:
    """One synthetic workload: model constants, page pool and index arrays.

    All index arrays are int32 numpy arrays. ``table`` is [rows, table_ld]
    with -1 in entries a row never uses."""
    name: str
    model: ModelShape
    n_pages: int
    table: np.ndarray
    # prefill part (packed prompts)
    pre_positions: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    pre_segments: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    # decode part (one token per row)
    dec_positions: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    dec_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    note: str = ""

    @property
    def n_pre(self) -> int:
        return int(self.pre_positions.shape[0])

    @property
    def n_dec(self) -> int:
        return int(self.dec_positions.shape[0])

    def key(self, *names):
        return stream_key(self.name, *names)

    def qkv(self, tag: str, n_tokens: int, device="cpu", row0: int = 0) -> torch.Tensor:
        """Pre-rope fused q,k,v rows [n_tokens, (Hq+2Hkv)*D] as bf16 bits."""
        return normal_matrix(self.key("qkv", tag), n_tokens, self.model.qkv_width, device, row0)

    def pages(self, which: str, page_ids, device="cpu") -> torch.Tensor:
        """Pre-filled logical page contents for 'k' or 'v'."""
        m = self.model
        return page_values(self.key("pool", which), page_ids, m.n_kv_heads, m.head_dim, device)

    def gains(self, which: str, device="cpu") -> torch.Tensor:
        """QK-norm per-dim gains [D] for 'q' or 'k', U(0.5, 1.5) in bf16 bits."""
        idx = torch.arange(self.model.head_dim, dtype=torch.int64, device=device)
        return uniform_bf16(self.key("gain", which), idx, 0.5, 1.5)


def _rng(name: str) -> np.random.Generator:
    ss = np.random.SeedSequence(SEED)
    # one child stream per workload, keyed by a stable digest of its name
    salt = int.from_bytes(hashlib.blake2b(name.encode(), digest_size=4).digest(), "little")
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, salt])))


def _assign_pages(rng, needs: List[int], table_ld: int, shared: Optional[dict] = None):
    """Give each row ``needs[r]`` physical pages from one seeded permutation of
    the pool. ``shared`` maps row -> list of (table slot, shared page ordinal)
    that reuse the first pages of the permutation instead."""
    shared = shared or {}
    n_shared = 0
    for lst in shared.values():
        for _, k in lst:
            n_shared = max(n_shared, k + 1)
    own = sum(needs) - sum(len(v) for v in shared.values())
    n_pages = n_shared + own
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((len(needs), table_ld), -1, np.int32)
    nxt = n_shared
    for r, need in enumerate(needs):
        sh = dict(shared.get(r, []))
        for j in range(need):
            if j in sh:
                table[r, j] = perm[sh[j]]
            else:
                table[r, j] = perm[nxt]
                nxt += 1
    assert nxt == n_pages
    return n_pages, table


def _ceil_div(a, b):
    return -(-a // b)


def tiny(permuted: bool = False) -> Workload:
    """Tiny single layer: Hq 4, Hkv 2, D 64, theta 1e4, no window; one
    128-token prompt at positions 0..127 then 16 decode steps at 128..143."""
    m = ModelShape("tiny", 4, 2, 64, 1e4, max_position=144)
    if permuted:
        table = np.array([[2, 0, 1]], np.int32)
    else:
        table = np.array([[0, 1, 2]], np.int32)
    return Workload("tiny" + ("-perm" if permuted else ""), m, 3, table,
                    pre_positions=np.arange(128, dtype=np.int32),
                    pre_segments=np.zeros(128, np.int32),
                    dec_positions=np.array([128], np.int32), dec_rows=np.zeros(1, np.int32),
                    note="decode steps run at 128..143, one at a time")


PHI3_PROMPTS = (512, 1024, 1536, 1024)
PHI3_DECODE_END = 3000


def phi3() -> Workload:
    """Phi-3-mini shape: Hq = Hkv = 32, D 96, theta 1e4, window 2047; a
    256-page pool (4 rows x 64 pages, MaxSeq 4096 each) under one seeded
    permutation; 4 packed prompts of 512/1024/1536/1024 tokens."""
    m = ModelShape("phi3", 32, 32, 96, 1e4, window=2047, max_position=4096)
    rng = _rng("phi3")
    n_pages, table = _assign_pages(rng, [64] * 4, 64)
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in PHI3_PROMPTS])
    seg = np.concatenate([np.full(L, r, np.int32) for r, L in enumerate(PHI3_PROMPTS)])
    return Workload("phi3", m, n_pages, table, pre_positions=pos, pre_segments=seg,
                    dec_positions=np.full(4, PHI3_DECODE_END, np.int32),
                    dec_rows=np.arange(4, dtype=np.int32),
                    note="decode loop from each prompt end to position 3000")


def phi3_decode_schedule():
    """Decode loop: at step t, row m is active iff L_m + t <= 3000, at
    position L_m + t. Returns a list of (rows, positions) per step."""
    steps = []
    t = 0
    while True:
        rows = [r for r, L in enumerate(PHI3_PROMPTS) if L + t <= PHI3_DECODE_END]
        if not rows:
            break
        steps.append((np.array(rows, np.int32),
                      np.array([PHI3_PROMPTS[r] + t for r in rows], np.int32)))
        t += 1
    return steps


def mistral() -> Workload:
    """Mistral-7B-v0.3 decode: Hq 32, Hkv 8, D 128, theta 1e6, no window;
    64 rows, context L_b ~ U{1024..32768}, new token at position L_b - 1."""
    m = ModelShape("mistral", 32, 8, 128, 1e6, max_position=32768)
    rng = _rng("mistral")
    L = rng.integers(1024, 32768, size=64, endpoint=True).astype(np.int32)
    needs = [_ceil_div(int(x), PAGE) for x in L]
    n_pages, table = _assign_pages(rng, needs, 512)
    return Workload("mistral", m, n_pages, table, dec_positions=(L - 1).astype(np.int32),
                    dec_rows=np.arange(64, dtype=np.int32))


LLAMA_PREFIX = 57344
LLAMA_CHUNK = 8192


def llama31() -> Workload:
    """Llama-3.1-8B chunked prefill: Hq 32, Hkv 8, D 128, theta 5e5 with
    llama3 scaling (8, 1, 4, 8192); one row of 1024 pages; an 8192-token
    chunk at positions 57344..65535 over a pre-filled prefix."""
    m = ModelShape("llama31", 32, 8, 128, 5e5, llama3=(8.0, 1.0, 4.0, 8192.0), max_position=65536)
    rng = _rng("llama31")
    n_pages, table = _assign_pages(rng, [1024], 1024)
    pos = np.arange(LLAMA_PREFIX, LLAMA_PREFIX + LLAMA_CHUNK, dtype=np.int32)
    return Workload("llama31", m, n_pages, table, pre_positions=pos,
                    pre_segments=np.zeros(LLAMA_CHUNK, np.int32))


def qwen3() -> Workload:
    """Qwen3-4B step: Hq 32, Hkv 8, D 128, QK-norm eps 1e-6, theta 1e6.
    Rows 0-7 are prompts of 256 new tokens (rows 0-3 at 0..255; rows 4-7 at
    128..383 after a 128-position prefix held in 2 physical pages they
    share); rows 8-135 decode one token at p ~ U{512..40959}."""
    m = ModelShape("qwen3", 32, 8, 128, 1e6, qk_norm_eps=1e-6, max_position=40960)
    rng = _rng("qwen3")
    dec_p = rng.integers(512, 40959, size=128, endpoint=True).astype(np.int32)
    needs = [4] * 4 + [6] * 4 + [_ceil_div(int(p) + 1, PAGE) for p in dec_p]
    shared = {r: [(0, 0), (1, 1)] for r in range(4, 8)}
    n_pages, table = _assign_pages(rng, needs, 640, shared)
    pos = np.concatenate([np.arange(256, dtype=np.int32)] * 4 +
                         [np.arange(128, 384, dtype=np.int32)] * 4)
    seg = np.repeat(np.arange(8, dtype=np.int32), 256)
    return Workload("qwen3", m, n_pages, table, pre_positions=pos, pre_segments=seg,
                    dec_positions=dec_p, dec_rows=np.arange(8, 136, dtype=np.int32))


def mistral_contiguous() -> Workload:
    """The Mistral decode rows on a contiguous cache: 64 rows of MaxSeq 32768,
    row r owning pages 512r .. 512r + 511 (the identity table), same
    contexts as mistral()."""
    src = mistral()
    table = np.arange(64 * 512, dtype=np.int32).reshape(64, 512)
    return Workload("mistral_contiguous", src.model, 64 * 512, table, dec_positions=src.dec_positions,
                    dec_rows=src.dec_rows)


PACKED_PROMPTS = 8
PACKED_LEN = 4096


def packed_train() -> Workload:
    """A packed training forward on the Llama-3.1-8B shape: 8 prompts of 4096
    tokens packed end to end, each at positions 0..4095, attending among
    themselves (no cache, so no pool)."""
    m = ModelShape("llama31", 32, 8, 128, 5e5, llama3=(8.0, 1.0, 4.0, 8192.0), max_position=65536)
    pos = np.tile(np.arange(PACKED_LEN, dtype=np.int32), PACKED_PROMPTS)
    seg = np.repeat(np.arange(PACKED_PROMPTS, dtype=np.int32), PACKED_LEN)
    return Workload("packed_train", m, 0, np.zeros((0, 1), np.int32), pre_positions=pos, pre_segments=seg)


ALL = {"tiny": tiny, "phi3": phi3, "mistral": mistral, "llama31": llama31, "qwen3": qwen3,
       "mistral_contiguous": mistral_contiguous, "packed_train": packed_train}
