"""Causal, optionally windowed, grouped-query softmax attention in float64.

Sources ("Phi-3 Mini 4K Instruct" files, src/attention.linnet):
- `window_mask` and the `seen` masks of `decode`, `prefill`, `decode_rows`:
  a query at position p sees key positions j with j <= p and j > p - WINDOW
  (itself and WINDOW-1 before it); with no window, every j <= p;
- every entry scales scores by rsqrt(head_dim) before the softmax;
- `prefill_packed` / `packed`: token i sees token j iff they share a
  segment and the position test above holds (the `own` mask);
- `step_packed`: prompts attend among themselves, each row's step over its
  own row of the cache.
"Mistral 7B Instruct v0.3", Entries: `decode_paged` reads row b's positions
through the pages `table[b]` lists; `prefill_paged` lets each token attend
over its row's pages up to its position.

Readings: query head h reads kv head h // (Hq / Hkv) (consecutive query
heads share a kv head); for the paged prefill, a token's segment id names its
table row; queries are float64 and are not rounded.
"""
import math

import numpy as np

from .pages import PAGE


def key_range(p: int, window: int):
    """Inclusive range [lo, p] of key positions a query at p attends."""
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, p


def softmax_attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for q [..., nq, D], keys/values [..., n, D]."""
    s = np.matmul(q, np.swapaxes(keys, -1, -2)) * scale
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    return np.matmul(e, values) / np.sum(e, axis=-1, keepdims=True)


def gather_row(table_row, n_positions: int, read_page):
    """Positions 0..n_positions-1 of one table row, read page by page.

    read_page(page) -> (K [Hkv, 64, D], V [Hkv, 64, D]) float64.
    Returns K, V as [Hkv, n_positions, D]."""
    n_pg = -(-n_positions // PAGE)
    ks, vs = [], []
    for j in range(n_pg):
        k, v = read_page(int(table_row[j]))
        ks.append(k)
        vs.append(v)
    K = np.concatenate(ks, axis=1)[:, :n_positions]
    V = np.concatenate(vs, axis=1)[:, :n_positions]
    return K, V


def attend_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, p: int, window: int) -> np.ndarray:
    """One query token: q [Hq, D] over keys/values [Hkv, >p, D] of its row."""
    hq, d = q.shape
    hkv = K.shape[0]
    g = hq // hkv
    lo, hi = key_range(p, window)
    qg = q.reshape(hkv, g, d)
    out = softmax_attend(qg, K[:, lo:hi + 1], V[:, lo:hi + 1], 1.0 / math.sqrt(d))
    return out.reshape(hq, d)


def attend_many(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, window: int) -> np.ndarray:
    """Several query tokens of one row: q [n, Hq, D] at ``positions`` over the
    row's keys/values [Hkv, > max(positions), D].

    The same definition as attend_one for each query, written as one masked
    product: the scores of every query against every key of the block's span
    [min lo, max p], with keys outside a query's own range [lo, p] set to
    -inf before its softmax, so their weight is exactly 0. Because a zero
    weight still multiplies its key's value, every value in the span must be
    finite (the row's written history, as it is for consecutive positions)."""
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    n, hq, d = q.shape
    hkv = K.shape[0]
    g = hq // hkv
    lo = np.maximum(0, positions - window + 1) if window > 0 else np.zeros_like(positions)
    a, b = int(lo.min()), int(positions.max()) + 1
    Ks, Vs = K[:, a:b], V[:, a:b]                               # [Hkv, L, D]
    qg = q.reshape(n, hkv, g, d).transpose(1, 0, 2, 3).reshape(hkv, n * g, d)
    s = np.matmul(qg, np.swapaxes(Ks, -1, -2))                  # [Hkv, n*g, L]
    s *= 1.0 / math.sqrt(d)
    j = np.arange(a, b)
    seen = (j[None, :] >= lo[:, None]) & (j[None, :] <= positions[:, None])   # [n, L]
    np.copyto(s, -np.inf, where=~np.repeat(seen, g, axis=0)[None])
    s -= np.max(s, axis=-1, keepdims=True)
    e = np.exp(s, out=s)
    out = np.matmul(e, Vs) / np.sum(e, axis=-1, keepdims=True)             # [Hkv, n*g, D]
    return out.reshape(hkv, n, g, d).transpose(1, 0, 2, 3).reshape(n, hq, d)


def paged(q: np.ndarray, positions, rows, table: np.ndarray, read_page, window: int = 0) -> np.ndarray:
    """Attention of query tokens over their rows' pages.

    q: [T, Hq, D] float64; positions, rows: [T]; table: [rows, table_ld].
    Covers both paged entries: decode (one token per row, rows = the
    decoding rows) and packed prefill (rows = segment ids)."""
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty_like(q)
    for r in np.unique(rows):
        idx = np.nonzero(rows == r)[0]
        n = int(positions[idx].max()) + 1
        K, V = gather_row(table[r], n, read_page)
        for t in idx:
            out[t] = attend_one(q[t], K, V, int(positions[t]), window)
    return out


def contiguous(q: np.ndarray, positions, rows, cache_k: np.ndarray, cache_v: np.ndarray,
               window: int = 0) -> np.ndarray:
    """The same attention over dense caches [Batch, Hkv, MaxSeq, D] (no pages)."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    for t in range(q.shape[0]):
        r = int(rows[t])
        out[t] = attend_one(q[t], cache_k[r], cache_v[r], int(positions[t]), window)
    return out


def packed_inpass(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions, segments,
                  window: int = 0) -> np.ndarray:
    """The pages' `packed` entry: attention among the pass's own tokens under
    the `own` mask (same segment, key position <= query position, within the
    window). q [P, Hq, D], k/v [P, Hkv, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    segments = np.asarray(segments, dtype=np.int64)
    P, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.empty_like(q)
    for i in range(P):
        own = (segments == segments[i]) & (positions <= positions[i])
        if window > 0:
            own &= positions > positions[i] - window
        j = np.nonzero(own)[0]
        Kj = np.swapaxes(k[j], 0, 1)          # [Hkv, n, D]
        Vj = np.swapaxes(v[j], 0, 1)
        o = softmax_attend(q[i].reshape(hkv, g, d), Kj, Vj, 1.0 / math.sqrt(d))
        out[i] = o.reshape(hq, d)
    return out
