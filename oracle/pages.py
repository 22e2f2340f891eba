"""Page addressing, the pool layout and the K/V write.

Sources: "Mistral 7B Instruct v0.3", Entries table: `decode_paged` keeps a
pool of positions in pages of PageSize 64 and row b's positions lie in the
pages `table[b]` lists; `prefill_paged` writes each token at its place in the
pool. "Phi-3 Mini 4K Instruct" files, src/attention.linnet: the caches are
[Batch, Heads, MaxSeq, D] state written at each token's (row, position)
(`write_rows`, `write_tokens`) and nothing else in them changes.

Position j of table row r lives in physical page table[r][j // 64], at slot
index j % 64 inside it; its pool slot number is page * 64 + j % 64.

The oracle keeps its pools in a layout of its own (the pages fix only
where a position lives, not how a page stores its elements), bf16:
  K pool [n_pages, n_kv_heads, 64, D]   one page tile per kv head, slot-major
  V pool [n_pages, n_kv_heads, D, 64]   one page tile per kv head, dim-major
It is not the GPU library's tile layout: comparisons between the two go
through logical [page, kv head, slot, dim] contents (page_logical here, the
library's published per-element tile offsets on the other side).
"""
import numpy as np

PAGE = 64


def slot_of(table: np.ndarray, rows, positions) -> np.ndarray:
    """Pool slot numbers of (row, position) pairs, int64."""
    rows = np.asarray(rows, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    page = np.asarray(table, dtype=np.int64)[rows, positions // PAGE]
    return page * PAGE + positions % PAGE


def k_offset(slot, head, dim, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Element offset of K[slot, head, dim] in the K pool."""
    slot = np.asarray(slot, dtype=np.int64)
    return ((slot // PAGE * n_kv_heads + head) * PAGE + slot % PAGE) * head_dim + dim


def v_offset(slot, head, dim, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Element offset of V[slot, head, dim] in the V pool (dim-major tiles)."""
    slot = np.asarray(slot, dtype=np.int64)
    return ((slot // PAGE * n_kv_heads + head) * head_dim + dim) * PAGE + slot % PAGE


def write(k_pool: np.ndarray, v_pool: np.ndarray, slots, k_bits: np.ndarray, v_bits: np.ndarray):
    """Return copies of the flat pools with token t's K/V placed at slots[t].

    k_bits, v_bits: [T, n_kv_heads, D] bf16 bit patterns. Every other
    element keeps its bits."""
    T, hkv, d = k_bits.shape
    kp = np.array(k_pool, copy=True).reshape(-1)
    vp = np.array(v_pool, copy=True).reshape(-1)
    s = np.asarray(slots, dtype=np.int64)[:, None, None]
    h = np.arange(hkv, dtype=np.int64)[None, :, None]
    dd = np.arange(d, dtype=np.int64)[None, None, :]
    kp[k_offset(s, h, dd, hkv, d)] = k_bits
    vp[v_offset(s, h, dd, hkv, d)] = v_bits
    return kp.reshape(np.shape(k_pool)), vp.reshape(np.shape(v_pool))


def page_logical(k_pool: np.ndarray, v_pool: np.ndarray, page: int, n_kv_heads: int, head_dim: int):
    """Logical (K, V) contents of one physical page: two [n_kv_heads, 64, D] arrays of bits."""
    s = page * PAGE + np.arange(PAGE, dtype=np.int64)[None, :, None]
    h = np.arange(n_kv_heads, dtype=np.int64)[:, None, None]
    dd = np.arange(head_dim, dtype=np.int64)[None, None, :]
    kp = np.asarray(k_pool).reshape(-1)
    vp = np.asarray(v_pool).reshape(-1)
    return (kp[k_offset(s, h, dd, n_kv_heads, head_dim)],
            vp[v_offset(s, h, dd, n_kv_heads, head_dim)])


def empty_pools(n_pages: int, n_kv_heads: int, head_dim: int, fill: int = 0):
    """Flat-shaped K and V pools of bf16 bits in the oracle's layout."""
    k = np.full((n_pages, n_kv_heads, PAGE, head_dim), fill, dtype=np.uint16)
    v = np.full((n_pages, n_kv_heads, head_dim, PAGE), fill, dtype=np.uint16)
    return k, v


def pools_from_logical(k_logical: np.ndarray, v_logical: np.ndarray):
    """Pools in the oracle's layout from logical [n_pages, Hkv, 64, D] contents."""
    return (np.ascontiguousarray(k_logical),
            np.ascontiguousarray(np.swapaxes(v_logical, -1, -2)))
