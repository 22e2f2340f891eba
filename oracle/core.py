"""The per-token front half of the path: split, QK-norm, rope, write.

Sources: "Phi-3 Mini 4K Instruct" (model card and files,
src/attention.linnet): the fused projection is query, then key, then value
along its output axis, and head h owns columns h*D .. h*D+D-1 of its slice
(`split_heads`); q and k are roped, v is not; each token's k and v go to its
row at its position. "Qwen3-4B": QK-norm per head slice, before rope.
"Mistral 7B Instruct v0.3", Entries: `prefill_paged(tokens, positions, rows,
slots, ...)` writes each token at its place in the pool.

Reading: a token's slot is `slots[t]` when given, else the slot its
(row, position) addresses through the table. Rounded results are bf16 of the
float64 value, rounded once.
"""
import numpy as np

from . import bf16, norm, pages, rope


def prepare_tokens(qkv_bits: np.ndarray, positions, n_q_heads: int, n_kv_heads: int,
                   head_dim: int, freqs: np.ndarray, q_gain=None, k_gain=None, eps=None):
    """qkv_bits: [T, (Hq + 2 Hkv) * D] bf16 bits.

    Returns (q, k, v_bits): q [T, Hq, D] and k [T, Hkv, D] float64 after the
    optional norm and rope; v_bits [T, Hkv, D] the untouched value bits."""
    T = qkv_bits.shape[0]
    D = head_dim
    x = bf16.to_f64(qkv_bits)
    q = x[:, : n_q_heads * D].reshape(T, n_q_heads, D)
    k = x[:, n_q_heads * D: (n_q_heads + n_kv_heads) * D].reshape(T, n_kv_heads, D)
    v_bits = np.asarray(qkv_bits)[:, (n_q_heads + n_kv_heads) * D:].reshape(T, n_kv_heads, D)
    if q_gain is not None:
        q = norm.rms_norm_heads(q, bf16.to_f64(q_gain), eps)
        k = norm.rms_norm_heads(k, bf16.to_f64(k_gain), eps)
    q = rope.rotate(q, positions, freqs)
    k = rope.rotate(k, positions, freqs)
    return q, k, np.asarray(v_bits).astype(np.uint16)


def write_tokens(k_pool, v_pool, table, rows, positions, slots, k, v_bits):
    """Pools after writing every token's roped k (rounded to bf16) and raw v."""
    if slots is None:
        slots = pages.slot_of(table, rows, positions)
    return pages.write(k_pool, v_pool, slots, bf16.from_f64(k), v_bits)
