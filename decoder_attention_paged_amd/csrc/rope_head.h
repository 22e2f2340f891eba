// Per-head QK-RMSNorm + rotary positions + rounding of one token, shared by
// the page-write kernel and the decode that writes its own step tokens, so
// both produce the same bits. float64 throughout, one rounding to bf16.
//
// Sources: "Phi-3 Mini 4K Instruct" files, src/rope.linnet (tables: angles
// s*f[i], concatenated so frequency i serves dims i and i+D/2) and
// src/attention.linnet (rope of q and k; write_tokens at each token's row
// and position); "Qwen3-4B" (QK-norm per head slice, before rope, eps 1e-6).
#pragma once
#include "dap_internal.h"

namespace dap {

namespace {

constexpr int kLanesPerHead = 8;   // rotation work of one head: up to 8 lanes x 8 pairs

// Slot of token t (-1 if an index is out of range; flags the error word).
__device__ __forceinline__ long long token_slot(const WriteArgs& a, int t, int p, bool flag) {
    if (p < 0 || p >= a.max_position) {
        if (flag) atomicOr(a.err, kErrPosition);
        return -1;
    }
    if (a.slots) {
        const long long s = a.slots[t];
        if (s < 0 || s >= (long long)a.n_pages * kPage) {
            if (flag) atomicOr(a.err, kErrSlot);
            return -1;
        }
        return s;
    }
    const int r = a.rows[t];
    const int j = p / kPage;
    if (r < 0 || r >= a.n_table_rows) {
        if (flag) atomicOr(a.err, kErrRow);
        return -1;
    }
    if (j >= a.table_ld) {
        if (flag) atomicOr(a.err, kErrTable);
        return -1;
    }
    const int pg = a.table[(long long)r * a.table_ld + j];
    if (pg < 0 || pg >= a.n_pages) {
        if (flag) atomicOr(a.err, kErrPage);
        return -1;
    }
    return (long long)pg * kPage + (p % kPage);
}

// The token's D/2 angles p*f[i] and their sine and cosine, in float64.
template <int D>
__device__ __forceinline__ void angle_table(const double* inv_freq, int p, int tid, int n_threads, double* cs,
                                            double* sn) {
    for (int i = tid; i < D / 2; i += n_threads) {
        const double ang = (double)p * inv_freq[i];
        double s, c;
        sincos(ang, &s, &c);
        sn[i] = s;
        cs[i] = c;
    }
}

// One q or k head chunk pair: lanes 8h..8h+7 of a head hold its dims
// 8j..8j+7 and D/2+8j..D/2+8j+7 (rlo, rhi, raw bf16). Norm (the head's sum
// of squares over its 8 lanes), rotate by the token's angles (cs, sn),
// round once to bf16 into ol, oh. Every lane of the wave calls it (the
// shuffles are wave-wide); the result of an inactive lane is unspecified.
template <int D>
__device__ __forceinline__ void rope_chunk_pair(const WriteArgs& a, bool is_q, int j, bool active, u32x4 rlo,
                                                u32x4 rhi, const double* cs, const double* sn, u32x4& ol,
                                                u32x4& oh) {
    constexpr int kHalf = D / 2;
    double xl[8], xh[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        xl[2 * w] = (double)bf16_to_f32(rlo[w] & 0xffffu);
        xl[2 * w + 1] = (double)bf16_to_f32(rlo[w] >> 16);
        xh[2 * w] = (double)bf16_to_f32(rhi[w] & 0xffffu);
        xh[2 * w + 1] = (double)bf16_to_f32(rhi[w] >> 16);
    }
    if (a.qk_norm) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += xl[i] * xl[i] + xh[i] * xh[i];
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        if (active) {
            // one reciprocal instead of a division per element: the float64
            // value moves by an ulp or so, which changes the bf16 rounding
            // only at a rounding near-tie
            const double inv = 1.0 / sqrt(ss / (double)D + a.eps);
            const uint16_t* g = is_q ? a.q_gain : a.k_gain;
            const u32x4 gl = *reinterpret_cast<const u32x4*>(g + 8 * j);
            const u32x4 gh = *reinterpret_cast<const u32x4*>(g + kHalf + 8 * j);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xl[2 * w] = (double)bf16_to_f32(gl[w] & 0xffffu) * xl[2 * w] * inv;
                xl[2 * w + 1] = (double)bf16_to_f32(gl[w] >> 16) * xl[2 * w + 1] * inv;
                xh[2 * w] = (double)bf16_to_f32(gh[w] & 0xffffu) * xh[2 * w] * inv;
                xh[2 * w + 1] = (double)bf16_to_f32(gh[w] >> 16) * xh[2 * w + 1] * inv;
            }
        }
    }
    if (!active) return;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t l2[2], h2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int i = 2 * w + e;
            const double c = cs[8 * j + i];
            const double s = sn[8 * j + i];
            l2[e] = f64_to_bf16(xl[i] * c - xh[i] * s);
            h2[e] = f64_to_bf16(xh[i] * c + xl[i] * s);
        }
        ol[w] = l2[0] | (l2[1] << 16);
        oh[w] = h2[0] | (h2[1] << 16);
    }
}

// rope_chunk_pair, then the store: q to q_out row t, k to the K tile of slot.
template <int D>
__device__ __forceinline__ void rope_item(const WriteArgs& a, int t, int head, int j, bool active, u32x4 rlo,
                                          u32x4 rhi, const double* cs, const double* sn, long long slot) {
    constexpr int kHalf = D / 2;
    const bool is_q = head < a.n_q_heads;
    u32x4 ol, oh;
    rope_chunk_pair<D>(a, is_q, j, active, rlo, rhi, cs, sn, ol, oh);
    if (!active) return;
    if (is_q) {
        uint16_t* dst = a.q_out + (long long)t * a.ld_q_out + (long long)head * D;
        *reinterpret_cast<u32x4*>(dst + 8 * j) = ol;
        *reinterpret_cast<u32x4*>(dst + kHalf + 8 * j) = oh;
        return;
    }
    if (slot < 0) return;
    const int kh = head - a.n_q_heads;
    const int in_page = (int)(slot & (kPage - 1));
    uint16_t* tile = a.k_pool + ((slot >> 6) * a.n_kv_heads + kh) * (long long)(D * kPage);
    *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, 8 * j, D)) = ol;
    *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, kHalf + 8 * j, D)) = oh;
}

}  // namespace

}  // namespace dap
