// Fused per-head QK-RMSNorm + rotary positions + page write.
//
// One wave per token for q and k: the token's D/2 rotation angles p*f[i]
// and their sine/cosine are computed once in float64 into LDS, then every q
// and k head of the token is normed (optionally), rotated and rounded to
// bf16 once. In the same launch, one workgroup per (64 tokens, kv head)
// copies v into the V tiles through an LDS transpose, so the consecutive
// slots of one dim are written as contiguous runs (the tile layout keeps 8
// consecutive keys of a dim together). Page tiles are in the library's
// tile layout, 16-byte chunks in the order the decode loads them. This is a
// bandwidth-bound pass (a few flops per byte), so the
// float64 arithmetic costs nothing and lets K pages match the float64
// definition bit for bit up to a final rounding tie.
//
// Sources: "Phi-3 Mini 4K Instruct" files, src/rope.linnet (tables: angles
// s*f[i], concatenated so frequency i serves dims i and i+D/2) and
// src/attention.linnet (q, k, v slices of the fused projection; rope of q
// and k; write_tokens at each token's row and position); "Qwen3-4B"
// (QK-norm per head slice, before rope, eps 1e-6).
#include "dap_internal.h"

namespace dap {

namespace {

constexpr int kWriteThreads = 256;
constexpr int kLanesPerHead = 8;   // rotation work of one head: up to 8 lanes x 8 pairs

constexpr int kVTile = 64;         // tokens per V-transpose workgroup

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

// V of kVTile consecutive tokens, per kv head: rows read coalesced, turned
// around in LDS, and stored with lanes running along tokens, so the tokens
// of one page land as contiguous runs of 8 keys per dim.
template <int D>
__device__ __forceinline__ void write_v_tile(const WriteArgs& a, int t0, int kh) {
    constexpr int VS = kVTile + 2;     // LDS row stride (elements), odd word stride
    __shared__ uint16_t s_v[D * VS];
    __shared__ long long s_slot[kVTile];
    const int tid = threadIdx.x;
    const int n = min(kVTile, a.n_tokens - t0);
    if (tid < kVTile) s_slot[tid] = tid < n ? token_slot(a, t0 + tid, a.positions[t0 + tid], false) : -1;
    {
        for (int c = tid; c < n * (D / 8); c += kWriteThreads) {
            const int tt = c / (D / 8), d8 = c % (D / 8);
            const u32x4 x = *reinterpret_cast<const u32x4*>(a.v + (long long)(t0 + tt) * a.ld_in +
                                                            (long long)kh * D + 8 * d8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                s_v[(8 * d8 + 2 * w) * VS + tt] = (uint16_t)(x[w] & 0xffffu);
                s_v[(8 * d8 + 2 * w + 1) * VS + tt] = (uint16_t)(x[w] >> 16);
            }
        }
        __syncthreads();
        for (int e = tid; e < D * kVTile; e += kWriteThreads) {
            const int d = e / kVTile, tt = e % kVTile;
            const long long slot = s_slot[tt];
            if (tt >= n || slot < 0) continue;
            a.v_pool[((slot >> 6) * a.n_kv_heads + kh) * (long long)(D * kPage) +
                     v_tile_offset((int)(slot & (kPage - 1)), d, D)] = s_v[d * VS + tt];
        }
    }
}

template <int D>
__global__ __launch_bounds__(kWriteThreads) void rope_write_kernel(WriteArgs a, int n_vtiles) {
    if ((int)blockIdx.x < n_vtiles * a.n_kv_heads) {  // uniform per workgroup
        write_v_tile<D>(a, (blockIdx.x / a.n_kv_heads) * kVTile, blockIdx.x % a.n_kv_heads);
        return;
    }
    static_assert(D % 16 == 0 && D / 16 <= kLanesPerHead, "head_dim");
    constexpr int kHalf = D / 2;
    constexpr int kChunks = D / 16;   // 8-pair chunks per head half
    constexpr int kTokens = kWriteThreads / 64;   // one wave per token

    __shared__ double s_cos[kTokens][kHalf];
    __shared__ double s_sin[kTokens][kHalf];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = ((int)blockIdx.x - n_vtiles * a.n_kv_heads) * kTokens + wave;
    const bool have = t < a.n_tokens;                // uniform per wave
    const int p = have ? a.positions[t] : 0;
    const bool pos_ok = have && p >= 0 && p < a.max_position;
    long long slot = -1;
    if (have && lane == 0) slot = token_slot(a, t, p, true);
    slot = __shfl(slot, 0);
    for (int i = lane; i < kHalf; i += 64) {
        const double ang = (double)p * a.inv_freq[i];
        double sn, cs;
        sincos(ang, &sn, &cs);
        s_sin[wave][i] = sn;
        s_cos[wave][i] = cs;
    }
    __syncthreads();
    if (!pos_ok) return;                             // uniform per wave; no barrier follows
    const long long page = slot >> 6;
    const int in_page = (int)(slot & (kPage - 1));

    // ---- q and k heads: norm, rotate, round, store ------------------------
    const int n_rope_heads = a.n_q_heads + a.n_kv_heads;
    const int n_items = n_rope_heads * kLanesPerHead;
    const int n_iter = (n_items + 63) / 64;
    for (int it = 0; it < n_iter; ++it) {         // uniform trip count: shuffles stay wave-wide
        const int item = it * 64 + lane;
        const int head = item / kLanesPerHead;
        const int j = item % kLanesPerHead;
        const bool active = head < n_rope_heads && j < kChunks;
        const bool is_q = head < a.n_q_heads;

        double xl[8], xh[8];
        const uint16_t* src = nullptr;
        if (active) {
            src = is_q ? a.q + (long long)t * a.ld_in + (long long)head * D
                       : a.k + (long long)t * a.ld_in + (long long)(head - a.n_q_heads) * D;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(src + 8 * j);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(src + kHalf + 8 * j);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xl[2 * w] = (double)bf16_to_f32(lo[w] & 0xffffu);
                xl[2 * w + 1] = (double)bf16_to_f32(lo[w] >> 16);
                xh[2 * w] = (double)bf16_to_f32(hi[w] & 0xffffu);
                xh[2 * w + 1] = (double)bf16_to_f32(hi[w] >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) { xl[i] = 0.0; xh[i] = 0.0; }
        }

        if (a.qk_norm) {
            double ss = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += xl[i] * xl[i] + xh[i] * xh[i];
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            if (active) {
                const double denom = sqrt(ss / (double)D + a.eps);
                const uint16_t* g = is_q ? a.q_gain : a.k_gain;
                const u32x4 gl = *reinterpret_cast<const u32x4*>(g + 8 * j);
                const u32x4 gh = *reinterpret_cast<const u32x4*>(g + kHalf + 8 * j);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    xl[2 * w] = (double)bf16_to_f32(gl[w] & 0xffffu) * xl[2 * w] / denom;
                    xl[2 * w + 1] = (double)bf16_to_f32(gl[w] >> 16) * xl[2 * w + 1] / denom;
                    xh[2 * w] = (double)bf16_to_f32(gh[w] & 0xffffu) * xh[2 * w] / denom;
                    xh[2 * w + 1] = (double)bf16_to_f32(gh[w] >> 16) * xh[2 * w + 1] / denom;
                }
            }
        }
        if (!active) continue;

        u32x4 ol, oh;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t l2[2], h2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * w + e;
                const double c = s_cos[wave][8 * j + i];
                const double s = s_sin[wave][8 * j + i];
                l2[e] = f64_to_bf16(xl[i] * c - xh[i] * s);
                h2[e] = f64_to_bf16(xh[i] * c + xl[i] * s);
            }
            ol[w] = l2[0] | (l2[1] << 16);
            oh[w] = h2[0] | (h2[1] << 16);
        }
        uint16_t* dst;
        if (is_q) {
            dst = a.q_out + (long long)t * a.ld_q_out + (long long)head * D;
        } else {
            if (slot < 0) continue;
            const int kh = head - a.n_q_heads;
            uint16_t* tile = a.k_pool + (page * a.n_kv_heads + kh) * (long long)(D * kPage);
            *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, 8 * j, D)) = ol;
            *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, kHalf + 8 * j, D)) = oh;
            continue;
        }
        *reinterpret_cast<u32x4*>(dst + 8 * j) = ol;
        *reinterpret_cast<u32x4*>(dst + kHalf + 8 * j) = oh;
    }

    // V is written by the tile workgroups
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t s, Profiler* prof) {
    if (a.n_tokens <= 0) return hipSuccess;
    const int n_vtiles = (a.n_tokens + kVTile - 1) / kVTile;
    const int n_token_groups = (a.n_tokens + kWriteThreads / 64 - 1) / (kWriteThreads / 64);
    dim3 grid(n_vtiles * a.n_kv_heads + n_token_groups), block(kWriteThreads);
    if (prof) prof->begin(DAP_KERNEL_WRITE, s);
    switch (a.head_dim) {
        case 64: hipLaunchKernelGGL(rope_write_kernel<64>, grid, block, 0, s, a, n_vtiles); break;
        case 96: hipLaunchKernelGGL(rope_write_kernel<96>, grid, block, 0, s, a, n_vtiles); break;
        case 128: hipLaunchKernelGGL(rope_write_kernel<128>, grid, block, 0, s, a, n_vtiles); break;
        default: return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_WRITE, s);
    return hipGetLastError();
}

}  // namespace dap
