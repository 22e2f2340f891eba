// Fused per-head QK-RMSNorm + rotary positions + page write.
//
// One workgroup per token. The token's D/2 rotation angles p*f[i] and their
// sine/cosine are computed once in float64 into LDS, then every q and k head
// of the token is normed (optionally), rotated and rounded to bf16 once, and
// v is copied. This is a bandwidth-bound pass (a few flops per byte), so the
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

template <int D>
__global__ __launch_bounds__(kWriteThreads) void rope_write_kernel(WriteArgs a) {
    static_assert(D % 16 == 0 && D / 16 <= kLanesPerHead, "head_dim");
    constexpr int kHalf = D / 2;
    constexpr int kChunks = D / 16;   // 8-pair chunks per head half

    __shared__ double s_cos[kHalf];
    __shared__ double s_sin[kHalf];
    __shared__ long long s_slot;      // -1: do not write K/V
    __shared__ int s_pos_ok;

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int p = a.positions[t];

    if (tid == 0) {
        int pos_ok = (p >= 0 && p < a.max_position);
        long long slot = -1;
        if (!pos_ok) {
            atomicOr(a.err, kErrPosition);
        } else if (a.slots) {
            const long long s = a.slots[t];
            if (s < 0 || s >= (long long)a.n_pages * kPage) atomicOr(a.err, kErrSlot);
            else slot = s;
        } else {
            const int r = a.rows[t];
            const int j = p / kPage;
            if (r < 0 || r >= a.n_table_rows) {
                atomicOr(a.err, kErrRow);
            } else if (j >= a.table_ld) {
                atomicOr(a.err, kErrTable);
            } else {
                const int pg = a.table[(long long)r * a.table_ld + j];
                if (pg < 0 || pg >= a.n_pages) atomicOr(a.err, kErrPage);
                else slot = (long long)pg * kPage + (p % kPage);
            }
        }
        s_slot = slot;
        s_pos_ok = pos_ok;
    }
    for (int i = tid; i < kHalf; i += kWriteThreads) {
        const double ang = (double)p * a.inv_freq[i];
        double sn, cs;
        sincos(ang, &sn, &cs);
        s_sin[i] = sn;
        s_cos[i] = cs;
    }
    __syncthreads();
    if (!s_pos_ok) return;
    const long long slot = s_slot;
    const long long page = slot >> 6;
    const int in_page = (int)(slot & (kPage - 1));

    // ---- q and k heads: norm, rotate, round, store ------------------------
    const int n_rope_heads = a.n_q_heads + a.n_kv_heads;
    const int n_items = n_rope_heads * kLanesPerHead;
    const int n_iter = (n_items + kWriteThreads - 1) / kWriteThreads;
    for (int it = 0; it < n_iter; ++it) {         // uniform trip count: shuffles stay wave-wide
        const int item = it * kWriteThreads + tid;
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
                const double c = s_cos[8 * j + i];
                const double s = s_sin[8 * j + i];
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
            dst = a.k_pool + ((page * a.n_kv_heads + kh) * kPage + in_page) * (long long)D;
        }
        *reinterpret_cast<u32x4*>(dst + 8 * j) = ol;
        *reinterpret_cast<u32x4*>(dst + kHalf + 8 * j) = oh;
    }

    // ---- v heads: bit copy into the dim-major V page tile ------------------
    if (slot < 0) return;
    constexpr int kVChunks = D / 8;
    const int n_v = a.n_kv_heads * kVChunks;
    for (int item = tid; item < n_v; item += kWriteThreads) {
        const int kh = item / kVChunks;
        const int c = item % kVChunks;
        const u32x4 x = *reinterpret_cast<const u32x4*>(a.v + (long long)t * a.ld_in + (long long)kh * D + 8 * c);
        uint16_t* dst = a.v_pool + ((page * a.n_kv_heads + kh) * D + 8 * c) * (long long)kPage + in_page;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            dst[(2 * w) * kPage] = (uint16_t)(x[w] & 0xffffu);
            dst[(2 * w + 1) * kPage] = (uint16_t)(x[w] >> 16);
        }
    }
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t s, Profiler* prof) {
    if (a.n_tokens <= 0) return hipSuccess;
    dim3 grid(a.n_tokens), block(kWriteThreads);
    if (prof) prof->begin(DAP_KERNEL_WRITE, s);
    switch (a.head_dim) {
        case 64: hipLaunchKernelGGL(rope_write_kernel<64>, grid, block, 0, s, a); break;
        case 96: hipLaunchKernelGGL(rope_write_kernel<96>, grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL(rope_write_kernel<128>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_WRITE, s);
    return hipGetLastError();
}

}  // namespace dap
