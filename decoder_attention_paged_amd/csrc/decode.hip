// Decode over pages: one query token per row, split over chunks of pages,
// then an exact cross-chunk merge.
//
// Sources: "Mistral 7B Instruct v0.3", Entries (decode_paged: decode_rows
// over pages, row b's positions in the pages table[b] lists); "Phi-3 Mini 4K
// Instruct" files, src/attention.linnet (decode_rows: the row's query sees
// positions j <= p and j > p - WINDOW; scores scaled by rsqrt(head_dim)).
//
// One workgroup per (row, kv head, chunk of pages); each of
// its four waves walks every fourth page of the chunk with its own running
// max / sum / weighted-V sum. The g query heads that share the kv head are
// the N columns of 16x16x32 bf16 MFMAs: S[key][head] = K q^T and
// O^T[dim][head] += V^T P^T, so a page's K and V are read from HBM once for
// all g heads and the VALU only runs the softmax. A page tile is one
// contiguous block per kv head, stored in the order the waves load it, so
// every load of a wave reads one contiguous kilobyte.
//
// Merge: a row whose range fits one chunk is finished by that workgroup.
// Otherwise each chunk stores its fp32 (m, l, o) per head in the workspace
// and a second, small kernel merges the chunks with the max-shifted rescale
// (exactly the single-pass softmax in real arithmetic) and rounds to bf16.
#include "decode_chunk.h"

namespace dap {

namespace {

using namespace dec;

template <int D, bool kFused>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(AttnArgs a, int pps, int max_splits,
                                                                   float* __restrict__ ws, WriteArgs w) {
    extern __shared__ float s_o[];
    decode_chunk<D, kFused>(a, pps, max_splits, ws, w, blockIdx.x, s_o);
}

// Merge kernel: one workgroup per (row, kv head) whose range spans several
// chunks: M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// (Rows that fit one chunk were finished by the decode kernel.) Running it
// as its own launch makes the chunks' partials visible without a device-wide
// fence in every workgroup, which on a multi-XCD part writes back and
// invalidates the whole L2.
template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(AttnArgs a, int pps, int max_splits,
                                                                      const float* __restrict__ ws) {
    __shared__ float s_w[kMaxSplits * 16];     // per (chunk, head): m_s, then 2^(m_s - M)
    __shared__ float s_l[kMaxSplits * 16];     // per (chunk, head): l_s
    __shared__ float s_inv_l[16];
    const int kh = blockIdx.x;
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const RowRange rr = row_range(a, b, false);
    if (!rr.ok) return;
    const int n_splits = (rr.n_pg + pps - 1) / pps;
    if (n_splits == 1) return;
    const int G = a.n_q_heads / a.n_kv_heads;
    const long long slot0 = ((long long)b * a.n_kv_heads + kh) * max_splits;
    const float* part_o = ws + slot0 * G * D;
    const float* part_ml = ws + (long long)a.n_tokens * a.n_kv_heads * max_splits * G * D + slot0 * G * 2;
    // every chunk's (m, l) in parallel, then per head the max, the weights
    // and 1/L from LDS
    for (int i = tid; i < n_splits * G; i += kDecodeThreads) {
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * i);
        s_w[i] = ml.x;
        s_l[i] = ml.y;
    }
    __syncthreads();
    if (tid < G) {
        float M = -INFINITY;
        for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, s_w[sp * G + tid]);
        float L = 0.f;
        for (int sp = 0; sp < n_splits; ++sp) {
            const float w = M == -INFINITY ? 0.f : exp2f(s_w[sp * G + tid] - M);
            s_w[sp * G + tid] = w;
            L += w * s_l[sp * G + tid];
        }
        s_inv_l[tid] = L > 0.f ? 1.f / L : 0.f;
    }
    __syncthreads();
    for (int item = tid; item < G * D; item += kDecodeThreads) {
        const int j = item / D;
        const float* src = part_o + item;
        // four accumulators, chunk sp into accumulator sp % 4; eight chunks'
        // loads in flight together
        float ov0 = 0.f, ov1 = 0.f, ov2 = 0.f, ov3 = 0.f;
        int sp = 0;
        for (; sp + 8 <= n_splits; sp += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = src[(long long)(sp + u) * G * D];
            ov0 += s_w[sp * G + j] * x[0];
            ov1 += s_w[(sp + 1) * G + j] * x[1];
            ov2 += s_w[(sp + 2) * G + j] * x[2];
            ov3 += s_w[(sp + 3) * G + j] * x[3];
            ov0 += s_w[(sp + 4) * G + j] * x[4];
            ov1 += s_w[(sp + 5) * G + j] * x[5];
            ov2 += s_w[(sp + 6) * G + j] * x[6];
            ov3 += s_w[(sp + 7) * G + j] * x[7];
        }
        if (sp + 4 <= n_splits) {
            ov0 += s_w[sp * G + j] * src[(long long)sp * G * D];
            ov1 += s_w[(sp + 1) * G + j] * src[(long long)(sp + 1) * G * D];
            ov2 += s_w[(sp + 2) * G + j] * src[(long long)(sp + 2) * G * D];
            ov3 += s_w[(sp + 3) * G + j] * src[(long long)(sp + 3) * G * D];
            sp += 4;
        }
        for (; sp < n_splits; ++sp) ov0 += s_w[sp * G + j] * src[(long long)sp * G * D];
        const float ov = (ov0 + ov1) + (ov2 + ov3);
        a.out[(long long)b * a.ld_out + (long long)(kh * G) * D + item] = (uint16_t)f32_to_bf16(ov * s_inv_l[j]);
    }
}

}  // namespace

hipError_t launch_decode_merge(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t s,
                               Profiler* prof) {
    if (a.n_tokens <= 0 || plan.max_splits <= 1) return hipSuccess;
    const float* ws = static_cast<const float*>(workspace);
    const dim3 grid(a.n_kv_heads, a.n_tokens), block(kDecodeThreads);
    const int pps = plan.pages_per_split, ms = plan.max_splits;
    if (prof) prof->begin(DAP_KERNEL_DECODE_MERGE, s);
    switch (a.head_dim) {
        case 64: hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, s, a, pps, ms, ws); break;
        case 96: hipLaunchKernelGGL(decode_merge_kernel<96>, grid, block, 0, s, a, pps, ms, ws); break;
        case 128: hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, s, a, pps, ms, ws); break;
        default: return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_DECODE_MERGE, s);
    return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t s,
                         Profiler* prof, const WriteArgs* fused) {
    if (a.n_tokens <= 0) return hipSuccess;
    float* ws = static_cast<float*>(workspace);
    dim3 grid((unsigned)plan.max_splits * a.n_kv_heads * a.n_tokens), block(kDecodeThreads);
    const size_t lds = (size_t)kDecodeWaves * a.head_dim * (a.n_q_heads / a.n_kv_heads) * sizeof(float);
    const int pps = plan.pages_per_split, ms = plan.max_splits;
#define DAP_DECODE_CASE(DD)                                                                             \
    case DD:                                                                                            \
        if (prof) prof->begin(DAP_KERNEL_DECODE, s);                                                    \
        if (fused)                                                                                      \
            hipLaunchKernelGGL((decode_kernel<DD, true>), grid, block, lds, s, a, pps, ms, ws, *fused);   \
        else                                                                                            \
            hipLaunchKernelGGL((decode_kernel<DD, false>), grid, block, lds, s, a, pps, ms, ws, WriteArgs{}); \
        if (prof) prof->end(DAP_KERNEL_DECODE, s);                                                      \
        break;
    switch (a.head_dim) {
        DAP_DECODE_CASE(64)
        DAP_DECODE_CASE(96)
        DAP_DECODE_CASE(128)
        default:
            return hipErrorInvalidValue;
    }
#undef DAP_DECODE_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(a, plan, workspace, s, prof);
}

}  // namespace dap
