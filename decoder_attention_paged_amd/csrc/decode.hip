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
// contiguous block per kv head (K slot-major, V dim-major), and every lane
// reads 16 contiguous bytes per load.
//
// Merge: a row whose range fits one chunk is finished by that workgroup.
// Otherwise each chunk stores its fp32 (m, l, o) per head in the workspace
// and bumps a per-(row, kv head) counter; the last chunk to arrive merges all
// chunks with the max-shifted rescale (exactly the single-pass softmax in
// real arithmetic), rounds to bf16 and resets the counter to zero, so one
// launch does the whole decode and the counters stay zeroed between calls.
#include "dap_internal.h"

namespace dap {

namespace {

constexpr int kDecodeThreads = 256;   // 4 waves
constexpr int kDecodeWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Key (within a 64-key page) held in row i of the S block blk. Chosen so the
// four lanes groups' S values line up with contiguous 8-key runs of the V^T
// rows in the PV step (group g, step t holds keys 16g + 8t .. 16g + 8t + 7).
__device__ __forceinline__ int decode_key(int blk, int i) {
    return 16 * (i >> 2) + 8 * (blk >> 1) + 4 * (blk & 1) + (i & 3);
}

struct RowRange {
    int ok;
    int row;        // table row
    int p, lo;      // attended positions [lo, p]
    int first_pg;   // table index of lo's page
    int n_pg;       // pages in [lo, p]
};

__device__ __forceinline__ RowRange row_range(const AttnArgs& a, int b, bool flag) {
    RowRange r;
    r.ok = 0;
    r.p = a.positions[b];
    r.row = a.rows ? a.rows[b] : b;
    if (r.p < 0 || r.p >= a.max_position) {
        if (flag) atomicOr(a.err, kErrPosition);
        return r;
    }
    if (r.row < 0 || r.row >= a.n_table_rows) {
        if (flag) atomicOr(a.err, kErrRow);
        return r;
    }
    if ((r.p >> 6) >= a.table_ld) {
        if (flag) atomicOr(a.err, kErrTable);
        return r;
    }
    r.lo = a.window > 0 ? max(0, r.p - a.window + 1) : 0;
    r.first_pg = r.lo >> 6;
    r.n_pg = (r.p >> 6) - r.first_pg + 1;
    r.ok = 1;
    return r;
}

template <int D>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(AttnArgs a, int pps, int max_splits,
                                                                   float* __restrict__ ws, int* ws_counters) {
    constexpr int kSteps = D / 32;     // QK k-steps of 32 dims
    constexpr int kDimBlocks = D / 16; // PV output blocks of 16 dims

    __shared__ float s_m[kDecodeWaves][16];
    __shared__ float s_l[kDecodeWaves][16];
    __shared__ float s_o[kDecodeWaves][D][17];

    const int split = blockIdx.x;
    const int kh = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;         // MFMA column: query head within the group
    const int grp = lane >> 4;         // lane group 0..3

    const RowRange rr = row_range(a, b, split == 0 && kh == 0 && tid == 0);
    if (!rr.ok) return;
    const int n_splits = (rr.n_pg + pps - 1) / pps;
    if (split >= n_splits) return;
    const int j0 = rr.first_pg + split * pps;
    const int j1 = min(j0 + pps, rr.first_pg + rr.n_pg);
    const int G = a.n_q_heads / a.n_kv_heads;

    // q^T as the B operand: column = head, rows = dims 32s + 8*grp .. +7.
    bf16x8 qf[kSteps];
    {
        const bool real = col < G;
        const uint16_t* qrow = a.q + (long long)b * a.ld_q + (long long)(kh * G + (real ? col : 0)) * D;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 u = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp);
            if (!real) u = u32x4{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(u);
        }
    }

    const float c = kLog2e / sqrtf((float)D);
    float m = -INFINITY;
    float lsum = 0.f;
    f32x4 o[kDimBlocks];
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int* trow = a.table + (long long)rr.row * a.table_ld;
    for (int jj = j0 + wave; jj < j1; jj += kDecodeWaves) {
        const int pg = trow[jj];
        if (pg < 0 || pg >= a.n_pages) {
            atomicOr(a.err, kErrPage);
            continue;
        }
        const uint16_t* kt = a.k_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);
        const uint16_t* vt = a.v_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);

        u32x4 kf[4][kSteps];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const uint16_t* kr = kt + decode_key(blk, col) * D + 8 * grp;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) kf[blk][s] = *reinterpret_cast<const u32x4*>(kr + 32 * s);
        }
        u32x4 vf[2][kDimBlocks];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                vf[t][db] = *reinterpret_cast<const u32x4*>(vt + (16 * db + col) * kPage + 16 * grp + 8 * t);
        }

        // S = K q^T, 16 keys per block
        f32x4 sc[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[blk][s]), qf[s], acc, 0, 0, 0);
            sc[blk] = acc * c;
        }
        // mask the window's lower edge and the tail past p
        const int base = jj * kPage;
        if (base < rr.lo || base + kPage - 1 > rr.p) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kp = base + decode_key(blk, 4 * grp + r);
                    if (kp < rr.lo || kp > rr.p) sc[blk][r] = -INFINITY;
                }
        }
        float mx = sc[0][0];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[blk][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);        // finite: every page holds a visible key
        const float alpha = exp2f(m - m_new);
        float ps = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = exp2f(sc[blk][r] - m_new);
                sc[blk][r] = e;
                ps += e;
            }
        lsum = lsum * alpha + ps;
        m = m_new;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db) o[db] *= alpha;

        // O^T += V^T P^T, 32 keys per step
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8 pf;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pf[r] = (__bf16)sc[2 * t][r];
                pf[4 + r] = (__bf16)sc[2 * t + 1][r];
            }
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[t][db]), pf, o[db], 0, 0, 0);
        }
    }

    // combine the four lane groups' partial sums (same column = same head)
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (grp == 0) {
        s_m[wave][col] = m;
        s_l[wave][col] = lsum;
    }
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[wave][16 * db + 4 * grp + r][col] = o[db][r];
    __syncthreads();

    // merge the waves: this chunk's (m, l, o) for each real head
    const long long pair = (long long)b * a.n_kv_heads + kh;
    float* part = ws + pair * G * (long long)max_splits * (D + 2);   // [G][max_splits][D + 2]
    for (int item = tid; item < G * D; item += kDecodeThreads) {
        const int j = item / D;
        const int d = item % D;
        float M = s_m[0][j];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][j]);
        float ov = 0.f, lv = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float sw = exp2f(s_m[w][j] - M);
                ov += sw * s_o[w][d][j];
                lv += sw * s_l[w][j];
            }
        }
        if (n_splits == 1) {               // the whole row in one chunk: finish here
            a.out[(long long)b * a.ld_out + (long long)(kh * G + j) * D + d] =
                (uint16_t)f32_to_bf16(lv > 0.f ? ov / lv : 0.f);
            continue;
        }
        float* dst = part + ((long long)j * max_splits + split) * (D + 2);
        dst[d] = ov;
        if (d == 0) {
            dst[D] = M;
            dst[D + 1] = lv;
        }
    }
    if (n_splits == 1) return;

    // The last chunk to finish for this (row, kv head) merges all chunks:
    // M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
    __shared__ int s_last;
    __threadfence();                       // publish this chunk's partial device-wide
    __syncthreads();
    int* counter = reinterpret_cast<int*>(ws_counters) + pair;
    if (tid == 0) s_last = atomicAdd(counter, 1) == n_splits - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();                       // see every other chunk's partial
    if (tid == 0) *counter = 0;            // leave the counter zeroed for the next call
    for (int item = tid; item < G * D; item += kDecodeThreads) {
        const int j = item / D;
        const int d = item % D;
        const float* src = part + (long long)j * max_splits * (D + 2);
        float M = -INFINITY;
        for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, __builtin_nontemporal_load(src + sp * (D + 2) + D));
        float ov = 0.f, lv = 0.f;
        if (M != -INFINITY) {
            for (int sp = 0; sp < n_splits; ++sp) {
                const float* e = src + sp * (D + 2);
                const float w = exp2f(__builtin_nontemporal_load(e + D) - M);
                ov += w * __builtin_nontemporal_load(e + d);
                lv += w * __builtin_nontemporal_load(e + D + 1);
            }
        }
        a.out[(long long)b * a.ld_out + (long long)(kh * G + j) * D + d] =
            (uint16_t)f32_to_bf16(lv > 0.f ? ov / lv : 0.f);
    }
}

}  // namespace

DecodePlan decode_plan(int n_rows, int n_q_heads, int n_kv_heads, int head_dim, int window,
                       int max_position) {
    DecodePlan p;
    const int span = window > 0 ? min(window, max_position) : max_position;
    const int max_pages = (span + kPage - 1) / kPage + (window > 0 ? 1 : 0);
    const long long pairs = (long long)n_rows * n_kv_heads;
    // aim at ~8K workgroups in total (about half active for uniformly spread
    // lengths), at least one page per wave
    long long pps = (pairs * max_pages + 8191) / 8192;
    pps = (pps + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
    if (pps < kDecodeWaves) pps = kDecodeWaves;
    p.pages_per_split = (int)pps;
    p.max_splits = (int)((max_pages + pps - 1) / pps);
    // one counter per (row, kv head) for the largest row count a call may
    // have, at a fixed place: calls with different row counts share a
    // workspace without their partials ever landing on counters
    p.counter_bytes = ((size_t)kMaxDecodeRows * n_kv_heads * sizeof(int) + 255) / 256 * 256;
    p.workspace_bytes = p.counter_bytes + (size_t)n_rows * n_q_heads * p.max_splits * (head_dim + 2) * sizeof(float);
    return p;
}

hipError_t launch_decode(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t s,
                         Profiler* prof) {
    if (a.n_tokens <= 0) return hipSuccess;
    int* counters = static_cast<int*>(workspace);
    float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes);
    dim3 grid(plan.max_splits, a.n_kv_heads, a.n_tokens), block(kDecodeThreads);
    if (prof) prof->begin(DAP_KERNEL_DECODE, s);
    switch (a.head_dim) {
        case 64:
            hipLaunchKernelGGL(decode_kernel<64>, grid, block, 0, s, a, plan.pages_per_split, plan.max_splits, ws, counters);
            break;
        case 96:
            hipLaunchKernelGGL(decode_kernel<96>, grid, block, 0, s, a, plan.pages_per_split, plan.max_splits, ws, counters);
            break;
        case 128:
            hipLaunchKernelGGL(decode_kernel<128>, grid, block, 0, s, a, plan.pages_per_split, plan.max_splits, ws, counters);
            break;
        default:
            return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_DECODE, s);
    return hipGetLastError();
}

}  // namespace dap
