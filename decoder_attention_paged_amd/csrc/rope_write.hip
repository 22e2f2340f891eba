// Fused per-head QK-RMSNorm + rotary positions + page write.
//
// One wave per token for q and k: the token's D/2 rotation angles p*f[i]
// and their sine/cosine are computed once in float64 into LDS, then every q
// and k head of the token is normed (optionally), rotated and rounded to
// bf16 once. In the same launch, after the token workgroups, one workgroup
// per (64 tokens, kv head) copies v into the V tiles through an LDS
// transpose, so the consecutive slots of one dim are written as contiguous
// runs (the tile layout keeps 8 consecutive keys of a dim together). Page tiles are in the library's
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
#include "rope_head.h"

namespace dap {

namespace {

constexpr int kWriteThreads = 256;

constexpr int kVTile = 64;         // tokens per V-transpose workgroup

// V of kVTile consecutive tokens, per kv head: rows read coalesced, turned
// around in LDS, and stored along tokens. The tile layout keeps 8 consecutive
// keys of a dim in one 16-byte chunk, so 8 tokens of the tile whose slots are
// one aligned run of 8 (the usual case: a prompt's tokens fill their pages in
// order) are stored as one chunk; any other group is stored element by element.
template <int D>
__device__ __forceinline__ void write_v_tile(const WriteArgs& a, int t0, int kh) {
    // LDS: dim d's 64 tokens in 8 groups of 8, group g stored at position
    // g ^ ((d >> 3) & 7): the transpose writes (16 lanes, one token, 16 dims)
    // spread over 8 banks and every group stays one aligned 16-byte chunk
    __shared__ __attribute__((aligned(16))) uint16_t s_v[D * kVTile];
    __shared__ long long s_slot[kVTile];
    __shared__ int s_run[kVTile / 8];  // group g's 8 slots form one aligned run
    auto at = [](int d, int tt) { return d * kVTile + 8 * ((tt >> 3) ^ ((d >> 3) & 7)) + (tt & 7); };
    const int tid = threadIdx.x;
    const int n = min(kVTile, a.n_tokens - t0);
    if (tid < kVTile) s_slot[tid] = tid < n ? token_slot(a, t0 + tid, a.positions[t0 + tid], false) : -1;
    for (int c = tid; c < n * (D / 8); c += kWriteThreads) {
        const int tt = c / (D / 8), d8 = c % (D / 8);
        const u32x4 x = *reinterpret_cast<const u32x4*>(a.v + (long long)(t0 + tt) * a.ld_in +
                                                        (long long)kh * D + 8 * d8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            s_v[at(8 * d8 + 2 * w, tt)] = (uint16_t)(x[w] & 0xffffu);
            s_v[at(8 * d8 + 2 * w + 1, tt)] = (uint16_t)(x[w] >> 16);
        }
    }
    __syncthreads();
    if (tid < kVTile / 8) {
        const long long s0 = s_slot[8 * tid];
        bool run = s0 >= 0 && (s0 & 7) == 0;
#pragma unroll
        for (int i = 1; i < 8; ++i) run = run && s_slot[8 * tid + i] == s0 + i;
        s_run[tid] = run;
    }
    __syncthreads();
    // one item per (dim, group of 8 tokens)
    for (int e = tid; e < D * (kVTile / 8); e += kWriteThreads) {
        const int d = e / (kVTile / 8), g = e % (kVTile / 8);
        if (s_run[g]) {
            const long long slot = s_slot[8 * g];
            const u32x4 x = *reinterpret_cast<const u32x4*>(&s_v[at(d, 8 * g)]);
            *reinterpret_cast<u32x4*>(a.v_pool + ((slot >> 6) * a.n_kv_heads + kh) * (long long)(D * kPage) +
                                      v_tile_offset((int)(slot & (kPage - 1)), d, D)) = x;
            continue;
        }
        for (int i = 0; i < 8; ++i) {
            const int tt = 8 * g + i;
            const long long slot = s_slot[tt];
            if (tt >= n || slot < 0) continue;
            a.v_pool[((slot >> 6) * a.n_kv_heads + kh) * (long long)(D * kPage) +
                     v_tile_offset((int)(slot & (kPage - 1)), d, D)] = s_v[at(d, tt)];
        }
    }
}

// raw rows of item `item` (8 lanes per head) of token t, zeros past the heads
template <int D>
__device__ __forceinline__ void load_item(const WriteArgs& a, int t, int item, int n_rope_heads, u32x4& lo,
                                          u32x4& hi, int& head, int& j, bool& active) {
    head = item / kLanesPerHead;
    j = item % kLanesPerHead;
    active = head < n_rope_heads && j < D / 16;
    lo = u32x4{0u, 0u, 0u, 0u};
    hi = lo;
    if (active) {
        const uint16_t* src = head < a.n_q_heads ? a.q + (long long)t * a.ld_in + (long long)head * D
                                                 : a.k + (long long)t * a.ld_in + (long long)(head - a.n_q_heads) * D;
        lo = *reinterpret_cast<const u32x4*>(src + 8 * j);
        hi = *reinterpret_cast<const u32x4*>(src + D / 2 + 8 * j);
    }
}

// Many tokens: one wave per token, four tokens per workgroup. Items (8
// lanes per head) are software-pipelined two deep: the rows of item i+1 are
// loaded before item i is rotated and stored (q_out may alias q, so the
// compiler would not move a later load above an earlier store by itself),
// and the first item's rows are loaded before the sin/cos.
template <int D>
__global__ __launch_bounds__(kWriteThreads) void rope_write_kernel(WriteArgs a) {
    static_assert(D % 16 == 0 && D / 16 <= kLanesPerHead, "head_dim");
    constexpr int kHalf = D / 2;
    constexpr int kTokens = kWriteThreads / 64;   // one wave per token
    // the token workgroups come first, so their latency-bound chains start
    // before the V workgroups fill the machine
    const int n_tb = (a.n_tokens + kTokens - 1) / kTokens;
    if ((int)blockIdx.x >= n_tb) {                   // uniform per workgroup
        const int vb = (int)blockIdx.x - n_tb;
        write_v_tile<D>(a, (vb / a.n_kv_heads) * kVTile, vb % a.n_kv_heads);
        return;
    }

    __shared__ double s_cos[kTokens][kHalf];
    __shared__ double s_sin[kTokens][kHalf];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = (int)blockIdx.x * kTokens + wave;
    const bool have = t < a.n_tokens;                // uniform per wave
    const int p = have ? a.positions[t] : 0;
    const bool pos_ok = have && p >= 0 && p < a.max_position;
    const int n_rope_heads = a.n_q_heads + a.n_kv_heads;
    const int n_iter = (n_rope_heads * kLanesPerHead + 63) / 64;

    u32x4 lo0, hi0, lo1, hi1;
    int head0, j0, head1, j1;
    bool act0, act1;
    if (pos_ok) load_item<D>(a, t, lane, n_rope_heads, lo0, hi0, head0, j0, act0);

    long long slot = -1;
    if (have && lane == 0) slot = token_slot(a, t, p, true);
    slot = __shfl(slot, 0);
    angle_table<D>(a.inv_freq, p, lane, 64, s_cos[wave], s_sin[wave]);
    __syncthreads();
    if (!pos_ok) return;                             // uniform per wave; no barrier follows

    for (int it = 0; it < n_iter; it += 2) {         // uniform trip count: shuffles stay wave-wide
        const bool two = it + 1 < n_iter;
        if (two) load_item<D>(a, t, (it + 1) * 64 + lane, n_rope_heads, lo1, hi1, head1, j1, act1);
        rope_item<D>(a, t, head0, j0, act0, lo0, hi0, s_cos[wave], s_sin[wave], slot);
        if (it + 2 < n_iter) load_item<D>(a, t, (it + 2) * 64 + lane, n_rope_heads, lo0, hi0, head0, j0, act0);
        if (two) rope_item<D>(a, t, head1, j1, act1, lo1, hi1, s_cos[wave], s_sin[wave], slot);
    }
    // V is written by the tile workgroups
}

// Few tokens: one workgroup (4 waves) per token, so a token's heads run in
// parallel; the first two items of every thread are loaded before the
// sin/cos, so the row loads overlap them. Held to 128 VGPRs (four
// workgroups per CU): 2176 tokens 34 -> 32 us against the 134 it would use.
template <int D>
__global__ __launch_bounds__(kWriteThreads, 4) void rope_write_token_kernel(WriteArgs a) {
    const int n_vb = (a.n_tokens + kVTile - 1) / kVTile * a.n_kv_heads;
    // V tiles first: dispatched last they ran as the kernel's tail (2176
    // tokens of 8 kv heads: 32.0 -> 30.1 us)
    if ((int)blockIdx.x < n_vb) {                    // uniform per workgroup
        const int vb = (int)blockIdx.x;
        write_v_tile<D>(a, (vb / a.n_kv_heads) * kVTile, vb % a.n_kv_heads);
        return;
    }
    constexpr int kHalf = D / 2;
    constexpr int kBatch = 2;
    __shared__ double s_cos[kHalf];
    __shared__ double s_sin[kHalf];
    __shared__ long long s_slot;

    const int tid = threadIdx.x;
    const int t = (int)blockIdx.x - n_vb;
    const int p = a.positions[t];
    if (p < 0 || p >= a.max_position) {                       // uniform per workgroup
        if (tid == 0) atomicOr(a.err, kErrPosition);
        return;
    }
    const int n_rope_heads = a.n_q_heads + a.n_kv_heads;
    const int n_iter = (n_rope_heads * kLanesPerHead + kWriteThreads - 1) / kWriteThreads;
    long long slot = -1;
    for (int it0 = 0; it0 < n_iter; it0 += kBatch) {
        u32x4 lo[kBatch], hi[kBatch];
        int head[kBatch], j[kBatch];
        bool active[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            load_item<D>(a, t, (it0 + b) * kWriteThreads + tid, n_rope_heads, lo[b], hi[b], head[b], j[b],
                         active[b]);
        if (it0 == 0) {                                       // uniform: the angle table, once
            // the slot lookup (two dependent loads) in the last wave, the
            // angle table in the first
            if (tid == kWriteThreads - 64) s_slot = token_slot(a, t, p, true);
            angle_table<D>(a.inv_freq, p, tid, kWriteThreads, s_cos, s_sin);
            __syncthreads();
            slot = s_slot;
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (it0 + b < n_iter)                            // uniform
                rope_item<D>(a, t, head[b], j[b], active[b], lo[b], hi[b], s_cos, s_sin, slot);
    }
}

}  // namespace

// Below kWideTokens tokens the one-workgroup-per-token form fills the chip
// better; above it, one wave per token.
constexpr int kWideTokens = 4096;

hipError_t launch_write(const WriteArgs& a, hipStream_t s, Profiler* prof) {
    if (a.n_tokens <= 0) return hipSuccess;
    const int n_vtiles = (a.n_tokens + kVTile - 1) / kVTile;
    const bool per_token = a.n_tokens < kWideTokens;
    const int n_token_blocks = per_token ? a.n_tokens : (a.n_tokens + kWriteThreads / 64 - 1) / (kWriteThreads / 64);
    dim3 grid(n_vtiles * a.n_kv_heads + n_token_blocks), block(kWriteThreads);
    if (prof) prof->begin(DAP_KERNEL_WRITE, s);
#define DAP_WRITE_CASE(DD)                                                                                       \
    case DD:                                                                                                    \
        if (per_token) hipLaunchKernelGGL(rope_write_token_kernel<DD>, grid, block, 0, s, a);                   \
        else hipLaunchKernelGGL(rope_write_kernel<DD>, grid, block, 0, s, a);                                   \
        break;
    switch (a.head_dim) {
        DAP_WRITE_CASE(64)
        DAP_WRITE_CASE(96)
        DAP_WRITE_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef DAP_WRITE_CASE
    if (prof) prof->end(DAP_KERNEL_WRITE, s);
    return hipGetLastError();
}

}  // namespace dap
