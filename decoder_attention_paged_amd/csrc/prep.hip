// Index preparation for the contiguous-cache and in-pass entries.
//
// Sources: "Phi-3 Mini 4K Instruct" files, src/attention.linnet: `decode`
// (one position for every row of the cache), `prefill` (a span of positions
// from `pos`), `decode_rows` (each row at its own position), `prefill_slots`
// (prompts from position 0 into chosen cache rows), `forward` and `packed`
// (attention among the pass's own tokens, no cache written: same segment,
// key position at or before the query's, within the window).
//
// A contiguous cache of R rows and MaxSeq positions is a page pool whose row
// r owns pages r*P .. r*P + P - 1 (P = MaxSeq / 64): the identity table. The
// in-pass entries put each segment's keys into scratch pages, from the
// segment's first position on, so that the paged prefill over those pages
// with positions counted from that first position sees exactly the pass's
// own tokens of the segment (the mask only depends on position differences;
// rope has already used the absolute positions).
#include "dap_internal.h"

namespace dap {

namespace {

constexpr int kLayoutThreads = 256;
constexpr int kInpassThreads = 1024;

__global__ __launch_bounds__(kLayoutThreads) void layout_prep_kernel(LayoutPrep p) {
    const long long n_table = p.table ? (long long)p.table_rows * p.table_ld : 0;
    const long long n = n_table > p.n_tokens ? n_table : p.n_tokens;
    for (long long i = blockIdx.x * (long long)kLayoutThreads + threadIdx.x; i < n;
         i += (long long)gridDim.x * kLayoutThreads) {
        if (i < p.n_tokens) {
            const int t = (int)i;
            const int grp = t / p.per_group, k = t % p.per_group;
            switch (p.mode) {
                case kLayoutConstPos:
                    p.positions[t] = p.base_pos;
                    p.rows[t] = t;
                    break;
                case kLayoutSpan:
                    p.positions[t] = p.base_pos + k;
                    p.rows[t] = grp;
                    break;
                case kLayoutSlots:
                    p.positions[t] = k;
                    p.rows[t] = p.row_map[grp];
                    break;
                default:
                    p.rows[t] = t;
                    break;
            }
        }
        if (i < n_table) p.table[i] = (int32_t)i;      // row r, entry j -> page r * table_ld + j
    }
}

// In-pass preparation, four launches: (1) each segment's bounds set to
// empty, (2) every segment's first and last positions by global atomics
// from many workgroups (one update per wave whose tokens share a segment,
// the usual case since segments are runs of the pack), (3) one workgroup
// turns the bounds into page counts and an exclusive scan, each segment's
// first scratch page, (4) every token's scratch slot and relative position
// and every table entry.
constexpr int kInpassRounds = 4;                                   // tokens per thread in the bounds pass
constexpr int kBoundsThreads = 256;
constexpr int kBoundsTokens = kBoundsThreads * kInpassRounds;     // tokens per bounds workgroup

__global__ __launch_bounds__(kLayoutThreads) void inpass_init_kernel(InpassPrep p) {
    const int s = blockIdx.x * kLayoutThreads + threadIdx.x;
    if (s < p.n_segments) {
        p.seg_lo[s] = 0x7fffffff;
        p.seg_hi[s] = -1;
    }
}

__global__ __launch_bounds__(kBoundsThreads) void inpass_bounds_kernel(InpassPrep p) {
    const int lane = threadIdx.x & 63;
    const int ns = p.n_segments;
    // a wave takes kInpassRounds groups of 64 consecutive tokens (group k at
    // base + 64 k); every group's tokens are loaded before any is used
    const int base = blockIdx.x * kBoundsTokens + (threadIdx.x - lane) * kInpassRounds;
    int sgs[kInpassRounds], poss[kInpassRounds];
#pragma unroll
    for (int k = 0; k < kInpassRounds; ++k) {
        const int t = base + 64 * k + lane;
        sgs[k] = t < p.n_tokens ? p.segments[t] : -1;
        poss[k] = t < p.n_tokens ? p.positions[t] : 0;
    }
#pragma unroll
    for (int k = 0; k < kInpassRounds; ++k) {
        const int t = base + 64 * k + lane;
        if (base + 64 * k >= p.n_tokens) break;               // uniform: this wave has no token at k
        const bool valid = t < p.n_tokens;
        const int sg = sgs[k], pos = poss[k];
        const int s0 = __builtin_amdgcn_readfirstlane(sg);    // lane 0 holds a token
        if (__ballot(valid && sg != s0) == 0 && s0 >= 0 && s0 < ns) {   // uniform
            int lo = valid ? pos : 0x7fffffff, hi = valid ? pos : -1;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                lo = min(lo, __shfl_xor(lo, o));
                hi = max(hi, __shfl_xor(hi, o));
            }
            if (lane == 0) {
                atomicMin(&p.seg_lo[s0], lo);
                atomicMax(&p.seg_hi[s0], hi);
            }
            continue;
        }
        if (!valid) continue;
        if (sg < 0 || sg >= ns) {
            atomicOr(p.err, kErrRow);
            continue;
        }
        atomicMin(&p.seg_lo[sg], pos);
        atomicMax(&p.seg_hi[sg], pos);
    }
}

// pages per segment and their exclusive scan: each segment's first scratch page
__global__ __launch_bounds__(kInpassThreads) void inpass_scan_kernel(InpassPrep p) {
    __shared__ int s_part[kInpassThreads];
    const int tid = threadIdx.x;
    const int ns = p.n_segments;
    constexpr int kPer = kMaxInpassSegments / kInpassThreads;      // each thread owns a run of segments
    int cnt[kPer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int s = tid * kPer + k;
        const int hi = s < ns ? p.seg_hi[s] : -1;
        cnt[k] = hi >= 0 ? (hi - p.seg_lo[s]) / kPage + 1 : 0;
        sum += cnt[k];
    }
    s_part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kInpassThreads; off <<= 1) {
        const int v = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    int run = s_part[tid] - sum;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int s = tid * kPer + k;
        if (s < ns) p.seg_first[s] = run;
        run += cnt[k];
    }
}

// every token's scratch slot and relative position, and every table entry
// (page j of segment s, if it exists and fits)
__global__ __launch_bounds__(kLayoutThreads) void inpass_slots_kernel(InpassPrep p) {
    const int ns = p.n_segments;
    const long long n_table = (long long)ns * p.table_ld;
    const long long n = n_table > p.n_tokens ? n_table : p.n_tokens;
    for (long long i = blockIdx.x * (long long)kLayoutThreads + threadIdx.x; i < n;
         i += (long long)gridDim.x * kLayoutThreads) {
        if (i < p.n_tokens) {
            const int t = (int)i;
            const int sg = p.segments[t];
            if (sg < 0 || sg >= ns) {
                p.slots[t] = -1;
                p.rel_positions[t] = 0;
            } else {
                const int rel = p.positions[t] - p.seg_lo[sg];
                const int j = rel / kPage;
                const int pg = p.seg_first[sg] + j;
                const bool fits = j < p.table_ld && pg < p.capacity;
                if (!fits) atomicOr(p.err, kErrSpan);
                p.slots[t] = fits ? pg * kPage + rel % kPage : -1;
                p.rel_positions[t] = rel;
            }
        }
        if (i < n_table) {
            const int s = (int)(i / p.table_ld), j = (int)(i % p.table_ld);
            const int hi = p.seg_hi[s];
            const int pages = hi >= 0 ? (hi - p.seg_lo[s]) / kPage + 1 : 0;
            const int pg = p.seg_first[s] + j;
            p.table[i] = (j < pages && pg < p.capacity) ? pg : -1;
        }
    }
}

}  // namespace

hipError_t launch_layout_prep(const LayoutPrep& p, hipStream_t s, Profiler* prof) {
    const long long n_table = p.table ? (long long)p.table_rows * p.table_ld : 0;
    const long long n = n_table > p.n_tokens ? n_table : p.n_tokens;
    if (n <= 0) return hipSuccess;
    const long long blocks = (n + kLayoutThreads - 1) / kLayoutThreads;
    if (prof) prof->begin(DAP_KERNEL_PREP, s);
    hipLaunchKernelGGL(layout_prep_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kLayoutThreads), 0, s,
                       p);
    if (prof) prof->end(DAP_KERNEL_PREP, s);
    return hipGetLastError();
}

hipError_t launch_inpass_prep(const InpassPrep& p, hipStream_t s, Profiler* prof) {
    if (p.n_tokens <= 0) return hipSuccess;
    if (p.n_segments <= 0 || p.n_segments > kMaxInpassSegments) return hipErrorInvalidValue;
    const long long n_table = (long long)p.n_segments * p.table_ld;
    const long long n = n_table > p.n_tokens ? n_table : p.n_tokens;
    const long long slot_blocks = (n + kLayoutThreads - 1) / kLayoutThreads;
    if (prof) prof->begin(DAP_KERNEL_PREP, s);
    hipLaunchKernelGGL(inpass_init_kernel, dim3((p.n_segments + kLayoutThreads - 1) / kLayoutThreads),
                       dim3(kLayoutThreads), 0, s, p);
    hipLaunchKernelGGL(inpass_bounds_kernel, dim3((p.n_tokens + kBoundsTokens - 1) / kBoundsTokens),
                       dim3(kBoundsThreads), 0, s, p);
    hipLaunchKernelGGL(inpass_scan_kernel, dim3(1), dim3(kInpassThreads), 0, s, p);
    hipLaunchKernelGGL(inpass_slots_kernel, dim3((unsigned)(slot_blocks < 4096 ? slot_blocks : 4096)),
                       dim3(kLayoutThreads), 0, s, p);
    if (prof) prof->end(DAP_KERNEL_PREP, s);
    return hipGetLastError();
}

}  // namespace dap
