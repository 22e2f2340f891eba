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

// One workgroup: per-segment first and last positions (LDS atomics), page
// counts, an exclusive scan for each segment's first scratch page, then the
// table and every token's scratch slot.
__global__ __launch_bounds__(kInpassThreads) void inpass_prep_kernel(InpassPrep p) {
    __shared__ int s_lo[kMaxInpassSegments];
    __shared__ int s_hi[kMaxInpassSegments];
    __shared__ int s_first[kMaxInpassSegments];
    __shared__ int s_part[kInpassThreads];
    const int tid = threadIdx.x;
    const int ns = p.n_segments;
    for (int s = tid; s < ns; s += kInpassThreads) {
        s_lo[s] = 0x7fffffff;
        s_hi[s] = -1;
    }
    __syncthreads();
    // A wave whose tokens all lie in one segment (the usual case: segments
    // are runs of the pack) reduces their positions by shuffles and makes
    // one update; otherwise each lane updates its own segment. Four rounds'
    // tokens are loaded before any is used, to keep loads in flight.
    constexpr int kRounds = 4;
    const int lane = tid & 63;
    for (int tb = tid - lane; tb < p.n_tokens; tb += kRounds * kInpassThreads) {
        int sgs[kRounds], poss[kRounds];
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const int t = tb + k * kInpassThreads + lane;
            sgs[k] = t < p.n_tokens ? p.segments[t] : -1;
            poss[k] = t < p.n_tokens ? p.positions[t] : 0;
        }
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const int t = tb + k * kInpassThreads + lane;
            const bool valid = t < p.n_tokens;
            const int sg = sgs[k], pos = poss[k];
            if (tb + k * kInpassThreads >= p.n_tokens) break;     // uniform: no token left in this round
            const int s0 = __builtin_amdgcn_readfirstlane(sg);  // lane 0 holds a token
            if (__ballot(valid && sg != s0) == 0 && s0 >= 0 && s0 < ns) {   // uniform
                int lo = valid ? pos : 0x7fffffff, hi = valid ? pos : -1;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    lo = min(lo, __shfl_xor(lo, o));
                    hi = max(hi, __shfl_xor(hi, o));
                }
                if (lane == 0) {
                    atomicMin(&s_lo[s0], lo);
                    atomicMax(&s_hi[s0], hi);
                }
                continue;
            }
            if (!valid) continue;
            if (sg < 0 || sg >= ns) {
                atomicOr(p.err, kErrRow);
                continue;
            }
            atomicMin(&s_lo[sg], pos);
            atomicMax(&s_hi[sg], pos);
        }
    }
    __syncthreads();
    // pages per segment, exclusive scan (each thread owns a run of segments)
    constexpr int kPer = kMaxInpassSegments / kInpassThreads;
    int cnt[kPer];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int s = tid * kPer + k;
        cnt[k] = (s < ns && s_hi[s] >= 0) ? (s_hi[s] - s_lo[s]) / kPage + 1 : 0;
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
        if (s < ns) s_first[s] = run;
        run += cnt[k];
    }
    __syncthreads();
    // table rows: page j of segment s, if it exists and fits
    const long long n_table = (long long)ns * p.table_ld;
    for (long long i = tid; i < n_table; i += kInpassThreads) {
        const int s = (int)(i / p.table_ld), j = (int)(i % p.table_ld);
        const int pages = s_hi[s] >= 0 ? (s_hi[s] - s_lo[s]) / kPage + 1 : 0;
        const int pg = s_first[s] + j;
        p.table[i] = (j < pages && pg < p.capacity) ? pg : -1;
    }
    for (int tb = tid; tb < p.n_tokens; tb += kRounds * kInpassThreads) {
        int sgs[kRounds], poss[kRounds];
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const int t = tb + k * kInpassThreads;
            sgs[k] = t < p.n_tokens ? p.segments[t] : -1;
            poss[k] = t < p.n_tokens ? p.positions[t] : 0;
        }
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const int t = tb + k * kInpassThreads;
            if (t >= p.n_tokens) break;
            const int sg = sgs[k];
            if (sg < 0 || sg >= ns) {
                p.slots[t] = -1;
                p.rel_positions[t] = 0;
                continue;
            }
            const int rel = poss[k] - s_lo[sg];
            const int j = rel / kPage;
            const int pg = s_first[sg] + j;
            const bool fits = j < p.table_ld && pg < p.capacity;
            if (!fits) atomicOr(p.err, kErrSpan);
            p.slots[t] = fits ? pg * kPage + rel % kPage : -1;
            p.rel_positions[t] = rel;
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
    if (prof) prof->begin(DAP_KERNEL_PREP, s);
    hipLaunchKernelGGL(inpass_prep_kernel, dim3(1), dim3(kInpassThreads), 0, s, p);
    if (prof) prof->end(DAP_KERNEL_PREP, s);
    return hipGetLastError();
}

}  // namespace dap
