// One pass over pages for packed prompts and decode rows together: the
// packed prefill's tiles and the decode's page chunks in one launch.
//
// Sources: "Mistral 7B Instruct v0.3", Entries (step_paged: prefill_paged
// and decode_paged in one pass); "Phi-3 Mini 4K Instruct" files,
// src/attention.linnet (step_packed: every token written first, then the
// prompts attend and each row's step attends over its row).
//
// The tokens are written beforehand (their keys must be in the pool before
// any query reads them). Every workgroup has four waves and less than half
// of a CU's LDS, so two run on each CU; the decode's chunks are dispatched
// first and the prefill tiles after them (step_order.h), so the tiles run in
// the CUs the decode's last round leaves idle. There is no tile-list launch:
// each prefill workgroup finds its own tile with one scan of the segment
// ids. The decode's cross-chunk merge follows as its own launch.
#include <atomic>

#include "decode_chunk.h"
#include "prefill_tile.h"
#include "step_order.h"

namespace dap {

namespace {

constexpr int kStepThreads = 256;                  // four waves per workgroup
constexpr int kStepWaves = kStepThreads / 64;
static_assert(kStepThreads == dec::kDecodeThreads, "a decode chunk takes one workgroup");

// LDS page buffers of a prefill tile here (a page is D/4 KB): 64 KB at 128,
// 72 KB at 96 and 64 KB at 64, so two workgroups fit on a CU
__host__ __device__ constexpr int step_buffers(int D) { return D == 128 ? 2 : (D == 96 ? 3 : 4); }
__host__ __device__ constexpr int step_tile_tokens(int G) { return 32 * kStepWaves / G; }

// Tile k of the prompt tokens [0, n): the runs of equal segment ids, each cut
// into bm-token tiles from its first token (bm a power of two), numbered in
// token order. The whole workgroup takes part: thread i reads a contiguous
// piece of the ids, the pieces' run starts and tile counts are scanned
// across the block, the thread holding tile k's first token publishes it,
// and the tile ends at bm tokens, the run's end or n. Returns false when
// there is no tile k; flags kErrSegments (slot 0, kv head 0) when the tiles
// outnumber the workgroup slots.
__device__ bool find_tile(const int32_t* __restrict__ seg, int n, int bm, int k, int cap, bool flag, unsigned* err,
                          int& t0, int& t1) {
    __shared__ int s_w[kStepThreads / 64];
    __shared__ int s_t0, s_t1;
    const int tid = threadIdx.x;
    const int chunk = (n + kStepThreads - 1) / kStepThreads;
    const int c0 = min(n, tid * chunk), c1 = min(n, c0 + chunk);
    int prev = c0 > 0 ? seg[c0 - 1] : 0;
    int last_start = -1;
    for (int t = c0; t < c1; ++t) {
        const int sg = seg[t];
        if (t == 0 || sg != prev) last_start = t;
        prev = sg;
    }
    const int rs = pf::block_excl_max(last_start, s_w);     // the run my piece begins in
    int r = rs, cnt = 0;
    prev = c0 > 0 ? seg[c0 - 1] : 0;
    for (int t = c0; t < c1; ++t) {
        const int sg = seg[t];
        if (t == 0 || sg != prev) r = t;
        prev = sg;
        cnt += ((t - r) & (bm - 1)) == 0;
    }
    int total;
    const int first = pf::block_incl_sum(cnt, s_w, total) - cnt;
    if (tid == 0) {
        s_t0 = -1;
        s_t1 = n;
        if (flag && total > cap) atomicOr(err, kErrSegments);
    }
    __syncthreads();
    if (k >= first && k < first + cnt) {
        r = rs;
        int idx = first;
        prev = c0 > 0 ? seg[c0 - 1] : 0;
        for (int t = c0; t < c1; ++t) {
            const int sg = seg[t];
            if (t == 0 || sg != prev) r = t;
            prev = sg;
            if (((t - r) & (bm - 1)) == 0) {
                if (idx == k) s_t0 = t;
                ++idx;
            }
        }
    }
    __syncthreads();
    t0 = s_t0;
    if (t0 < 0) return false;
    // the first token after t0 in another run, if any, within the tile's span
    const int t = t0 + 1 + tid;
    if (tid < bm - 1 && t < n && seg[t] != seg[t0]) atomicMin(&s_t1, t);
    __syncthreads();
    t1 = min(s_t1, min(t0 + bm, n));
    return true;
}

template <int D, int G>
__global__ __launch_bounds__(kStepThreads, 2) void step_kernel(AttnArgs pre, int cap, AttnArgs dec, int pps,
                                                               int max_splits, float* __restrict__ ws) {
    // page buffers of a prefill tile, or the decode's per-wave O
    extern __shared__ __attribute__((aligned(1024))) u32x4 s_dyn[];
    const unsigned n_pre = (unsigned)cap * pre.n_kv_heads;
    const unsigned n_dec = (unsigned)max_splits * dec.n_kv_heads * dec.n_tokens;
    const StepRole role = step_role(blockIdx.x, n_pre, n_dec);
    if (role.prefill) {
        if (role.id >= n_pre) return;
        // kv head fastest, as in the prefill kernel
        const int kh = role.id % pre.n_kv_heads;
        const int slot = role.id / pre.n_kv_heads;
        int t0, t1;
        if (!find_tile(pre.rows, pre.n_tokens, step_tile_tokens(G), slot, cap, role.id == 0, pre.err, t0, t1))
            return;
        pf::prefill_tile<D, G, kStepWaves, step_buffers(D)>(pre, t0, t1, kh, s_dyn);
        return;
    }
    if (role.id >= n_dec) return;
    dec::decode_chunk<D, false>(dec, pps, max_splits, ws, WriteArgs{}, role.id, reinterpret_cast<float*>(s_dyn));
}

template <int D, int G>
hipError_t launch_step_dg(const AttnArgs& pre, int cap, const AttnArgs& dec, const DecodePlan& plan, float* ws,
                          hipStream_t s) {
    constexpr size_t pre_lds = (size_t)step_buffers(D) * (D / 4) * 1024;
    constexpr size_t dec_lds = (size_t)kDecodeWaves * D * G * sizeof(float);
    constexpr size_t lds = pre_lds > dec_lds ? pre_lds : dec_lds;
    // the dynamic LDS limit is raised once per device (bit d: device d)
    static std::atomic<unsigned long long> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&step_kernel<D, G>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_release);
    }
    const unsigned blocks = step_blocks((unsigned)cap * pre.n_kv_heads,
                                        (unsigned)plan.max_splits * dec.n_kv_heads * dec.n_tokens);
    hipLaunchKernelGGL((step_kernel<D, G>), dim3(blocks), dim3(kStepThreads), lds, s, pre, cap, dec,
                       plan.pages_per_split, plan.max_splits, ws);
    return hipGetLastError();
}

template <int D>
hipError_t launch_step_d(const AttnArgs& pre, int cap, const AttnArgs& dec, const DecodePlan& plan, float* ws,
                         hipStream_t s) {
    switch (pre.n_q_heads / pre.n_kv_heads) {
        case 1: return launch_step_dg<D, 1>(pre, cap, dec, plan, ws, s);
        case 2: return launch_step_dg<D, 2>(pre, cap, dec, plan, ws, s);
        case 4: return launch_step_dg<D, 4>(pre, cap, dec, plan, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int step_tile_cap(int n_prompt, int n_segments, int group) {
    const int bm = step_tile_tokens(group);
    return (n_prompt + bm - 1) / bm + n_segments;
}

hipError_t launch_step(const AttnArgs& pre, int n_segments, const AttnArgs& dec, const DecodePlan& plan,
                       void* workspace, hipStream_t s, Profiler* prof) {
    if (pre.n_tokens <= 0 || dec.n_tokens <= 0) return hipErrorInvalidValue;
    const int cap = step_tile_cap(pre.n_tokens, n_segments, pre.n_q_heads / pre.n_kv_heads);
    float* ws = static_cast<float*>(workspace);
    hipError_t e;
    if (prof) prof->begin(DAP_KERNEL_STEP, s);
    switch (pre.head_dim) {
        case 64: e = launch_step_d<64>(pre, cap, dec, plan, ws, s); break;
        case 96: e = launch_step_d<96>(pre, cap, dec, plan, ws, s); break;
        case 128: e = launch_step_d<128>(pre, cap, dec, plan, ws, s); break;
        default: return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_STEP, s);
    if (e != hipSuccess) return e;
    return launch_decode_merge(dec, plan, workspace, s, prof);
}

}  // namespace dap
