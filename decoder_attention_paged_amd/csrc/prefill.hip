// Packed prefill over pages: flash-style MFMA attention.
//
// Sources: "Phi-3 Mini 4K Instruct" files, src/attention.linnet
// (prefill_packed: token i sees token j iff they share a segment and
// positions[j] <= positions[i] and positions[j] > positions[i] - WINDOW;
// scores scaled by rsqrt(head_dim)); "Mistral 7B Instruct v0.3", Entries
// (prefill_paged: each token attends over its row's pages up to its
// position, which covers chunks and shared prefixes).
//
// A tile-list pass cuts the packed tokens into runs of equal segment id and
// each run into tiles of at most 32*W/g tokens. One workgroup (W waves) takes
// one (tile, kv head): wave w owns 32 query rows = one of the g query heads
// sharing the kv head, for 32 of the tile's tokens, so each K/V page tile is
// read from memory once per workgroup for all g heads and 32*W query rows.
// W is 8 at head_dim 128 (one workgroup per CU, most rows per staged page)
// and 4 below, where the softmax outweighs the matrix work per key: two
// workgroups share a CU and, not tied by one barrier, overlap each other's
// MFMA and VALU phases, and shorter tiles waste less at the causal diagonal.
// Per 64-key page the workgroup loads K and V^T straight from the pool into
// one of 3-4 LDS buffers (buffer loads that write LDS, two or three pages
// ahead, no registers involved), laid out as the MFMA A-operand fragments in
// lane order so every fragment read is one contiguous kilobyte; one barrier
// per page. Each wave computes S^T = K Q^T and O^T += V^T P^T with 32x32x16
// bf16 MFMAs and
// an online softmax in float32 (exp2 with the scale folded in; a row's
// reference max, and with it O, moves only when a score passes it by more
// than 2^8, so the weights stay at most 256). Pages fully
// outside a wave's rows are skipped; only pages that straddle a row's causal
// or window edge are masked element by element. Workgroups are numbered
// kv-head-fastest so blocks sharing a kv head land on the same XCD (L2).
#include <atomic>

#include "prefill_tile.h"

namespace dap {

namespace {

using namespace pf;

constexpr int kTilesThreads = 1024;
constexpr int kSortTiles = 4096;       // tiles ordered longest first by the tile pass

// ---------------------------------------------------------------- tile list
// tiles[k] = first token of tile k (k < n_tiles), tiles[n_tiles] = end of the
// last tile, tiles[cap + 1] = n_tiles (at most cap tiles are kept), then
// tiles[cap + 2 + i] = the tile the i-th workgroup group takes.
// A tile starts where (t - start of t's run) is a multiple of bm (a power of
// two). Thread i owns a contiguous chunk of the tokens; each chunk is read
// once, eight loads in flight, and its run starts kept in a bit mask (chunks
// above 64 tokens, past 65536 tokens in a call, read the segments again).

__global__ __launch_bounds__(kTilesThreads) void prefill_tiles_kernel(const int32_t* __restrict__ seg,
                                                                      const int32_t* __restrict__ pos, int n,
                                                                      int bm, int cap, int window,
                                                                      int* __restrict__ tiles, unsigned* err) {
    __shared__ int s_w[kTilesThreads / 64];
    __shared__ int s_start[kSortTiles + 1];
    __shared__ int s_work[kSortTiles];
    __shared__ int s_idx[kSortTiles];
    const int tid = threadIdx.x;
    const int chunk = (n + kTilesThreads - 1) / kTilesThreads;
    const int c0 = min(n, tid * chunk);
    const int c1 = min(n, c0 + chunk);
    const bool masked = chunk <= 64;
    auto starts_run = [&](int t) { return t == 0 || seg[t] != seg[t - 1]; };

    // run starts of my chunk; the last one. Chunks of 8 ids or more whose
    // ids are 16-byte aligned are read with 16-byte loads, 8 ids at a time,
    // the id before each group carried from the group before; shorter ones
    // 8 (or fewer) single ids at a time.
    unsigned long long flags = 0ull;
    int my_start = -1;
    auto mark = [&](const int* v, int b) {
#pragma unroll
        for (int i = 1; i < 9; ++i) {
            const int t = b - 1 + i;
            if (t < c1 && (t == 0 || v[i] != v[i - 1])) {
                my_start = t;
                if (masked) flags |= 1ull << (t - c0);
            }
        }
    };
    auto load_scalar = [&](int* v, int b) {
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            const int t = b - 1 + i;
            v[i] = t >= 0 && t < c1 ? seg[t] : 0;
        }
    };
    if ((reinterpret_cast<uintptr_t>(seg) & 15) == 0 && (chunk & 3) == 0 && chunk >= 8) {
        int prev = 0;
#pragma unroll 4
        for (int b = c0; b < c1; b += 8) {
            int v[9];
            if (b + 8 <= c1) {
                v[0] = b > c0 ? prev : (b > 0 ? seg[b - 1] : 0);
                const int4 x = *reinterpret_cast<const int4*>(seg + b);
                const int4 y = *reinterpret_cast<const int4*>(seg + b + 4);
                v[1] = x.x; v[2] = x.y; v[3] = x.z; v[4] = x.w;
                v[5] = y.x; v[6] = y.y; v[7] = y.z; v[8] = y.w;
            } else {
                load_scalar(v, b);
            }
            mark(v, b);
            prev = v[8];
        }
    } else {
        for (int b = c0; b < c1; b += 8) {
            int v[9];
            load_scalar(v, b);
            mark(v, b);
        }
    }
    auto is_start = [&](int t) { return masked ? ((flags >> (t - c0)) & 1ull) != 0 : starts_run(t); };
    const int rs = block_excl_max(my_start, s_w);   // the run my chunk starts in

    // tile starts in my chunk, their count and place
    int cnt = 0;
    int r = rs;
    for (int t = c0; t < c1; ++t) {
        if (is_start(t)) r = t;
        if (((t - r) & (bm - 1)) == 0) ++cnt;
    }
    int total;
    int idx = block_incl_sum(cnt, s_w, total) - cnt;
    r = rs;
    for (int t = c0; t < c1; ++t) {
        if (is_start(t)) r = t;
        if (((t - r) & (bm - 1)) == 0) {
            // index cap holds the first dropped tile's start (the end of the last kept one)
            if (idx <= cap) tiles[idx] = t;
            if (idx < kSortTiles) s_start[idx] = t;
            ++idx;
        }
    }
    if (tid == 0) {
        if (total <= cap) tiles[total] = n;
        else atomicOr(err, kErrSegments);
        tiles[cap + 1] = min(total, cap);
    }

    // Dispatch order, longest first: tile k's work is the pages its tokens
    // attend (first token's window start to last token's position). A
    // bitonic sort orders the tiles by it (in one wave's registers up to 64
    // tiles, in LDS up to kSortTiles), so the workgroups with the most pages
    // start first and the short ones fill in behind them.
    const int n_tiles = min(total, cap);
    int* order = tiles + cap + 2;
    if (n_tiles > kSortTiles) {                       // too many to sort here: pack order
        for (int k = tid; k < n_tiles; k += kTilesThreads) order[k] = k;
        return;
    }
    if (tid == 0) s_start[n_tiles] = n;
    __syncthreads();
    auto work = [&](int k) {
        const int t0 = s_start[k];
        const int t1 = min(s_start[k + 1], t0 + bm);
        const int pf = pos[t0], pl = pos[t1 - 1];
        const int lo = window > 0 ? max(0, pf - window + 1) : 0;
        return max(0, (pl >> 6) - (lo >> 6) + 1);
    };
    if (n_tiles <= 64) {
        if (tid >= 64) return;
        int w = tid < n_tiles ? work(tid) : -1;       // padding sorts last
        int id = tid;
        for (int size = 2; size <= 64; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const int ow = __shfl_xor(w, stride);
                const int oid = __shfl_xor(id, stride);
                const bool lower = (tid & stride) == 0;
                const bool desc = (tid & size) == 0;   // the whole sequence ends descending
                // the lower lane of a pair keeps the larger work in a descending block
                const bool take = lower == desc ? ow > w : ow < w;
                if (take) {
                    w = ow;
                    id = oid;
                }
            }
        }
        if (tid < n_tiles) order[tid] = id;
        return;
    }
    int m2 = 1;
    while (m2 < n_tiles) m2 <<= 1;
    for (int k = tid; k < m2; k += kTilesThreads) {
        s_work[k] = k < n_tiles ? work(k) : -1;
        s_idx[k] = k;
    }
    __syncthreads();
    for (int size = 2; size <= m2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int k = tid; k < m2; k += kTilesThreads) {
                const int l = k ^ stride;
                if (l > k) {
                    const bool desc = (k & size) == 0;   // the whole sequence ends descending
                    const int wk = s_work[k], wl = s_work[l];
                    if (desc ? (wk < wl) : (wk > wl)) {
                        s_work[k] = wl;
                        s_work[l] = wk;
                        const int ik = s_idx[k];
                        s_idx[k] = s_idx[l];
                        s_idx[l] = ik;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int k = tid; k < n_tiles; k += kTilesThreads) order[k] = s_idx[k];
}

template <int D, int G>
__global__ __launch_bounds__(64 * prefill_waves(D), 8 / prefill_waves(D))
void prefill_kernel(AttnArgs a, const int* __restrict__ tiles, int cap) {
    constexpr int BM = 32 * prefill_waves(D) / G;   // tokens per tile
    // NB page buffers, each holding the page's K and V^T as MFMA A-operand
    // fragments of 1 KB in lane order (lane l's 16 bytes at 16*l)
    extern __shared__ __attribute__((aligned(1024))) u32x4 s_buf[];
    const int n_tiles = tiles[cap + 1];
    const int kh = blockIdx.x % a.n_kv_heads;
    const int slot = blockIdx.x / a.n_kv_heads;
    if (slot >= n_tiles) return;
    const int tile = tiles[cap + 2 + slot];          // longest tiles first
    const int t0 = tiles[tile];
    const int t1 = min(tiles[tile + 1], t0 + BM);
    prefill_tile<D, G, prefill_waves(D), prefill_buffers(D)>(a, t0, t1, kh, s_buf);
}

template <int D, int G>
hipError_t launch_prefill_dg(const AttnArgs& a, int cap, const int* tiles, hipStream_t s) {
    constexpr size_t lds = (size_t)prefill_buffers(D) * (D / 4) * 1024;
    // The dynamic LDS limit is raised once per device (the attribute is per
    // device); bit d of `configured` records device d. Devices past 63 set
    // it on every launch.
    static std::atomic<unsigned long long> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
    if (!(configured.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, G>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured.fetch_or(bit, std::memory_order_release);
    }
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3((unsigned)cap * a.n_kv_heads), dim3(64 * prefill_waves(D)), lds,
                       s, a, tiles, cap);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const AttnArgs& a, int G, int cap, const int* tiles, hipStream_t s) {
    switch (G) {
        case 1: return launch_prefill_dg<D, 1>(a, cap, tiles, s);
        case 2: return launch_prefill_dg<D, 2>(a, cap, tiles, s);
        case 4: return launch_prefill_dg<D, 4>(a, cap, tiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int tile_cap(int n_tokens, int n_segments, int group, int head_dim) {
    const int bm = 32 * prefill_waves(head_dim) / group;
    return (n_tokens + bm - 1) / bm + n_segments;
}

size_t prefill_workspace(int n_tokens, int n_segments, int group, int head_dim) {
    return (size_t)(2 * tile_cap(n_tokens, n_segments, group, head_dim) + 2) * sizeof(int);   // starts, count, order
}

hipError_t launch_prefill(const AttnArgs& a, int n_segments, void* workspace, hipStream_t s, Profiler* prof) {
    if (a.n_tokens <= 0) return hipSuccess;
    const int G = a.n_q_heads / a.n_kv_heads;
    const int cap = tile_cap(a.n_tokens, n_segments, G, a.head_dim);
    int* tiles = static_cast<int*>(workspace);
    if (prof) prof->begin(DAP_KERNEL_PREFILL_TILES, s);
    hipLaunchKernelGGL(prefill_tiles_kernel, dim3(1), dim3(kTilesThreads), 0, s, a.rows, a.positions, a.n_tokens,
                       32 * prefill_waves(a.head_dim) / G, cap, a.window, tiles, a.err);
    if (prof) prof->end(DAP_KERNEL_PREFILL_TILES, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (prof) prof->begin(DAP_KERNEL_PREFILL, s);
    switch (a.head_dim) {
        case 64: e = launch_prefill_d<64>(a, G, cap, tiles, s); break;
        case 96: e = launch_prefill_d<96>(a, G, cap, tiles, s); break;
        case 128: e = launch_prefill_d<128>(a, G, cap, tiles, s); break;
        default: return hipErrorInvalidValue;
    }
    if (prof) prof->end(DAP_KERNEL_PREFILL, s);
    return e;
}

}  // namespace dap
