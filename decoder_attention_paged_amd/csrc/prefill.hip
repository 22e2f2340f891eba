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
// Per 64-key page the workgroup stages K (key-major) and V^T (dim-major)
// into one of two LDS buffers (one barrier per page), and each
// wave computes S^T = K Q^T and O^T += V^T P^T with 32x32x16 bf16 MFMAs and
// an online softmax in float32 (exp2 with the scale folded in; a row's
// reference max, and with it O, moves only when a score passes it by more
// than 2^8, so the weights stay at most 256). Pages fully
// outside a wave's rows are skipped; only pages that straddle a row's causal
// or window edge are masked element by element. Workgroups are numbered
// kv-head-fastest so blocks sharing a kv head land on the same XCD (L2).
#include "dap_internal.h"

namespace dap {

namespace {

// waves per prefill workgroup at head_dim D
__host__ __device__ constexpr int prefill_waves(int D) { return D >= 128 ? 8 : 4; }
constexpr int kTilesThreads = 1024;
constexpr int kSortTiles = 4096;       // tiles ordered longest first by the tile pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.f;        // log2 of the largest softmax weight before a rescale
constexpr unsigned kErrSegments = 32u;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// ---------------------------------------------------------------- tile list
// tiles[k] = first token of tile k (k < n_tiles), tiles[n_tiles] = end of the
// last tile, tiles[cap + 1] = n_tiles (at most cap tiles are kept), then
// tiles[cap + 2 + i] = the tile the i-th workgroup group takes.
// A tile starts where (t - start of t's run) is a multiple of bm (a power of
// two). Thread i owns a contiguous chunk of the tokens; each chunk is read
// once, eight loads in flight, and its run starts kept in a bit mask (chunks
// above 64 tokens, past 65536 tokens in a call, read the segments again).

// exclusive max-scan (identity -1) and inclusive sum-scan over the block:
// within each wave by shuffles, then one exchange of the wave totals
__device__ __forceinline__ int block_excl_max(int v, int* s_w) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x = max(x, y);
    }
    if (lane == 63) s_w[wv] = x;
    __syncthreads();
    int pre = -1;
    for (int w = 0; w < wv; ++w) pre = max(pre, s_w[w]);
    int ex = __shfl_up(x, 1);
    if (lane == 0) ex = -1;
    __syncthreads();
    return max(ex, pre);
}
__device__ __forceinline__ int block_incl_sum(int v, int* s_w, int& total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_w[wv] = x;
    __syncthreads();
    int pre = 0;
    total = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        if (w < wv) pre += s_w[w];
        total += s_w[w];
    }
    __syncthreads();
    return x + pre;
}

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

    // run starts of my chunk; the last one
    unsigned long long flags = 0ull;
    int my_start = -1;
    for (int b = c0; b < c1; b += 8) {
        int v[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            const int t = b - 1 + i;
            v[i] = t >= 0 && t < c1 ? seg[t] : 0;
        }
#pragma unroll
        for (int i = 1; i < 9; ++i) {
            const int t = b - 1 + i;
            if (t < c1 && (t == 0 || v[i] != v[i - 1])) {
                my_start = t;
                if (masked) flags |= 1ull << (t - c0);
            }
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

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// Key (within a 32-key S block) held in A-row i: bits 2 and 3 of i swapped,
// so that in the 32x32 output layout lane group g's registers 8h..8h+7 are
// the 8 contiguous keys 16h + 8g .. 16h + 8g + 7 the PV step needs.
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int G>
__global__ __launch_bounds__(64 * prefill_waves(D), 8 / prefill_waves(D))
void prefill_kernel(AttnArgs a, const int* __restrict__ tiles, int cap) {
    constexpr int kPrefillThreads = 64 * prefill_waves(D);
    constexpr int BM = 32 * prefill_waves(D) / G;   // tokens per tile
    constexpr int KS = D + 8;           // LDS row stride of K (elements)
    constexpr int VS = kPage + 8;       // LDS row stride of V^T (elements)
    constexpr int kSteps = D / 16;      // QK k-steps
    constexpr int kDimBlocks = D / 32;  // PV output blocks
    constexpr int kTileChunks = 8 * D;  // 16-byte chunks per tensor per page
    constexpr int kChunks = (kTileChunks + kPrefillThreads - 1) / kPrefillThreads;
    constexpr int kBufElems = kPage * KS + D * VS;

    // two page buffers (K then V^T in each), written and read alternately
    extern __shared__ __attribute__((aligned(16))) uint16_t s_buf[];

    const int n_tiles = tiles[cap + 1];
    const int kh = blockIdx.x % a.n_kv_heads;
    const int slot = blockIdx.x / a.n_kv_heads;
    if (slot >= n_tiles) return;
    const int tile = tiles[cap + 2 + slot];          // longest tiles first
    const int t0 = tiles[tile];
    const int t1 = min(tiles[tile + 1], t0 + BM);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int row = lane & 31;
    const int half = lane >> 5;
    const int hq = kh * G + (wave % G);
    const int tok = t0 + 32 * (wave / G) + row;
    const bool row_valid = tok < t1;

    // table row of the tile (all its tokens share the segment)
    const int trow = a.rows[t0];
    if (trow < 0 || trow >= a.n_table_rows) {
        if (tid == 0 && kh == 0) atomicOr(a.err, kErrRow);
        return;
    }

    // per-row attended range [lo, p]
    int p = -1, lo = 1 << 30;
    if (row_valid) {
        p = a.positions[tok];
        if (p < 0 || p >= a.max_position) {
            if (kh == 0) atomicOr(a.err, kErrPosition);
            p = -1;
        } else {
            lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
        }
    }
    // workgroup-wide key range over every token of the tile
    int kmin = 1 << 30, kmax = -1;
    for (int t = t0 + lane; t < t1; t += 64) {
        const int pp = a.positions[t];
        if (pp >= 0 && pp < a.max_position) {
            kmax = max(kmax, pp);
            kmin = min(kmin, a.window > 0 ? max(0, pp - a.window + 1) : 0);
        }
    }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (kmax < 0) return;                        // uniform: no valid token
    if ((kmax >> 6) >= a.table_ld) {
        if (tid == 0 && kh == 0) atomicOr(a.err, kErrTable);
        return;
    }
    // this wave's rows
    const int w_pmax = wave_max(p);
    const int w_lomin = wave_min(lo);
    const int w_pmin = wave_min(row_valid && p >= 0 ? p : (1 << 30));
    const int w_lomax = wave_max(row_valid && p >= 0 ? lo : -1);

    // Q^T as the B operand: column = query row, k-group = dims 16s + 8*half
    bf16x8 qf[kSteps];
    {
        const uint16_t* qr = a.q + (long long)(row_valid ? tok : t0) * a.ld_q + (long long)hq * D + 8 * half;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 u = *reinterpret_cast<const u32x4*>(qr + 16 * s);
            if (!row_valid || p < 0) u = u32x4{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(u);
        }
    }

    const float c = kLog2e / sqrtf((float)D);
    float m = -INFINITY;
    float lsum = 0.f;
    f32x16 o[kDimBlocks];
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    const int* tr = a.table + (long long)trow * a.table_ld;
    const int j_first = kmin >> 6;
    const int j_last = kmax >> 6;

    // The row's page ids, 64 at a time in one register (lane l holds the id
    // of page j_base + l), so the loop reads them with readlane instead of
    // waiting on a table load after every barrier. Pages are asked for in
    // increasing order; a new window is loaded every 64 pages.
    int j_base = j_first;
    int ids = j_base + lane <= j_last ? tr[j_base + lane] : -1;
    auto page_id = [&](int j) -> int {
        if (j - j_base >= 64) {                        // uniform
            j_base += 64;
            ids = j_base + lane <= j_last ? tr[j_base + lane] : -1;
        }
        return __builtin_amdgcn_readlane(ids, j - j_base);
    };

    u32x4 pk[kChunks], pv[kChunks];
    auto prefetch = [&](int j) -> bool {
        const int pg = page_id(j);
        if (pg < 0 || pg >= a.n_pages) return false;
        const uint16_t* kt = a.k_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);
        const uint16_t* vt = a.v_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int cidx = tid + kPrefillThreads * i;
            if (kTileChunks % kPrefillThreads == 0 || cidx < kTileChunks) {
                pk[i] = *reinterpret_cast<const u32x4*>(kt + 8 * cidx);
                pv[i] = *reinterpret_cast<const u32x4*>(vt + 8 * cidx);
            }
        }
        return true;
    };
    auto stage = [&](int buf) {
        uint16_t* sk = s_buf + buf * kBufElems;
        uint16_t* sv = sk + kPage * KS;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int cidx = tid + kPrefillThreads * i;
            if (kTileChunks % kPrefillThreads == 0 || cidx < kTileChunks) {
                int key, d0, d, key0;                 // the chunk's place in the tile layout
                k_tile_chunk(cidx, D, key, d0);
                *reinterpret_cast<u32x4*>(&sk[key * KS + d0]) = pk[i];
                v_tile_chunk(cidx, D, d, key0);
                *reinterpret_cast<u32x4*>(&sv[d * VS + key0]) = pv[i];
            }
        }
    };

    // Pipeline: page j computes from LDS buffer (j - j_first) & 1 while page
    // j+1's tile, prefetched into registers during page j-1, is written to
    // the other buffer; one barrier per page.
    bool ok_next = prefetch(j_first);
    if (ok_next) stage(0);
    bool ok_cur = ok_next;
    __syncthreads();
    if (j_first < j_last) ok_next = prefetch(j_first + 1);

    for (int j = j_first; j <= j_last; ++j) {
        const int buf = (j - j_first) & 1;
        const uint16_t* s_k = s_buf + buf * kBufElems;
        const uint16_t* s_v = s_k + kPage * KS;
        const int k0 = j * kPage;
        if (!ok_cur && tid == 0 && kh == 0) atomicOr(a.err, kErrPage);
        if (ok_cur && !(k0 > w_pmax || k0 + kPage - 1 < w_lomin)) {   // skip pages invisible to this wave
        // S^T = K Q^T : two 32-key blocks. All K fragments are read from LDS
        // first (they return in order, so the MFMAs then issue back to back);
        // the scheduling barrier keeps the compiler from pairing each read
        // with its MFMA, which would expose the LDS latency every time.
        u32x4 kf[2][kSteps];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint16_t* kr = &s_k[(32 * blk + swap23(row)) * KS + 8 * half];
#pragma unroll
            for (int s = 0; s < kSteps; ++s) kf[blk][s] = *reinterpret_cast<const u32x4*>(kr + 16 * s);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[blk][s]), qf[s], acc, 0, 0, 0);
            sc[blk] = acc;                     // unscaled; the scale folds into the exp2 argument
        }
        // V^T fragments for the PV step, read now so their latency hides
        // under the softmax below
        u32x4 vfr[4][kDimBlocks];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                vfr[t][db] = *reinterpret_cast<const u32x4*>(&s_v[(32 * db + row) * VS + 16 * t + 8 * half]);
        __builtin_amdgcn_sched_barrier(0);
        // mask where this page crosses an edge of some row's range
        if (k0 < w_lomax || k0 + kPage - 1 > w_pmin) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q4 = r >> 2;
                    const int kp = k0 + 32 * blk + 16 * (q4 >> 1) + 8 * half + 4 * (q4 & 1) + (r & 3);
                    if (kp < lo || kp > p) sc[blk][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[blk][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // Reference max in scaled log2 units: it moves to a row's new max only
        // when a score exceeds it by more than 2^kLazyMax (any visible key
        // sets an unset one), so the weights stay at most 2^kLazyMax and O and
        // l are rescaled on a row's first pages only.
        const float ms = mx * c;
        const bool move = ms > m + kLazyMax;
        if (__any(move)) {
            const float alpha = move ? __builtin_amdgcn_exp2f(m - ms) : 1.f;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) o[db] *= alpha;
            if (move) m = ms;
        }
        const float m_ref = m == -INFINITY ? 0.f : m;     // a row with nothing visible yet
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sc[blk][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], c, -m_ref));

        // O^T += V^T P^T : four 16-key steps. The row sum adds the bf16
        // weights the MFMAs use, two per dot2 (the normaliser is then the sum
        // of exactly the weights applied to V).
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sc[t >> 1][8 * (t & 1) + e];
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfr[t][db]), pf, o[db], 0, 0, 0);
            ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), kOnes2, ps0, false);
            ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), kOnes2, ps1, false);
            ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), kOnes2, ps0, false);
            ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), kOnes2, ps1, false);
        }
        lsum += ps0 + ps1;
        }
        // next page into the other buffer (its previous contents were last read
        // before the previous barrier), then one barrier
        if (j < j_last && ok_next) stage(buf ^ 1);
        ok_cur = ok_next;
        __syncthreads();
        if (j + 1 < j_last) ok_next = prefetch(j + 2);
    }

    lsum += __shfl_xor(lsum, 32);
    if (!row_valid || p < 0) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t* dst = a.out + (long long)tok * a.ld_out + (long long)hq * D;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t w0 = f32_to_bf16(o[db][4 * q4 + 0] * inv) | (f32_to_bf16(o[db][4 * q4 + 1] * inv) << 16);
            uint32_t w1 = f32_to_bf16(o[db][4 * q4 + 2] * inv) | (f32_to_bf16(o[db][4 * q4 + 3] * inv) << 16);
            *reinterpret_cast<uint2*>(dst + 32 * db + 8 * q4 + 4 * half) = make_uint2(w0, w1);
        }
}

template <int D, int G>
hipError_t launch_prefill_dg(const AttnArgs& a, int cap, const int* tiles, hipStream_t s) {
    constexpr size_t lds = 2 * (kPage * (D + 8) + D * (kPage + 8)) * sizeof(uint16_t);
    static bool configured = false;     // raise the dynamic LDS limit once per instantiation
    if (!configured) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, G>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        configured = true;
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
