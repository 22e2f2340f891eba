// The packed prefill's per-tile attention, as a device function shared by
// the prefill kernel and the fused step kernel: one workgroup of W waves
// takes the tokens [t0, t1) of one run of equal segment ids for one kv head.
// Wave w owns 32 query rows = one of the g query heads sharing the kv head,
// for 32 of the tile's tokens, so each K/V page tile is read from memory
// once per workgroup for all g heads and 32*W query rows. Per 64-key page
// the workgroup loads K and V^T straight from the pool into one of NB LDS
// buffers (buffer loads that write LDS, NB-1 pages ahead, no registers
// involved), laid out as the MFMA A-operand fragments in lane order so every
// fragment read is one contiguous kilobyte; one barrier per page. Each wave
// computes S^T = K Q^T and O^T += V^T P^T with 32x32x16 bf16 MFMAs and an
// online softmax in float32 (exp2 with the scale folded in; a row's
// reference max, and with it O, moves only when a score passes it by more
// than 2^8, so the weights stay at most 256). Pages fully outside a wave's
// rows are skipped; only pages that straddle a row's causal or window edge
// are masked element by element. With eight waves (one workgroup per CU)
// each wave's fragment reads run beside its MFMAs (page j's V^T fragments
// beside its score MFMAs, page j+1's K fragments beside the second half of
// its PV MFMAs), so no wave waits for a page's K fragments after the
// barrier, and half of each page's exps run beside the first half of its
// PV MFMAs.
//
// Sources: "Phi-3 Mini 4K Instruct" files, src/attention.linnet
// (prefill_packed: token i sees token j iff they share a segment and
// positions[j] <= positions[i] and positions[j] > positions[i] - WINDOW;
// scores scaled by rsqrt(head_dim)); "Mistral 7B Instruct v0.3", Entries
// (prefill_paged: each token attends over its row's pages up to its
// position, which covers chunks and shared prefixes).
#pragma once

#include "dap_internal.h"

namespace dap {
namespace pf {

// waves per prefill workgroup at head_dim D
__host__ __device__ constexpr int prefill_waves(int D) { return D >= 128 ? 8 : 4; }
// LDS page buffers per workgroup (a page is D/4 KB): 128 KB at 128 (one
// workgroup per CU), 72 KB at 96 and 64 KB at 64 (two per CU)
__host__ __device__ constexpr int prefill_buffers(int D) { return D == 96 ? 3 : 4; }
// last word of a raw buffer descriptor (32-bit data format, no swizzle)
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt operand: vmcnt(n), lgkmcnt(0), no wait on expcnt
__host__ __device__ constexpr unsigned waitcnt_vmcnt(int n) {
    return (unsigned)(n & 15) | ((unsigned)(n >> 4) << 14) | (7u << 4);
}
constexpr float kLazyMax = 8.f;        // log2 of the largest softmax weight before a rescale


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

// One 16-byte-per-lane buffer load straight into LDS: lane l's bytes land at
// lds + 16*l (the LDS address must be the same on every lane).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, u32x4* lds, int byte_offset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, byte_offset, 0, 0, 0);
}

// Key (within a 32-key S block) held in A-row i: bits 2 and 3 of i swapped,
// so that in the 32x32 output layout lane group g's registers 8h..8h+7 are
// the 8 contiguous keys 16h + 8g .. 16h + 8g + 7 the PV step needs.
__device__ __forceinline__ int swap23(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int G, int W, int NB>
__device__ __forceinline__ void prefill_tile(const AttnArgs& a, int t0, int t1, int kh, u32x4* s_buf) {
    constexpr int kSteps = D / 16;      // QK k-steps
    constexpr int kDimBlocks = D / 32;  // PV output blocks
    constexpr int kFragK = 2 * kSteps;            // K fragments per page: (32-key block, k-step)
    constexpr int kFrags = 2 * kFragK;            // and as many V^T fragments: (16-key step, dim block)
    constexpr int kFragPerWave = kFrags / W;      // 1 KB loads per wave per page
    constexpr int kBufBytes = kFrags * 1024;
    static_assert(4 * kDimBlocks == kFragK && kFrags % W == 0 && kFragK % kFragPerWave == 0, "fragment split");

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
    if (a.n_pages <= 0) {                        // no page to read (every id is out of range)
        if (tid == 0 && kh == 0) atomicOr(a.err, kErrPage);
        return;
    }
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
    kmin = __builtin_amdgcn_readfirstlane(wave_min(kmin));
    kmax = __builtin_amdgcn_readfirstlane(wave_max(kmax));
    if (kmax < 0) return;                        // uniform: no valid token
    if ((kmax >> 6) >= a.table_ld) {
        if (tid == 0 && kh == 0) atomicOr(a.err, kErrTable);
        return;
    }
    // this wave's rows (the same in every lane: scalar registers and branches)
    const int w_pmax = __builtin_amdgcn_readfirstlane(wave_max(p));
    const int w_lomin = __builtin_amdgcn_readfirstlane(wave_min(lo));
    const int w_pmin = __builtin_amdgcn_readfirstlane(wave_min(row_valid && p >= 0 ? p : (1 << 30)));
    const int w_lomax = __builtin_amdgcn_readfirstlane(wave_max(row_valid && p >= 0 ? lo : -1));

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

    const int j_first = kmin >> 6;
    const int j_last = kmax >> 6;

    // Page ids come by scalar loads (the table is read-only during the call):
    // they count on lgkmcnt, so waiting for one never waits for page loads
    // in flight. Each is loaded one page before its loads are issued.
    typedef const __attribute__((address_space(4))) int* ConstIntPtr;
    const ConstIntPtr trs = (ConstIntPtr)(a.table + (long long)__builtin_amdgcn_readfirstlane(trow) * a.table_ld);
    auto page_id = [&](int j) -> int { return trs[__builtin_amdgcn_readfirstlane(j)]; };

    // Each wave fills kFragPerWave of a page's fragments with 1 KB loads that
    // go straight into LDS (lane l fetches the 16 bytes the MFMA later reads
    // from lane l): waves 0 .. W/2-1 the K fragments, the others the V^T
    // ones. The byte offsets inside a (page, kv head) tile are fixed per lane.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool k_side = wv < W / 2;
    const int f0 = (wv % (W / 2)) * kFragPerWave;      // first fragment of this wave in its tensor
    int src_off[kFragPerWave];
#pragma unroll
    for (int i = 0; i < kFragPerWave; ++i) {
        const int f = f0 + i;
        src_off[i] = k_side ? 2 * k_tile_offset(32 * (f / kSteps) + swap23(row), 16 * (f % kSteps) + 8 * half, D)
                            : 2 * v_tile_offset(16 * (f / kDimBlocks) + 8 * half, 32 * (f % kDimBlocks) + row, D);
    }
    // Loads of page pg into buffer b, issued whatever the id (an invalid one
    // reads page 0 and is flagged), so every wave counts the same loads. They
    // are buffer loads (counted by vmcnt alone) through a descriptor bounded
    // to the (page, kv head) tile.
    auto issue = [&](int pg, int b) -> bool {
        pg = __builtin_amdgcn_readfirstlane(pg);
        b = __builtin_amdgcn_readfirstlane(b);
        const bool ok = pg >= 0 && pg < a.n_pages;
        const long long tile = ((long long)(ok ? pg : 0) * a.n_kv_heads + kh) * (kPage * D);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((k_side ? a.k_pool : a.v_pool) + tile), (short)0, kPage * D * 2, kBufferWord3);
        u32x4* dst = s_buf + b * (kBufBytes / 16) + (k_side ? 0 : 64 * kFragK) + 64 * f0;
#pragma unroll
        for (int i = 0; i < kFragPerWave; ++i)
            lds_load16(rs, dst + 64 * i, src_off[i]);
        return ok;
    };
    // Wait until at most `ahead` pages of this wave's loads are in flight and
    // its LDS reads are done (loads retire in order, so the older page has landed).
    auto wait_loads = [&](int ahead) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(63));   // lgkmcnt(0) on every path
        ahead = __builtin_amdgcn_readfirstlane(ahead);   // uniform: scalar branches
        if (NB > 3 && ahead >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(2 * kFragPerWave));
        else if (NB > 2 && ahead >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(kFragPerWave));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
    };

    typedef f32x16 Scores[2];
    typedef u32x4 VFrags[4][kDimBlocks];
    typedef u32x4 KFrags[2][kSteps];
    // K fragment (32-key block blk, k-step s) and V^T fragment (16-key step
    // t, dim block db) of the page whose buffer starts at fr (lane-offset)
    auto kfrag = [&](const u32x4* fr, int blk, int s) { return fr[64 * (blk * kSteps + s)]; };
    auto vfrag = [&](const u32x4* fr, int t, int db) { return fr[64 * (kFragK + t * kDimBlocks + db)]; };
    // S^T = K Q^T for one page: two 32-key blocks of kSteps MFMAs each,
    // unscaled (the scale folds into the exp2 argument); the two blocks'
    // accumulation chains alternate so consecutive MFMAs are independent
    auto scores = [&](const KFrags& kf, Scores& sc) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[blk][r] = 0.f;
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
                sc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[blk][s]), qf[s], sc[blk], 0, 0, 0);
    };
    // The masks of a page starting at key k0, then its softmax weights in
    // place of the scores.
    auto weights = [&](int k0, Scores& sc, VFrags& vfr, bool exps = true) __attribute__((always_inline)) {
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
        // Keys no row of this wave attends (outside [w_lomin, w_pmax]) may
        // hold anything an earlier request left (NaN and Inf included):
        // their V elements become 0, so their zero weights add exactly 0.
        // Lane (row, half) holds in V^T fragment t the keys 16 t + 8 half
        // .. + 7, two per dword.
        if (k0 < w_lomin || k0 + kPage - 1 > w_pmax) {
            // element e of fragment t is kept iff rl <= 16 t + e <= rh (the
            // empty asm keeps the comparisons from becoming loop invariants)
            int rl = w_lomin - k0 - 8 * half, rh = w_pmax - k0 - 8 * half;
            asm volatile("" : "+v"(rl), "+v"(rh));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 keep;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int e = 16 * t + 2 * w;
                    keep[w] = (e >= rl && e <= rh ? 0x0000ffffu : 0u) |
                              (e + 1 >= rl && e + 1 <= rh ? 0xffff0000u : 0u);
                }
#pragma unroll
                for (int db = 0; db < kDimBlocks; ++db) vfr[t][db] &= keep;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[blk][r]);
        {   // the other half-wave's max, by a VALU lane swap (no LDS round trip)
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
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
        if (!exps) return;
        const float m_ref = m == -INFINITY ? 0.f : m;     // a row with nothing visible yet
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sc[blk][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], c, -m_ref));
    };
    // bf16 weights of 16-key step t (the P^T operand) from the float ones
    auto pfrag = [&](const Scores& sc, int t) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sc[t >> 1][8 * (t & 1) + e];
        return pf;
    };
    // The row sum adds the bf16 weights the MFMAs use, two per dot2 (the
    // normaliser is then the sum of exactly the weights applied to V).
    auto add_sums = [&](const bf16x8& pf, float& ps0, float& ps1) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), kOnes2, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), kOnes2, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), kOnes2, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), kOnes2, ps1, false);
    };

    constexpr bool kStream = W == 8 && NB >= 4;   // the streamed form (see the page loop)

    // Streamed steps of one page (eight waves; see below).
    auto read_k = [&](const u32x4* frk, KFrags& kf) __attribute__((always_inline)) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int s = 0; s < kSteps; ++s) kf[blk][s] = kfrag(frk, blk, s);
    };
    auto read_v = [&](const u32x4* fr, VFrags& vfr) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) vfr[t][db] = vfrag(fr, t, db);
    };
    // score MFMAs, each followed by one V^T fragment read of the page (into
    // the registers the MFMAs free)
    auto score_stream = [&](const KFrags& kf, const u32x4* fr, Scores& sc, VFrags& vfr)
        __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        scores(kf, sc);
        read_v(fr, vfr);
#pragma unroll
        for (int i = 0; i < 2 * kSteps; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Streamed form: the softmax of a scored page and its PV MFMAs, split at
    // the page's two 32-key blocks so that half of the exps run beside
    // MFMAs: block 0's weights first, then its PV MFMAs, each with two of
    // block 1's exps beside it, then block 1's PV MFMAs, each with two K
    // fragment reads of the page to score next (from frk, in the order its
    // score MFMAs use them; the first half's V fragments are free by then).
    // One chunk per MFMA, kept in order by scheduling barriers. The weights,
    // sums and products are the same operations in the same order as
    // weights() followed by the four 16-key steps.
    auto soft_pv = [&](int k0, Scores& sc, VFrags& vfr, const u32x4* frk, KFrags& kf)
        __attribute__((always_inline)) {
        weights(k0, sc, vfr, false);                      // masks, row max, reference move
        const float nm = -(m == -INFINITY ? 0.f : m);
        bf16x8 pf[4];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pf[t][e] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][8 * t + e], c, nm));
            add_sums(pf[t], ps0, ps1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * kDimBlocks; ++i) {
            const int t = i / kDimBlocks, db = i % kDimBlocks;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfr[t][db]), pf[t], o[db], 0, 0, 0);
#pragma unroll
            for (int x = (16 * i) / (2 * kDimBlocks); x < (16 * (i + 1)) / (2 * kDimBlocks); ++x)
                pf[2 + x / 8][x % 8] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][x], c, nm));
            __builtin_amdgcn_sched_barrier(0);
        }
        add_sums(pf[2], ps0, ps1);
        add_sums(pf[3], ps0, ps1);
        lsum += ps0 + ps1;
#pragma unroll
        for (int i = 2 * kDimBlocks; i < 4 * kDimBlocks; ++i) {
            const int t = i / kDimBlocks, db = i % kDimBlocks;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfr[t][db]), pf[t], o[db], 0, 0, 0);
            const int r = i - 2 * kDimBlocks;
#pragma unroll
            for (int x = (2 * kSteps * r) / (2 * kDimBlocks); x < (2 * kSteps * (r + 1)) / (2 * kDimBlocks); ++x)
                kf[x & 1][x >> 1] = kfrag(frk, x & 1, x >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline over NB buffers: page j is read from buffer (j - j_first) %
    // NB; after the barrier that opens page j the loads of page j+NB-1
    // start, into the buffer of page j-1, which every wave has finished
    // with. One barrier per page.
    //
    // Streamed form (eight waves, one workgroup per CU): the fragment reads
    // are spread over the matrix work instead of every wave reading a page's
    // K fragments at once after the barrier while the matrix units wait. The
    // barrier before page j also certifies that page j+1 has landed (each
    // wave first waits for its own loads of both; loads then lead their use
    // by two pages). A wave reads the V^T fragments of page j while its
    // score MFMAs of page j run, and the K fragments of page j+1 while its PV
    // MFMAs of page j run, one read per MFMA into the registers the MFMAs
    // free.
    constexpr int kLead = NB - 1;
    unsigned okbits = 0;                 // bit k: page j+k has a valid id
    int b_issue = 0, b_cur = 0;
    for (int jj = j_first; jj <= j_last && jj < j_first + kLead; ++jj) {
        okbits |= (unsigned)issue(page_id(jj), b_issue) << (jj - j_first);
        b_issue = b_issue + 1 == NB ? 0 : b_issue + 1;
    }
    int pg_next = j_first + kLead <= j_last ? page_id(j_first + kLead) : -1;
    KFrags kf;                           // streamed form: K fragments of the page to score next

    for (int j = j_first; j <= j_last; ++j) {
        // in flight after the wait: the loads of pages past j (past j+1 when streamed)
        wait_loads(kStream ? max(0, min(kLead - 2, j_last - j - 1)) : min(kLead - 1, j_last - j));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (j + kLead <= j_last) {
            okbits |= (unsigned)issue(pg_next, b_issue) << kLead;
            b_issue = b_issue + 1 == NB ? 0 : b_issue + 1;
            if (j + kLead + 1 <= j_last) pg_next = page_id(j + kLead + 1);
        }
        const bool ok_cur = okbits & 1u;
        okbits >>= 1;
        const u32x4* fr = s_buf + b_cur * (kBufBytes / 16) + lane;
        b_cur = b_cur + 1 == NB ? 0 : b_cur + 1;
        const u32x4* fr_next = s_buf + b_cur * (kBufBytes / 16) + lane;   // page j+1
        const int k0 = j * kPage;
        if (!ok_cur && tid == 0 && kh == 0) atomicOr(a.err, kErrPage);
        // pages invisible to this wave's rows are skipped
        const bool vis = __builtin_amdgcn_readfirstlane(
            (int)(ok_cur && !(k0 > w_pmax || k0 + kPage - 1 < w_lomin)));

        if constexpr (kStream) {
            // After the last page the K reads still run (from a buffer no
            // load writes any more, values unused) so the fragments are
            // defined on every path round the loop.
            if (j == j_first) read_k(fr, kf);
            if (vis) {
                Scores scj;
                VFrags vfr;
                score_stream(kf, fr, scj, vfr);
                soft_pv(k0, scj, vfr, fr_next, kf);
            } else {
                read_k(fr_next, kf);
            }
        } else if (vis) {
            // All K fragments are read from LDS first (they return in order,
            // so the MFMAs then issue back to back); the scheduling barrier
            // keeps the compiler from pairing each read with its MFMA, which
            // would expose the LDS latency every time.
            read_k(fr, kf);
            __builtin_amdgcn_sched_barrier(0);
            Scores scj;
            scores(kf, scj);
            // V^T fragments for the PV step, read now so their latency
            // hides under the softmax below
            VFrags vfr;
            read_v(fr, vfr);
            __builtin_amdgcn_sched_barrier(0);
            weights(k0, scj, vfr);
            // O^T += V^T P^T : four 16-key steps (the split of soft_pv measured
            // 1 % slower here, with two four-wave workgroups per CU)
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 pf = pfrag(scj, t);
#pragma unroll
                for (int db = 0; db < kDimBlocks; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfr[t][db]), pf, o[db], 0, 0, 0);
                add_sums(pf, ps0, ps1);
            }
            lsum += ps0 + ps1;
        }
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


}  // namespace pf
}  // namespace dap
