// The decode's per-chunk work, as a device function shared by the decode
// kernel and the fused step kernel: one workgroup of four waves takes one
// (row, kv head, chunk of pages). Each wave walks every fourth 32-key unit
// (half page) of the chunk with its own running max / sum / weighted-V sum;
// the g query heads that share the kv head are the N columns of 16x16x32
// bf16 MFMAs, S[key][head] = K q^T and O^T[dim][head] += V^T P^T, so a
// page's K and V are read from HBM once for all g heads and the VALU only
// runs the softmax. A page tile is one contiguous block per kv head, stored
// in the order the waves load it, so every load of a wave reads one
// contiguous kilobyte. A row whose range fits one chunk is finished here;
// otherwise the chunk's float32 (m, l, o) per head goes to the workspace for
// the merge kernel.
//
// Sources: "Mistral 7B Instruct v0.3", Entries (decode_paged: decode_rows
// over pages, row b's positions in the pages table[b] lists); "Phi-3 Mini 4K
// Instruct" files, src/attention.linnet (decode_rows: the row's query sees
// positions j <= p and j > p - WINDOW; scores scaled by rsqrt(head_dim)).
#pragma once

#include "rope_head.h"

namespace dap {
namespace dec {

constexpr int kDecodeThreads = 64 * kDecodeWaves;


// A wave works on 32-key units (half pages): two 16-key S blocks and the
// V^T of the same 32 keys. The tile layout (dap_internal.h) stores each of
// the unit's K and V fragments as the 1 KB one load of the wave reads, lane
// by lane, with unit_key placing in lane group g's S values the 8 contiguous
// keys its V fragment covers. The loads are non-temporal: the tiles are read
// once per call, and contiguous kilobytes read that way stream fastest.

template <int D>
struct UnitFrags {
    u32x4 k[2][D / 32];   // K rows, two 16-key blocks
    u32x4 v[D / 16];      // V^T, 16 dims x 32 keys per block
};

template <int D>
__device__ __forceinline__ void load_unit(UnitFrags<D>& f, const uint16_t* kt, const uint16_t* vt, int half,
                                          int lane) {
    const u32x4* kb = reinterpret_cast<const u32x4*>(kt) + lane;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            f.k[blk][s] = __builtin_nontemporal_load(kb + ((half * 2 + blk) * (D / 32) + s) * 64);
    const u32x4* vb = reinterpret_cast<const u32x4*>(vt) + lane;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) f.v[db] = __builtin_nontemporal_load(vb + (half * (D / 16) + db) * 64);
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
struct WaveState {
    float m, lsum;
    f32x4 o[D / 16];
};

// One 32-key unit: S = K q^T, mask, online softmax, O^T += V^T P^T.
// Running max m is kept in scaled log2 units (scale folded into one FMA);
// O is rescaled only when some head's max moved in this unit.
// On a unit that crosses lo or p, a key outside [lo, p] gets weight 0 and
// its V elements are replaced by 0 before the PV product: such a slot may
// hold anything a row left there earlier (NaN and Inf included), and 0 * NaN
// would otherwise reach every head's sum. Lane group grp's V fragment holds
// the same 8 keys (8 grp .. 8 grp + 7 of the unit) as its weights.
// The normaliser adds the bf16 parts the PV product applies, two per dot2.
template <int D>
__device__ __forceinline__ void compute_unit(WaveState<D>& st, UnitFrags<D>& f, const bf16x8* qf, float c,
                                             int base, int lo, int p, int grp) {
    f32x4 sc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[blk][s]), qf[s], acc, 0, 0, 0);
        sc[blk] = acc;
    }
    if (base < lo || base + 31 > p) {
        // element e of the lane group's 8 keys is key base + 8 grp + e, in
        // [lo, p] iff rl <= e <= rh (the empty asm keeps the compiler from
        // turning each comparison into a loop-invariant register of its own);
        // S block blk's value r is element 4 blk + r, V dword w holds 2w, 2w+1
        int rl = lo - base - 8 * grp, rh = p - base - 8 * grp;
        asm volatile("" : "+v"(rl), "+v"(rh));
        bool in[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) in[e] = e >= rl && e <= rh;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (!in[4 * blk + r]) sc[blk][r] = -INFINITY;
        u32x4 keep;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            keep[w] = (in[2 * w] ? 0x0000ffffu : 0u) | (in[2 * w + 1] ? 0xffff0000u : 0u);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) f.v[db] &= keep;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx * c);  // finite: every unit computed holds a visible key
    if (__any(m_new > st.m)) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
        st.lsum *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) st.o[db] *= alpha;
        st.m = m_new;
    }
    // Each weight w goes to the PV product as two bf16 parts, hi = bf16(w)
    // and lo = bf16(w - hi), so the weights applied carry 16 significant
    // bits: the rounding no longer depends on the running max the chunk has
    // reached, and the result does not depend on how the row is split into
    // chunks beyond float32 rounding. (The decode is bound by its page
    // reads; the second set of PV MFMAs is nearly free.)
    bf16x8 pf, pl;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float w = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], c, -st.m));
            const __bf16 hi = (__bf16)w;
            pf[4 * blk + r] = hi;
            pl[4 * blk + r] = (__bf16)(w - (float)hi);
        }
    float ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), kOnes2, 0.f, false);
    float ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), kOnes2, 0.f, false);
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), kOnes2, ps0, false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), kOnes2, ps1, false);
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pl, pl, 0, 1), kOnes2, ps0, false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pl, pl, 2, 3), kOnes2, ps1, false);
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pl, pl, 4, 5), kOnes2, ps0, false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pl, pl, 6, 7), kOnes2, ps1, false);
    st.lsum += ps0 + ps1;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[db]), pf, st.o[db], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[db]), pl, st.o[db], 0, 0, 0);
}

// kFused: the rows' tokens are also written here (step_paged's decode
// tokens, one per row): every workgroup ropes (and norms) its g query heads
// from the raw projection w.q into LDS, and the workgroup holding the row's
// last page also writes the token's roped K, its V and q_out before any page
// load, so its own key is in the pool when it is read. Other workgroups of
// the row read only earlier pages.
template <int D, bool kFused>
__device__ __forceinline__ void decode_chunk(const AttnArgs& a, int pps, int max_splits, float* __restrict__ ws,
                                             const WriteArgs& w, unsigned bid, float* s_o) {
    constexpr int kSteps = D / 32;     // QK k-steps of 32 dims
    constexpr int kDimBlocks = D / 16; // PV output blocks of 16 dims

    __shared__ float s_m[kDecodeWaves][16];
    __shared__ float s_l[kDecodeWaves][16];
    __shared__ int s_pg[kMaxPagesPerSplit];
    __shared__ double s_cs[kFused ? D / 2 : 1], s_sn[kFused ? D / 2 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[kFused ? 16 * D : 8];
    __shared__ long long s_slot;
    // s_o: per-wave O for the cross-wave merge, [wave][dim][head] for the g
    // real heads only (4 * D * g floats of the caller's dynamic LDS)

    // Workgroup order: kv head fastest (consecutive workgroups go to
    // different XCDs, so each XCD gets the same share of every kv head),
    // then row, then chunk index. Chunks are counted from the end of the row:
    // chunk 0 is always a full chunk of pps pages and a row's partial chunk
    // has its highest index, so the dispatcher starts full chunks first and
    // the last workgroups it hands out are mostly partial ones.
    const int kh = bid % a.n_kv_heads;
    const int b = (bid / a.n_kv_heads) % a.n_tokens;
    const int split = bid / (a.n_kv_heads * a.n_tokens);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 15;         // MFMA column: query head within the group
    const int grp = lane >> 4;         // lane group 0..3

    // The decode-step form's inputs depend only on the row and kv head, so
    // their loads are issued before the row's range and page ids are known.
    const int G = a.n_q_heads / a.n_kv_heads;
    const long long tok = kFused ? (long long)b * w.ld_in : 0;
    const bool writer = split == 0;
    const int j = wave < 2 ? tid % kLanesPerHead : lane;
    const int hh = tid / kLanesPerHead;
    const bool act = kFused && (wave < 2 ? hh < G && j < D / 16 : (wave == 2 && writer && j < D / 16));
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
    if (act) {
        const uint16_t* src = wave < 2 ? w.q + tok + (long long)(kh * G + hh) * D : w.k + tok + (long long)kh * D;
        lo = *reinterpret_cast<const u32x4*>(src + 8 * j);
        hi = *reinterpret_cast<const u32x4*>(src + D / 2 + 8 * j);
    }
    constexpr int kVPerLane = (D + 63) / 64;
    uint16_t vv[kVPerLane];
    if (kFused && wave == 3 && writer)
#pragma unroll
        for (int i = 0; i < kVPerLane; ++i)
            vv[i] = 64 * i + lane < D ? w.v[tok + (long long)kh * D + 64 * i + lane] : 0;
    const double freq = kFused && tid < D / 2 ? w.inv_freq[tid] : 0.0;

    const RowRange rr = row_range(a, b, split == 0 && kh == 0 && tid == 0);
    if (!rr.ok) return;
    const int n_splits = (rr.n_pg + pps - 1) / pps;
    if (split >= n_splits) return;
    const int j_hi = rr.first_pg + rr.n_pg - 1 - split * pps;      // last page of this chunk
    const int j0 = max(rr.first_pg, j_hi - pps + 1);
    const int n_local = j_hi - j0 + 1;

    // this chunk's page ids, once, into LDS (-1 marks an out-of-range id)
    const int* trow = a.table + (long long)rr.row * a.table_ld;
    for (int i = tid; i < n_local; i += kDecodeThreads) {
        const int pg = trow[j0 + i];
        const bool ok = pg >= 0 && pg < a.n_pages;
        if (!ok) atomicOr(a.err, kErrPage);
        s_pg[i] = ok ? pg : -1;
    }

    // units u = 2*page + half of this chunk; wave w takes u = w, w+4, ...
    // A unit is skipped if it lies past the chunk, its page id was bad, or
    // none of its keys is in [lo, p]. The next unit's fragments load while
    // the current one computes; the load is issued even for a skipped unit
    // (from the pool's first tile, always in bounds) so that the number of
    // loads in flight is the same on every path and the wait before the
    // compute covers only the current unit.
    const int n_units = 2 * n_local;
    auto prep = [&](int u, int& base, const uint16_t*& kt, const uint16_t*& vt, int& half) -> bool {
        kt = a.k_pool;
        vt = a.v_pool;
        half = 0;
        if (u >= n_units) return false;
        const int pg = __builtin_amdgcn_readfirstlane(s_pg[u >> 1]);   // the same for the whole wave
        base = (j0 + (u >> 1)) * kPage + 32 * (u & 1);
        if (pg < 0 || base > rr.p || base + 31 < rr.lo) return false;
        kt = a.k_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);
        vt = a.v_pool + ((long long)pg * a.n_kv_heads + kh) * (kPage * D);
        half = u & 1;
        return true;
    };
    UnitFrags<D> fa, fb;
    int base_a = 0, base_b = 0, half = 0;
    const uint16_t *kt = a.k_pool, *vt = a.v_pool;
    int u = wave;
    bool ok_a = false;
    // The fused prologue issues the first unit's load before its rope work
    // when that unit cannot hold the token's page (any workgroup but the
    // writer, or a writer whose chunk has more than two pages).
    const bool early_load = kFused && (split != 0 || n_local > 2);

    if constexpr (kFused) {
        // Waves 0-1 rope the g query heads (8 lanes a head) into LDS; in the
        // workgroup holding the token's page (the chunk's last) also q_out,
        // wave 2 the kv head's K and wave 3 its V, stored before the barrier
        // below. The token's slot is its page id, already in LDS.
        if (writer && tid == 0 && w.slots) s_slot = token_slot(w, b, rr.p, true);
        if (tid < D / 2) {
            const double ang = (double)rr.p * freq;       // as the write kernel's angle table
            double sn, cs;
            sincos(ang, &sn, &cs);
            s_sn[tid] = sn;
            s_cs[tid] = cs;
        }
        __syncthreads();
        if (early_load) {
            ok_a = prep(u, base_a, kt, vt, half);
            load_unit<D>(fa, kt, vt, half, lane);
        }
        long long slot = -1;
        if (writer) {
            if (w.slots) {
                slot = s_slot;
            } else {
                const int pg = s_pg[n_local - 1];           // the page of position p (-1: flagged above)
                slot = pg >= 0 ? (long long)pg * kPage + (rr.p & (kPage - 1)) : -1;
            }
        }
        if (wave < 3) {
            u32x4 ol, oh;
            rope_chunk_pair<D>(w, wave < 2, j & 7, act, lo, hi, s_cs, s_sn, ol, oh);
            if (act && wave < 2) {
                *reinterpret_cast<u32x4*>(&s_q[hh * D + 8 * j]) = ol;
                *reinterpret_cast<u32x4*>(&s_q[hh * D + D / 2 + 8 * j]) = oh;
                if (writer) {
                    uint16_t* dst = w.q_out + (long long)b * w.ld_q_out + (long long)(kh * G + hh) * D;
                    *reinterpret_cast<u32x4*>(dst + 8 * j) = ol;
                    *reinterpret_cast<u32x4*>(dst + D / 2 + 8 * j) = oh;
                }
            } else if (act && slot >= 0) {
                const int in_page = (int)(slot & (kPage - 1));
                uint16_t* tile = w.k_pool + ((slot >> 6) * w.n_kv_heads + kh) * (long long)(D * kPage);
                *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, 8 * j, D)) = ol;
                *reinterpret_cast<u32x4*>(tile + k_tile_offset(in_page, D / 2 + 8 * j, D)) = oh;
            }
        } else if (writer && slot >= 0) {
            const int in_page = (int)(slot & (kPage - 1));
            uint16_t* tile = w.v_pool + ((slot >> 6) * w.n_kv_heads + kh) * (long long)(D * kPage);
#pragma unroll
            for (int i = 0; i < kVPerLane; ++i)
                if (64 * i + lane < D) tile[v_tile_offset(in_page, 64 * i + lane, D)] = vv[i];
        }
        __syncthreads();        // the stores are complete before any page load below
    }

    // q^T as the B operand: column = head, rows = dims 32s + 8*grp .. +7.
    bf16x8 qf[kSteps];
    {
        const bool real = col < G;
        const uint16_t* qrow = kFused ? &s_q[(real ? col : 0) * D]
                                      : a.q + (long long)b * a.ld_q + (long long)(kh * G + (real ? col : 0)) * D;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            u32x4 u = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp);
            if (!real) u = u32x4{0u, 0u, 0u, 0u};
            qf[s] = as_bf16x8(u);
        }
    }
    __syncthreads();

    const float c = kLog2e / sqrtf((float)D);
    WaveState<D> st;
    st.m = -INFINITY;
    st.lsum = 0.f;
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // (the first unit's load is issued above in the fused case when early)
    if (!kFused || !early_load) {
        ok_a = prep(u, base_a, kt, vt, half);
        load_unit<D>(fa, kt, vt, half, lane);
    }
    while (u < n_units) {
        const bool ok_b = prep(u + kDecodeWaves, base_b, kt, vt, half);
        load_unit<D>(fb, kt, vt, half, lane);
        if (ok_a) compute_unit<D>(st, fa, qf, c, base_a, rr.lo, rr.p, grp);
        u += kDecodeWaves;
        if (u >= n_units) break;
        ok_a = prep(u + kDecodeWaves, base_a, kt, vt, half);
        load_unit<D>(fa, kt, vt, half, lane);
        if (ok_b) compute_unit<D>(st, fb, qf, c, base_b, rr.lo, rr.p, grp);
        u += kDecodeWaves;
    }
    float m = st.m, lsum = st.lsum;
    f32x4* o = st.o;

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
        for (int r = 0; r < 4; ++r)
            if (col < G) s_o[(wave * D + 16 * db + 4 * grp + r) * G + col] = o[db][r];
    __syncthreads();

    // merge the waves: this chunk's (m, l, o) for each real head
    const long long pair = (long long)b * a.n_kv_heads + kh;
    const long long slot = pair * max_splits + split;
    float* part_o = ws + slot * G * D;                                        // [G][D]
    float* part_ml = ws + (long long)a.n_tokens * a.n_kv_heads * max_splits * G * D + slot * G * 2;
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
                ov += sw * s_o[(w * D + d) * G + j];
                lv += sw * s_l[w][j];
            }
        }
        if (n_splits == 1) {               // the whole row in one chunk: finish here
            a.out[(long long)b * a.ld_out + (long long)(kh * G + j) * D + d] =
                (uint16_t)f32_to_bf16(lv > 0.f ? ov / lv : 0.f);
            continue;
        }
        part_o[item] = ov;
        if (d == 0) {
            part_ml[2 * j] = M;
            part_ml[2 * j + 1] = lv;
        }
    }
}

}  // namespace dec
}  // namespace dap
