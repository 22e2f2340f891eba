// Internal declarations shared by the library's HIP translation units.
// Device helpers (bf16 conversions, MFMA vector types) and the launchers
// each kernel file exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dap.h"
#include "decode_plan.h"

namespace dap {

// Bits of the device error word (kernels OR them in when an index read from
// device memory is out of range; the entry is skipped).
enum ErrorBits : unsigned {
    kErrPosition = 1u,
    kErrRow = 2u,
    kErrPage = 4u,
    kErrSlot = 8u,
    kErrTable = 16u,
    kErrSegments = 32u,  // more runs of equal segment ids than the prefill launch has tiles for
    kErrSpan = 64u,      // an in-pass segment's positions do not fit its scratch pages
};

// ---- page tile layout ------------------------------------------------------
// A (page, kv head) tile of 64 keys x D dims is stored as 16-byte chunks (8
// bf16) in the order one decode wave loads them, 64 lanes x 16 bytes = 1 KB
// per load, so every load reads one contiguous kilobyte.
// K: fragment f = (half * 2 + blk) * (D / 32) + s, lane l = 16 * grp + i holds
//    key 32 * half + unit_key(blk, i), dims 32 * s + 8 * grp .. + 7.
// V: fragment f = half * (D / 16) + db, lane l = 16 * grp + col holds dim
//    16 * db + col, keys 32 * half + 8 * grp .. + 7.
// unit_key permutes the keys of a 32-key half inside the 16x16 S blocks so
// that lane group g's S values are the 8 contiguous keys its V chunk holds.
__host__ __device__ __forceinline__ int unit_key(int blk, int i) { return 8 * (i >> 2) + 4 * blk + (i & 3); }

// element offset of K (key, d) / V (key, d) inside a tile
__host__ __device__ __forceinline__ int k_tile_offset(int key, int d, int D) {
    const int half = key >> 5, kk = key & 31;
    const int blk = (kk >> 2) & 1, i = ((kk >> 3) << 2) | (kk & 3);
    const int f = (half * 2 + blk) * (D / 32) + (d >> 5);
    return ((f * 64 + ((d >> 3) & 3) * 16 + i) << 3) + (d & 7);
}
__host__ __device__ __forceinline__ int v_tile_offset(int key, int d, int D) {
    const int half = key >> 5, kk = key & 31;
    const int f = half * (D / 16) + (d >> 4);
    return ((f * 64 + (kk >> 3) * 16 + (d & 15)) << 3) + (kk & 7);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};   // dot2 with this adds a pair
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// float64 -> bf16, rounded to nearest even as if in one step, without
// branches: first to float32 rounding to odd (to nearest, then, when that was
// inexact and left the last bit even, one step toward x), then to bf16 to
// nearest even. Rounding to odd with at least two spare bits followed by
// rounding to nearest gives the directly rounded result (the double-rounding
// theorem of Boldo and Melquiond); float32 keeps 16 bits more than bf16 at
// every exponent, subnormals included, and the two share the exponent range.
// NaN gives the quiet NaN 0x7fc0 with x's sign.
__host__ __device__ __forceinline__ uint32_t f64_to_bf16(double x) {
    const float f = (float)x;
    const double back = (double)f;
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    const bool step = back != x && !(u & 1u) && (u & 0x7f800000u) != 0x7f800000u;
    u += step ? (fabs(back) > fabs(x) ? 0xffffffffu : 1u) : 0u;
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = ((uint32_t)(__builtin_bit_cast(uint64_t, x) >> 48) & 0x8000u) | 0x7fc0u;
    return x != x ? nan : r;
}

// ---------------------------------------------------------------------------
// Kernel timing hook: when a handle has profiling on, every launch is
// bracketed by begin/end, which record a pair of hipEvents on the launch
// stream (see dap_set_profiling).
struct ProfilerState;
struct Profiler {
    ProfilerState* st;
    void begin(int kind, hipStream_t s);
    void end(int kind, hipStream_t s);
};

// Launchers (host functions living next to their kernels).

struct WriteArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ld_in;
    int32_t n_tokens;
    const int32_t* positions;
    const int32_t* rows;
    const int32_t* slots;
    const int32_t* table;
    int32_t table_ld;
    int32_t n_table_rows;
    const uint16_t* q_gain;
    const uint16_t* k_gain;
    uint16_t* q_out;
    int64_t ld_q_out;
    uint16_t* k_pool;
    uint16_t* v_pool;
    int32_t n_pages;
    int32_t n_q_heads, n_kv_heads, head_dim, max_position;
    int32_t qk_norm;
    double eps;
    const double* inv_freq;   // device [D/2]
    unsigned* err;
};
hipError_t launch_write(const WriteArgs& a, hipStream_t s, Profiler* prof);

struct AttnArgs {
    const uint16_t* q;
    int64_t ld_q;
    int32_t n_tokens;          // prefill: tokens; decode: rows
    const int32_t* positions;
    const int32_t* rows;       // prefill: segments (table rows); decode: nullable
    const int32_t* table;
    int32_t table_ld;
    int32_t n_table_rows;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    int32_t n_pages;
    uint16_t* out;
    int64_t ld_out;
    int32_t n_q_heads, n_kv_heads, head_dim, window, max_position;
    unsigned* err;
};

// Decode: split plan in decode_plan.h.
// fused: also write each row's token (rope, norm, K/V into its slot, q_out)
// from the raw projection, in the workgroups that read the token's page
hipError_t launch_decode(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t s,
                         Profiler* prof, const WriteArgs* fused = nullptr);

// the cross-chunk merge alone (rows of several chunks), after a decode whose
// partials are in `workspace`
hipError_t launch_decode_merge(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t s,
                               Profiler* prof);

// Fused step: the packed prefill's tiles (pre, its tokens) and the decode's
// chunks (dec, its rows) in one launch, then the decode's merge. Each prefill
// workgroup finds its own tile (no tile-list pass); pre.n_tokens > 0 and
// dec.n_tokens > 0, group 1, 2 or 4.
int step_tile_cap(int n_prompt, int n_segments, int group);     // prefill workgroup slots per kv head
hipError_t launch_step(const AttnArgs& pre, int n_segments, const AttnArgs& dec, const DecodePlan& plan,
                       void* workspace, hipStream_t s, Profiler* prof);

// Prefill: tile list sizing and launch.
size_t prefill_workspace(int n_tokens, int n_segments, int group, int head_dim);
int tile_cap(int n_tokens, int n_segments, int group, int head_dim);   // most tiles one prefill call may form
hipError_t launch_prefill(const AttnArgs& a, int n_segments, void* workspace, hipStream_t s, Profiler* prof);

// Index preparation for the contiguous-cache entries: per-token positions and
// rows for tokens laid out [groups][per_group], and an identity page table.
enum LayoutMode : int {
    kLayoutConstPos = 0,   // position = base_pos, row = token
    kLayoutSpan = 1,       // position = base_pos + i, row = group
    kLayoutSlots = 2,      // position = i, row = row_map[group]
    kLayoutRowsOnly = 3,   // row = token (positions given by the caller)
};
struct LayoutPrep {
    int mode;
    int n_tokens;
    int per_group;
    int base_pos;
    const int32_t* row_map;
    int32_t* positions;     // may be null (kLayoutRowsOnly)
    int32_t* rows;
    int32_t* table;         // identity table [table_rows][table_ld], may be null
    int table_rows;
    int table_ld;
};
hipError_t launch_layout_prep(const LayoutPrep& p, hipStream_t s, Profiler* prof);

// Index preparation for the in-pass entries (no cache): each segment's keys
// go to scratch pages, packed segment after segment from its first position.
constexpr int kMaxInpassSegments = 4096;
struct InpassPrep {
    const int32_t* positions;
    const int32_t* segments;
    int n_tokens;
    int n_segments;
    int32_t* table;         // [n_segments][table_ld] scratch page ids, -1 past a segment
    int table_ld;
    int capacity;           // scratch pages
    int32_t* slots;         // [n_tokens] scratch slot of each token, -1 if it does not fit
    int32_t* rel_positions; // [n_tokens] position minus its segment's first position
    int32_t* seg_lo;        // [n_segments] scratch: each segment's first position,
    int32_t* seg_hi;        //   last position
    int32_t* seg_first;     //   and first scratch page
    unsigned* err;
};
hipError_t launch_inpass_prep(const InpassPrep& p, hipStream_t s, Profiler* prof);

}  // namespace dap
