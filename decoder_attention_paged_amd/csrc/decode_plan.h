// Decode split plan: how many pages each chunk of a row covers and how many
// chunks a row may have, with the workspace that holds their partials.
// Host arithmetic only (no HIP), so it also builds into host-side checks.
#pragma once

#include <stddef.h>

namespace dap {

constexpr int kPage = 64;
constexpr int kDecodeWaves = 4;          // waves per decode workgroup
constexpr int kMaxPagesPerSplit = 256;   // the decode workgroup's LDS page-id array
constexpr int kMinPagesPerSplit = 2 * kDecodeWaves;
constexpr int kMaxSplits = 256;          // the merge's LDS chunk weights
constexpr int kMaxDecodeRows = 65535;
constexpr int kMaxPosition = 1 << 22;

// Workspace: partial o [n_rows][Hkv][max_splits][g][D] floats, then
// (m, l) [n_rows][Hkv][max_splits][g][2] floats.
struct DecodePlan {
    int pages_per_split;
    int max_splits;
    size_t workspace_bytes;
};

// Most pages one row's attended range [lo, p] can touch: the whole row up
// to max_position without a window; with a window W, ceil(W/64) pages plus
// one when the range straddles a page edge, but never more than the row has.
inline int decode_max_pages(int window, int max_position) {
    const long long row_pages = ((long long)max_position + kPage - 1) / kPage;
    long long pages = row_pages;
    if (window > 0) {
        const long long w = (long long)window < max_position ? window : max_position;
        pages = (w + kPage - 1) / kPage + 1;
        if (pages > row_pages) pages = row_pages;
    }
    return (int)pages;
}

// Chunk size: about 8K workgroups in total (about half active for uniformly
// spread lengths), at least two pages per wave (small decodes: fewer chunks
// per row repeat less per-workgroup set-up and merge fewer partials; a 1-4
// row decode over ~33 pages took 21.1 us per step at one page per wave,
// 19.3 at two, 20.8 at three, 20.3 at four), a multiple of the wave count,
// at most kMaxPagesPerSplit, and few enough chunks per row for the merge.
// With max_position <= kMaxPosition (65536 pages) both caps hold together:
// 65536 pages / 256 chunks = 256 pages per chunk.
inline DecodePlan decode_plan(int n_rows, int n_q_heads, int n_kv_heads, int head_dim, int window,
                              int max_position) {
    DecodePlan p;
    const int max_pages = decode_max_pages(window, max_position);
    const long long pairs = (long long)n_rows * n_kv_heads;
    long long pps = (pairs * max_pages + 8191) / 8192;
    pps = (pps + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
    if (pps < kMinPagesPerSplit) pps = kMinPagesPerSplit;
    if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
    if ((max_pages + pps - 1) / pps > kMaxSplits) pps = (max_pages + kMaxSplits - 1) / kMaxSplits;
    p.pages_per_split = (int)pps;
    p.max_splits = (int)((max_pages + pps - 1) / pps);
    p.workspace_bytes = (size_t)n_rows * n_q_heads * p.max_splits * (head_dim + 2) * sizeof(float);
    return p;
}

// Whether a plan fits the kernels' LDS arrays (false only past kMaxPosition).
inline bool decode_plan_fits(const DecodePlan& p) {
    return p.pages_per_split <= kMaxPagesPerSplit && p.max_splits <= kMaxSplits;
}

}  // namespace dap
