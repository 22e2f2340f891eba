// C-ABI layer: handle, argument checks, validate mode, launches.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <algorithm>
#include <unordered_set>
#include <vector>

#include "dap_internal.h"

// ---------------------------------------------------------------- kernel timing
namespace dap {

struct ProfilerState {
    static constexpr int kCap = 1024;
    std::vector<hipEvent_t> start, stop;
    std::vector<int> kind;
    int head = 0, count = 0, cur = -1;
    double total_ms[DAP_N_KERNELS] = {};
    int64_t launches[DAP_N_KERNELS] = {};

    hipError_t init() {
        start.assign(kCap, nullptr);
        stop.assign(kCap, nullptr);
        kind.assign(kCap, 0);
        for (int i = 0; i < kCap; ++i) {
            hipError_t e = hipEventCreate(&start[i]);
            if (e == hipSuccess) e = hipEventCreate(&stop[i]);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    ~ProfilerState() {
        for (auto ev : start) if (ev) (void)hipEventDestroy(ev);
        for (auto ev : stop) if (ev) (void)hipEventDestroy(ev);
    }
    hipError_t drain_one() {
        const int i = head;
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(stop[i]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, start[i], stop[i]);
        if (e != hipSuccess) return e;
        total_ms[kind[i]] += ms;
        launches[kind[i]] += 1;
        head = (head + 1) % kCap;
        --count;
        return hipSuccess;
    }
};

void Profiler::begin(int k, hipStream_t s) {
    if (st->count == ProfilerState::kCap) (void)st->drain_one();
    const int i = (st->head + st->count) % ProfilerState::kCap;
    st->kind[i] = k;
    st->cur = i;
    (void)hipEventRecord(st->start[i], s);
}

void Profiler::end(int, hipStream_t s) {
    if (st->cur < 0) return;
    (void)hipEventRecord(st->stop[st->cur], s);
    st->cur = -1;
    st->count += 1;
}

}  // namespace dap

// ---------------------------------------------------------------- static decode scratch
// dap_attn_decode_paged_noalloc keeps the decode's per-chunk partials in this
// file-scope device array instead of a caller workspace. Every device the
// library runs on holds its own copy until the process ends, and every call
// on that device shares it (overlapping calls on one device race). In host
// code the name is only a stand-in for the symbol, not a device address:
// the address comes from hipGetSymbolAddress, once per device (at the first
// dap_create there, with that device current), and is what the kernels get.
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static hipError_t scratch_address(int dev, void** out) {
    *out = nullptr;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

struct dap_handle {
    dap_model m;
    int device;
    void* scratch;     // this device's static decode scratch (its device address)
    int group;
    std::vector<double> h_inv_freq;
    double* d_inv_freq;
    unsigned* d_err;
    int validate;
    int one_pass_step;     // step_paged runs prompts and decode rows in one launch (DAP_FUSED_STEP=0: off)
    dap::ProfilerState* prof_state;
    dap::Profiler prof;
    dap::Profiler* profiler() { return prof_state ? &prof : nullptr; }
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(DAP_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define DAP_REQUIRE(cond, code, msg) \
    do {                             \
        if (!(cond)) return fail((code), (msg)); \
    } while (0)

// Frequency table in float64 (see dap_create in dap.h).
std::vector<double> build_inv_freq(const dap_model& m) {
    const int half = m.head_dim / 2;
    std::vector<double> f(half);
    for (int i = 0; i < half; ++i) f[i] = std::pow(m.rope_theta, -2.0 * i / m.head_dim);
    if (m.llama3) {
        const double factor = m.llama3_factor, low = m.llama3_low_freq_factor, high = m.llama3_high_freq_factor;
        const double orig = m.llama3_original_max_position;
        const double low_wavelen = orig / low, high_wavelen = orig / high;
        for (int i = 0; i < half; ++i) {
            const double wavelen = 2.0 * M_PI / f[i];
            if (wavelen < high_wavelen) continue;
            if (wavelen > low_wavelen) {
                f[i] = f[i] / factor;
            } else {
                const double s = (orig / wavelen - low) / (high - low);
                f[i] = (1.0 - s) * f[i] / factor + s * f[i];
            }
        }
    }
    return f;
}

// ---------------------------------------------------------------- validate mode
template <typename T>
bool to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
    dst.resize(n);
    if (n == 0) return true;
    if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess) return false;
    return hipStreamSynchronize(s) == hipSuccess;
}

int begin_validate(dap_handle* h, hipStream_t s) {
    hipError_t e = hipMemsetAsync(h->d_err, 0, sizeof(unsigned), s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(error word)");
    return DAP_OK;
}

int end_validate(dap_handle* h, hipStream_t s) {
    unsigned err = 0;
    hipError_t e = hipMemcpyAsync(&err, h->d_err, sizeof(unsigned), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the error word");
    if (err) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "a kernel skipped out-of-range index entries (error bits 0x%x: 1 position, 2 row, "
                      "4 page, 8 slot, 16 table width, 32 segment runs, 64 in-pass span)", err);
        return fail(DAP_BAD_INDEX, buf);
    }
    return DAP_OK;
}

// Host checks of (row, position) -> page through the table; returns DAP_OK or DAP_BAD_INDEX.
int check_rows(const dap_handle* h, const std::vector<int32_t>& pos, const std::vector<int32_t>& rows,
               const std::vector<int32_t>& table, int32_t table_ld, int32_t n_table_rows, int32_t n_pages,
               bool whole_range, std::vector<long long>* slots_out) {
    const int W = h->m.window;
    for (size_t t = 0; t < pos.size(); ++t) {
        const int p = pos[t];
        if (p < 0 || p >= h->m.max_position) return fail(DAP_BAD_INDEX, "position " + std::to_string(p) + " out of range at " + std::to_string(t));
        const int r = rows.empty() ? (int)t : rows[t];
        if (r < 0 || r >= n_table_rows) return fail(DAP_BAD_INDEX, "table row " + std::to_string(r) + " out of range at " + std::to_string(t));
        const int lo = whole_range ? (W > 0 ? std::max(0, p - W + 1) : 0) : p;
        if (p / dap::kPage >= table_ld) return fail(DAP_BAD_INDEX, "position beyond the table width at " + std::to_string(t));
        for (int j = lo / dap::kPage; j <= p / dap::kPage; ++j) {
            const int pg = table[(size_t)r * table_ld + j];
            if (pg < 0 || pg >= n_pages) return fail(DAP_BAD_INDEX, "page id " + std::to_string(pg) + " out of range (row " + std::to_string(r) + ", entry " + std::to_string(j) + ")");
        }
        if (slots_out) slots_out->push_back((long long)table[(size_t)r * table_ld + p / dap::kPage] * dap::kPage + p % dap::kPage);
    }
    return DAP_OK;
}

int check_handle(const dap_handle* h) {
    if (!h) return fail(DAP_INVALID_ARG, "null handle");
    return DAP_OK;
}

int check_table_args(const int32_t* table, int32_t table_ld, int32_t n_table_rows, int32_t n_pages) {
    DAP_REQUIRE(table && aligned4(table), DAP_INVALID_ARG, "table must be a non-null, 4-byte aligned device pointer");
    DAP_REQUIRE(table_ld > 0 && n_table_rows > 0, DAP_INVALID_ARG, "table_ld and n_table_rows must be positive");
    DAP_REQUIRE(n_pages > 0, DAP_INVALID_ARG, "n_pages must be positive");
    return DAP_OK;
}

int check_stride(int64_t ld, int64_t width, const char* name) {
    if (ld < width || ld % 8 != 0)
        return fail(DAP_INVALID_ARG, std::string(name) + " must be >= the row width and a multiple of 8 elements");
    return DAP_OK;
}

dap::AttnArgs attn_args(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n, const int32_t* positions,
                        const int32_t* rows, const int32_t* table, int32_t table_ld, int32_t n_table_rows,
                        const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages, uint16_t* out,
                        int64_t ld_out) {
    dap::AttnArgs a;
    a.q = q; a.ld_q = ld_q; a.n_tokens = n; a.positions = positions; a.rows = rows;
    a.table = table; a.table_ld = table_ld; a.n_table_rows = n_table_rows;
    a.k_pool = k_pool; a.v_pool = v_pool; a.n_pages = n_pages; a.out = out; a.ld_out = ld_out;
    a.n_q_heads = h->m.n_q_heads; a.n_kv_heads = h->m.n_kv_heads; a.head_dim = h->m.head_dim;
    a.window = h->m.window; a.max_position = h->m.max_position; a.err = h->d_err;
    return a;
}

// ---------------------------------------------------------------- entry bodies
// Argument checks of a write of n_tokens (and, in validate mode, the
// host-side index checks); fills `a`. Nothing is launched.
int write_args(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
               int32_t n_tokens, const int32_t* positions, const int32_t* rows, const int32_t* slots,
               const int32_t* table, int32_t table_ld, int32_t n_table_rows, const uint16_t* q_gain,
               const uint16_t* k_gain, uint16_t* q_out, int64_t ld_q_out, uint16_t* k_pool, uint16_t* v_pool,
               int32_t n_pages, dap::WriteArgs& a, hipStream_t s) {
    const dap_model& m = h->m;
    const int64_t D = m.head_dim;
    a = dap::WriteArgs{};
    DAP_REQUIRE(n_tokens >= 0, DAP_INVALID_ARG, "n_tokens must be >= 0");
    if (n_tokens == 0) return DAP_OK;
    DAP_REQUIRE(q && k && v && q_out && k_pool && v_pool, DAP_INVALID_ARG, "null tensor pointer");
    DAP_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(q_out) && aligned16(k_pool) && aligned16(v_pool),
                DAP_INVALID_ARG, "bf16 tensors must be 16-byte aligned");
    DAP_REQUIRE(positions && aligned4(positions), DAP_INVALID_ARG, "positions must be a non-null aligned pointer");
    DAP_REQUIRE(slots || rows, DAP_INVALID_ARG, "either slots or rows (with the table) is required");
    DAP_REQUIRE(n_pages > 0, DAP_INVALID_ARG, "n_pages must be positive");
    if (!slots) {
        int rc = check_table_args(table, table_ld, n_table_rows, n_pages);
        if (rc) return rc;
    }
    if (int rc = check_stride(ld_in, std::max<int64_t>(m.n_q_heads, m.n_kv_heads) * D, "ld_in")) return rc;
    if (int rc = check_stride(ld_q_out, m.n_q_heads * D, "ld_q_out")) return rc;
    if (m.qk_norm) {
        DAP_REQUIRE(q_gain && k_gain && aligned16(q_gain) && aligned16(k_gain), DAP_INVALID_ARG,
                    "qk_norm needs 16-byte aligned q_gain and k_gain");
    }
    if (q_out == q) DAP_REQUIRE(ld_q_out == ld_in, DAP_INVALID_ARG, "in-place q_out needs ld_q_out == ld_in");

    if (h->validate) {
        std::vector<int32_t> hp, hr, hs, ht;
        if (!to_host(hp, positions, n_tokens, s)) return fail(DAP_HIP_ERROR, "copying positions");
        std::vector<long long> sl;
        if (slots) {
            if (!to_host(hs, slots, n_tokens, s)) return fail(DAP_HIP_ERROR, "copying slots");
            for (int t = 0; t < n_tokens; ++t) {
                if (hp[t] < 0 || hp[t] >= m.max_position) return fail(DAP_BAD_INDEX, "position out of range at " + std::to_string(t));
                if (hs[t] < 0 || (long long)hs[t] >= (long long)n_pages * dap::kPage) return fail(DAP_BAD_INDEX, "slot out of range at " + std::to_string(t));
                sl.push_back(hs[t]);
            }
        } else {
            if (!to_host(hr, rows, n_tokens, s) || !to_host(ht, table, (size_t)table_ld * n_table_rows, s))
                return fail(DAP_HIP_ERROR, "copying rows/table");
            if (int rc = check_rows(h, hp, hr, ht, table_ld, n_table_rows, n_pages, false, &sl)) return rc;
        }
        std::unordered_set<long long> seen;
        for (long long x : sl)
            if (!seen.insert(x).second) return fail(DAP_BAD_INDEX, "two tokens write the same slot " + std::to_string(x));
    }
    a.q = q; a.k = k; a.v = v; a.ld_in = ld_in; a.n_tokens = n_tokens; a.positions = positions;
    a.rows = rows; a.slots = slots; a.table = table; a.table_ld = table_ld; a.n_table_rows = n_table_rows;
    a.q_gain = q_gain; a.k_gain = k_gain; a.q_out = q_out; a.ld_q_out = ld_q_out;
    a.k_pool = k_pool; a.v_pool = v_pool; a.n_pages = n_pages;
    a.n_q_heads = m.n_q_heads; a.n_kv_heads = m.n_kv_heads; a.head_dim = m.head_dim; a.max_position = m.max_position;
    a.qk_norm = m.qk_norm; a.eps = m.qk_norm_eps; a.inv_freq = h->d_inv_freq; a.err = h->d_err;
    return DAP_OK;
}

int launch_write_checked(dap_handle* h, const dap::WriteArgs& a, hipStream_t s) {
    if (a.n_tokens == 0) return DAP_OK;
    if (h->validate)
        if (int rc = begin_validate(h, s)) return rc;
    hipError_t e = dap::launch_write(a, s, h->profiler());
    if (e != hipSuccess) return hip_fail(e, "rope/write launch");
    return h->validate ? end_validate(h, s) : DAP_OK;
}

int do_write(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
             int32_t n_tokens, const int32_t* positions, const int32_t* rows, const int32_t* slots,
             const int32_t* table, int32_t table_ld, int32_t n_table_rows, const uint16_t* q_gain,
             const uint16_t* k_gain, uint16_t* q_out, int64_t ld_q_out, uint16_t* k_pool, uint16_t* v_pool,
             int32_t n_pages, hipStream_t s) {
    dap::WriteArgs a;
    if (int rc = write_args(h, q, k, v, ld_in, n_tokens, positions, rows, slots, table, table_ld, n_table_rows,
                            q_gain, k_gain, q_out, ld_q_out, k_pool, v_pool, n_pages, a, s))
        return rc;
    return launch_write_checked(h, a, s);
}

int attn_common_checks(dap_handle* h, const uint16_t* q, int64_t ld_q, const int32_t* positions, const int32_t* table,
                       int32_t table_ld, int32_t n_table_rows, const uint16_t* k_pool, const uint16_t* v_pool,
                       int32_t n_pages, const uint16_t* out, int64_t ld_out) {
    const int64_t W = (int64_t)h->m.n_q_heads * h->m.head_dim;
    DAP_REQUIRE(q && out && k_pool && v_pool, DAP_INVALID_ARG, "null tensor pointer");
    DAP_REQUIRE(aligned16(q) && aligned16(out) && aligned16(k_pool) && aligned16(v_pool), DAP_INVALID_ARG,
                "bf16 tensors must be 16-byte aligned");
    DAP_REQUIRE(positions && aligned4(positions), DAP_INVALID_ARG, "positions must be a non-null aligned pointer");
    if (int rc = check_table_args(table, table_ld, n_table_rows, n_pages)) return rc;
    if (int rc = check_stride(ld_q, W, "ld_q")) return rc;
    if (int rc = check_stride(ld_out, W, "ld_out")) return rc;
    DAP_REQUIRE(out != q, DAP_INVALID_ARG, "out must not alias q");
    return DAP_OK;
}

// Checks of a packed prefill of n_tokens > 0 tokens launched as tile_blocks
// workgroups (and, in validate mode, the host-side index checks). Nothing
// is launched.
int prefill_checks(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_tokens, const int32_t* positions,
                   const int32_t* segments, int32_t n_segments, const int32_t* table, int32_t table_ld,
                   int32_t n_table_rows, const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
                   const uint16_t* out, int64_t ld_out, long long tile_blocks, hipStream_t s) {
    DAP_REQUIRE(h->group == 1 || h->group == 2 || h->group == 4, DAP_UNSUPPORTED,
                "prefill supports Hq/Hkv of 1, 2 or 4");
    if (int rc = attn_common_checks(h, q, ld_q, positions, table, table_ld, n_table_rows, k_pool, v_pool, n_pages, out, ld_out))
        return rc;
    DAP_REQUIRE(segments && aligned4(segments), DAP_INVALID_ARG, "segments must be a non-null aligned pointer");
    DAP_REQUIRE(n_segments > 0, DAP_INVALID_ARG, "n_segments must be positive");
    DAP_REQUIRE(tile_blocks < (1ll << 31), DAP_UNSUPPORTED, "too many prefill tiles for one launch");
    if (h->validate) {
        std::vector<int32_t> hp, hs, ht;
        if (!to_host(hp, positions, n_tokens, s) || !to_host(hs, segments, n_tokens, s) ||
            !to_host(ht, table, (size_t)table_ld * n_table_rows, s))
            return fail(DAP_HIP_ERROR, "copying index arrays");
        if (int rc = check_rows(h, hp, hs, ht, table_ld, n_table_rows, n_pages, true, nullptr)) return rc;
        int runs = 0;
        for (int t = 0; t < n_tokens; ++t) runs += (t == 0 || hs[t] != hs[t - 1]);
        if (runs > n_segments) return fail(DAP_BAD_INDEX, "more runs of equal segment ids than n_segments");
    }
    return DAP_OK;
}

int do_prefill(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_tokens, const int32_t* positions,
               const int32_t* segments, int32_t n_segments, const int32_t* table, int32_t table_ld,
               int32_t n_table_rows, const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages, uint16_t* out,
               int64_t ld_out, void* workspace, size_t workspace_bytes, hipStream_t s) {
    DAP_REQUIRE(n_tokens >= 0, DAP_INVALID_ARG, "n_tokens must be >= 0");
    if (n_tokens == 0) return DAP_OK;
    const long long blocks =
        n_segments > 0 ? (long long)dap::tile_cap(n_tokens, n_segments, h->group, h->m.head_dim) * h->m.n_kv_heads : 0;
    if (int rc = prefill_checks(h, q, ld_q, n_tokens, positions, segments, n_segments, table, table_ld, n_table_rows,
                                k_pool, v_pool, n_pages, out, ld_out, blocks, s))
        return rc;
    const size_t need = dap::prefill_workspace(n_tokens, n_segments, h->group, h->m.head_dim);
    DAP_REQUIRE(workspace && workspace_bytes >= need && aligned16(workspace), DAP_WORKSPACE_TOO_SMALL,
                "workspace must be 16-byte aligned and at least dap_prefill_workspace_bytes()");
    if (h->validate)
        if (int rc = begin_validate(h, s)) return rc;
    dap::AttnArgs a = attn_args(h, q, ld_q, n_tokens, positions, segments, table, table_ld, n_table_rows, k_pool,
                                v_pool, n_pages, out, ld_out);
    hipError_t e = dap::launch_prefill(a, n_segments, workspace, s, h->profiler());
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return h->validate ? end_validate(h, s) : DAP_OK;
}

// Checks of a decode of n_rows > 0 rows (and, in validate mode, the host
// index checks); returns its plan in `plan`. Nothing is launched.
int decode_checks(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_rows, const int32_t* positions,
                  const int32_t* rows, const int32_t* table, int32_t table_ld, int32_t n_table_rows,
                  const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages, const uint16_t* out, int64_t ld_out,
                  size_t workspace_bytes, const void* workspace, dap::DecodePlan& plan, hipStream_t s) {
    DAP_REQUIRE(n_rows <= dap::kMaxDecodeRows, DAP_UNSUPPORTED, "at most 65535 rows per decode call");
    if (int rc = attn_common_checks(h, q, ld_q, positions, table, table_ld, n_table_rows, k_pool, v_pool, n_pages, out, ld_out))
        return rc;
    DAP_REQUIRE(!rows || aligned4(rows), DAP_INVALID_ARG, "rows must be aligned");
    plan = dap::decode_plan(n_rows, h->m.n_q_heads, h->m.n_kv_heads, h->m.head_dim, h->m.window, h->m.max_position);
    DAP_REQUIRE(dap::decode_plan_fits(plan), DAP_UNSUPPORTED, "decode split plan beyond the kernel's limits");
    DAP_REQUIRE(workspace && workspace_bytes >= plan.workspace_bytes && aligned16(workspace), DAP_WORKSPACE_TOO_SMALL,
                "workspace must be 16-byte aligned and at least dap_decode_workspace_bytes()");
    DAP_REQUIRE((long long)plan.max_splits * h->m.n_kv_heads * n_rows < (1ll << 31), DAP_UNSUPPORTED,
                "too many decode workgroups for one launch");
    if (h->validate) {
        std::vector<int32_t> hp, hr, ht;
        if (!to_host(hp, positions, n_rows, s) || (rows && !to_host(hr, rows, n_rows, s)) ||
            !to_host(ht, table, (size_t)table_ld * n_table_rows, s))
            return fail(DAP_HIP_ERROR, "copying index arrays");
        if (int rc = check_rows(h, hp, hr, ht, table_ld, n_table_rows, n_pages, true, nullptr)) return rc;
    }
    return DAP_OK;
}

int do_decode(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_rows, const int32_t* positions,
              const int32_t* rows, const int32_t* table, int32_t table_ld, int32_t n_table_rows,
              const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages, uint16_t* out, int64_t ld_out,
              void* workspace, size_t workspace_bytes, hipStream_t s, const dap::WriteArgs* fused = nullptr) {
    DAP_REQUIRE(n_rows >= 0, DAP_INVALID_ARG, "n_rows must be >= 0");
    if (n_rows == 0) return DAP_OK;
    dap::DecodePlan plan;
    if (int rc = decode_checks(h, q, ld_q, n_rows, positions, rows, table, table_ld, n_table_rows, k_pool, v_pool,
                               n_pages, out, ld_out, workspace_bytes, workspace, plan, s))
        return rc;
    if (h->validate)
        if (int rc = begin_validate(h, s)) return rc;
    dap::AttnArgs a = attn_args(h, q, ld_q, n_rows, positions, rows, table, table_ld, n_table_rows, k_pool, v_pool,
                                n_pages, out, ld_out);
    hipError_t e = dap::launch_decode(a, plan, workspace, s, h->profiler(), fused);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return h->validate ? end_validate(h, s) : DAP_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Whether a decode of n_rows rows should write its tokens itself. Each of its
// workgroups spends a few microseconds on the rope before its page loads;
// that pays for the write launch it saves (~8-10 us) only while the grid is
// about two rounds of the chip or less: the Phi-3 decode loop (1152
// workgroups) gains 9 %, a 64-row Mistral decode (8192) loses 1 %.
constexpr long long kFusedDecodeMaxBlocks = 2048;
bool fuse_decode(const dap_handle* h, int32_t n_rows) {
    const dap::DecodePlan plan = dap::decode_plan(n_rows, h->m.n_q_heads, h->m.n_kv_heads, h->m.head_dim,
                                                  h->m.window, h->m.max_position);
    return (long long)plan.max_splits * h->m.n_kv_heads * n_rows <= kFusedDecodeMaxBlocks;
}

// step_paged with both prompt tokens and decode rows, in one attention
// launch: every check first (nothing runs if one fails), then the write of
// every token, then the prompts' tiles and the rows' chunks together (one
// kernel), then the decode's merge. The prefill workgroups there find their
// own tiles by scanning the prompts' segment ids, which stays cheap up to a
// few thousand prompt tokens; longer prompt parts take the separate launches.
constexpr int kOnePassMaxPrompt = 4096;

int do_step_one_pass(dap_handle* h, const dap::WriteArgs& wa, int32_t n_prompt, int32_t n_segments, int32_t n_step,
                     const int32_t* positions, const int32_t* rows, const int32_t* table, int32_t table_ld,
                     int32_t n_table_rows, const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
                     uint16_t* out, int64_t ld_out, void* dec_ws, size_t dec_bytes, hipStream_t s) {
    const uint16_t* q_out = wa.q_out;
    const int64_t ld_q = wa.ld_q_out;
    const long long pre_blocks =
        n_segments > 0 ? (long long)dap::step_tile_cap(n_prompt, n_segments, h->group) * h->m.n_kv_heads : 0;
    if (int rc = prefill_checks(h, q_out, ld_q, n_prompt, positions, rows, n_segments, table, table_ld, n_table_rows,
                                k_pool, v_pool, n_pages, out, ld_out, pre_blocks, s))
        return rc;
    dap::DecodePlan plan;
    const uint16_t* q_step = q_out + (int64_t)n_prompt * ld_q;
    uint16_t* out_step = out + (int64_t)n_prompt * ld_out;
    if (int rc = decode_checks(h, q_step, ld_q, n_step, positions + n_prompt, rows + n_prompt, table, table_ld,
                               n_table_rows, k_pool, v_pool, n_pages, out_step, ld_out, dec_bytes, dec_ws, plan, s))
        return rc;
    DAP_REQUIRE(pre_blocks + (long long)plan.max_splits * h->m.n_kv_heads * n_step < (1ll << 31), DAP_UNSUPPORTED,
                "too many workgroups for one launch");
    if (int rc = launch_write_checked(h, wa, s)) return rc;
    if (h->validate)
        if (int rc = begin_validate(h, s)) return rc;
    const dap::AttnArgs pre = attn_args(h, q_out, ld_q, n_prompt, positions, rows, table, table_ld, n_table_rows,
                                        k_pool, v_pool, n_pages, out, ld_out);
    const dap::AttnArgs dec = attn_args(h, q_step, ld_q, n_step, positions + n_prompt, rows + n_prompt, table,
                                        table_ld, n_table_rows, k_pool, v_pool, n_pages, out_step, ld_out);
    hipError_t e = dap::launch_step(pre, n_segments, dec, plan, dec_ws, s, h->profiler());
    if (e != hipSuccess) return hip_fail(e, "step launch");
    return h->validate ? end_validate(h, s) : DAP_OK;
}

// ---------------------------------------------------------------- contiguous-cache and in-pass entries
// Consecutive 256-byte aligned pieces of a workspace (sizes only when base is null).
struct Carve {
    char* base;
    size_t off;
    template <typename T>
    T* take(size_t n) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += align256(n * sizeof(T));
        return p;
    }
};

size_t attn_workspace(const dap_handle* h, long long n_tokens, int n_groups) {
    size_t b = dap::prefill_workspace((int)n_tokens, n_groups, h->group, h->m.head_dim);
    if (n_tokens <= dap::kMaxDecodeRows) {
        const dap::DecodePlan plan = dap::decode_plan((int)n_tokens, h->m.n_q_heads, h->m.n_kv_heads, h->m.head_dim,
                                                      h->m.window, h->m.max_position);
        b = std::max(b, plan.workspace_bytes);
    }
    return b;
}

struct CacheLayout {
    int32_t* positions;
    int32_t* rows;
    int32_t* table;
    uint16_t* q_rope;
    char* attn;
    size_t bytes;
};

CacheLayout cache_layout(const dap_handle* h, void* ws, long long n_tokens, int n_groups, int cache_rows, int max_seq) {
    Carve c{static_cast<char*>(ws), 0};
    CacheLayout L;
    L.positions = c.take<int32_t>(n_tokens);
    L.rows = c.take<int32_t>(n_tokens);
    L.table = c.take<int32_t>((size_t)cache_rows * (max_seq / dap::kPage));
    L.q_rope = c.take<uint16_t>((size_t)n_tokens * h->m.n_q_heads * h->m.head_dim);
    L.attn = c.base ? c.base + c.off : nullptr;
    L.bytes = c.off + attn_workspace(h, n_tokens, n_groups);
    return L;
}

enum CacheKind { kCacheDecode, kCacheDecodeRows, kCachePrefill, kCachePrefillSlots };

// The contiguous-cache entries: identity table and per-token positions/rows
// built on the device, then the write and the paged prefill or decode.
int do_cache(dap_handle* h, CacheKind kind, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
             int32_t n_groups, int32_t per_group, int32_t pos, const int32_t* positions, const int32_t* slot_rows,
             int32_t cache_rows, int32_t max_seq, const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* k_pool,
             uint16_t* v_pool, uint16_t* out, int64_t ld_out, void* ws, size_t ws_bytes, hipStream_t s) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(n_groups >= 0 && per_group >= 0 && cache_rows >= 0, DAP_INVALID_ARG, "counts must be >= 0");
    DAP_REQUIRE(max_seq > 0 && max_seq % dap::kPage == 0, DAP_INVALID_ARG, "max_seq must be a positive multiple of 64");
    const long long n = (long long)n_groups * per_group;
    if (n == 0) return DAP_OK;
    DAP_REQUIRE(n < (1ll << 30), DAP_UNSUPPORTED, "too many tokens for one call");
    const int ppr = max_seq / dap::kPage;
    DAP_REQUIRE(cache_rows > 0 && (long long)cache_rows * ppr * dap::kPage < (1ll << 31), DAP_INVALID_ARG,
                "the cache must have rows and fewer than 2^31 slots");
    const int limit = std::min(max_seq, h->m.max_position);
    if (kind == kCacheDecode || kind == kCachePrefill)
        DAP_REQUIRE(pos >= 0 && (long long)pos + per_group <= limit, DAP_INVALID_ARG,
                    "positions must lie in [0, min(max_seq, max_position))");
    if (kind == kCacheDecodeRows)
        DAP_REQUIRE(positions && aligned4(positions), DAP_INVALID_ARG, "positions must be a non-null aligned pointer");
    if (kind == kCachePrefillSlots) {
        DAP_REQUIRE(slot_rows && aligned4(slot_rows), DAP_INVALID_ARG, "slots must be a non-null aligned pointer");
        DAP_REQUIRE(per_group <= limit, DAP_INVALID_ARG, "seq must be <= min(max_seq, max_position)");
    }
    const CacheLayout L = cache_layout(h, ws, n, n_groups, cache_rows, max_seq);
    DAP_REQUIRE(ws && ws_bytes >= L.bytes && aligned16(ws), DAP_WORKSPACE_TOO_SMALL,
                "workspace must be 16-byte aligned and at least dap_cache_workspace_bytes()");
    if (h->validate && kind == kCachePrefillSlots) {
        std::vector<int32_t> hs;
        if (!to_host(hs, slot_rows, n_groups, s)) return fail(DAP_HIP_ERROR, "copying slots");
        std::unordered_set<int32_t> seen;
        for (int32_t r : hs) {
            if (r < 0 || r >= cache_rows) return fail(DAP_BAD_INDEX, "cache row " + std::to_string(r) + " out of range");
            if (!seen.insert(r).second) return fail(DAP_BAD_INDEX, "two prompts fill cache row " + std::to_string(r));
        }
    }
    dap::LayoutPrep lp;
    lp.mode = kind == kCacheDecode ? dap::kLayoutConstPos
              : kind == kCachePrefill ? dap::kLayoutSpan
              : kind == kCachePrefillSlots ? dap::kLayoutSlots : dap::kLayoutRowsOnly;
    lp.n_tokens = (int)n;
    lp.per_group = per_group;
    lp.base_pos = pos;
    lp.row_map = slot_rows;
    lp.positions = kind == kCacheDecodeRows ? nullptr : L.positions;
    lp.rows = L.rows;
    lp.table = L.table;
    lp.table_rows = cache_rows;
    lp.table_ld = ppr;
    hipError_t e = dap::launch_layout_prep(lp, s, h->profiler());
    if (e != hipSuccess) return hip_fail(e, "index preparation launch");
    const int32_t* P = kind == kCacheDecodeRows ? positions : L.positions;
    const int n_pages = cache_rows * ppr;
    const int64_t wq = (int64_t)h->m.n_q_heads * h->m.head_dim;
    const size_t attn_bytes = ws_bytes - (size_t)(L.attn - static_cast<char*>(ws));
    if ((kind == kCacheDecode || kind == kCacheDecodeRows) && fuse_decode(h, (int)n)) {
        // one token per cache row, roped into the workspace: a small decode
        // writes the tokens itself (no separate write launch)
        dap::WriteArgs wa;
        if (int rc = write_args(h, q, k, v, ld_in, (int)n, P, L.rows, nullptr, L.table, ppr, cache_rows, q_gain,
                                k_gain, L.q_rope, wq, k_pool, v_pool, n_pages, wa, s))
            return rc;
        return do_decode(h, L.q_rope, wq, (int)n, P, L.rows, L.table, ppr, cache_rows, k_pool, v_pool, n_pages, out,
                         ld_out, L.attn, attn_bytes, s, &wa);
    }
    int rc = do_write(h, q, k, v, ld_in, (int)n, P, L.rows, nullptr, L.table, ppr, cache_rows, q_gain, k_gain, L.q_rope,
                      wq, k_pool, v_pool, n_pages, s);
    if (rc) return rc;
    if (kind == kCacheDecode || kind == kCacheDecodeRows)
        return do_decode(h, L.q_rope, wq, (int)n, P, L.rows, L.table, ppr, cache_rows, k_pool, v_pool, n_pages, out,
                         ld_out, L.attn, attn_bytes, s);
    return do_prefill(h, L.q_rope, wq, (int)n, P, L.rows, n_groups, L.table, ppr, cache_rows, k_pool, v_pool, n_pages,
                      out, ld_out, L.attn, attn_bytes, s);
}

struct InpassLayout {
    int32_t* positions;   // dap_forward's generated positions
    int32_t* segments;    // and segments
    int32_t* table;
    int32_t* slots;
    int32_t* rel;
    int32_t* seg_lo;      // per-segment scratch of the preparation
    int32_t* seg_hi;
    int32_t* seg_first;
    uint16_t* q_rope;
    char* prefill;
    uint16_t* k_pool;
    uint16_t* v_pool;
    int table_ld;
    int capacity;
    size_t bytes;
};

InpassLayout inpass_layout(const dap_handle* h, void* ws, long long n_tokens, int n_segments) {
    Carve c{static_cast<char*>(ws), 0};
    InpassLayout L;
    L.table_ld = (int)((n_tokens + dap::kPage - 1) / dap::kPage);
    L.capacity = L.table_ld + n_segments;
    L.positions = c.take<int32_t>(n_tokens);
    L.segments = c.take<int32_t>(n_tokens);
    L.table = c.take<int32_t>((size_t)n_segments * L.table_ld);
    L.slots = c.take<int32_t>(n_tokens);
    L.rel = c.take<int32_t>(n_tokens);
    L.seg_lo = c.take<int32_t>(n_segments);
    L.seg_hi = c.take<int32_t>(n_segments);
    L.seg_first = c.take<int32_t>(n_segments);
    L.q_rope = c.take<uint16_t>((size_t)n_tokens * h->m.n_q_heads * h->m.head_dim);
    L.prefill = c.base ? c.base + c.off : nullptr;
    c.off += align256(dap::prefill_workspace((int)n_tokens, n_segments, h->group, h->m.head_dim));
    const size_t tile = (size_t)h->m.n_kv_heads * dap::kPage * h->m.head_dim;
    L.k_pool = c.take<uint16_t>((size_t)L.capacity * tile);
    L.v_pool = c.take<uint16_t>((size_t)L.capacity * tile);
    L.bytes = c.off;
    return L;
}

// Host check for the in-pass entries: each segment one run of the pack,
// holding consecutive distinct positions.
int check_inpass(const std::vector<int32_t>& pos, const std::vector<int32_t>& seg, int n_segments) {
    std::vector<std::vector<int32_t>> by(n_segments);
    std::vector<int> last_run(n_segments, -1);
    for (size_t t = 0; t < pos.size(); ++t) {
        const int sg = seg[t];
        if (sg < 0 || sg >= n_segments) return fail(DAP_BAD_INDEX, "segment id out of range at " + std::to_string(t));
        if (last_run[sg] >= 0 && last_run[sg] != (int)t - 1)
            return fail(DAP_BAD_INDEX, "segment " + std::to_string(sg) + " is not one run of the pack");
        last_run[sg] = (int)t;
        by[sg].push_back(pos[t]);
    }
    for (int sg = 0; sg < n_segments; ++sg) {
        std::vector<int32_t>& v = by[sg];
        std::sort(v.begin(), v.end());
        for (size_t i = 1; i < v.size(); ++i)
            if (v[i] != v[i - 1] + 1)
                return fail(DAP_BAD_INDEX, "segment " + std::to_string(sg) + " positions are not consecutive and distinct");
    }
    return DAP_OK;
}

int do_inpass(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
              long long n, const int32_t* positions, const int32_t* segments, int32_t n_segments, int32_t seq,
              const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* out, int64_t ld_out, void* ws,
              size_t ws_bytes, hipStream_t s) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(n >= 0, DAP_INVALID_ARG, "counts must be >= 0");
    if (n == 0) return DAP_OK;
    DAP_REQUIRE(n < (1ll << 30), DAP_UNSUPPORTED, "too many tokens for one call");
    DAP_REQUIRE(n_segments > 0 && n_segments <= dap::kMaxInpassSegments, DAP_UNSUPPORTED,
                "in-pass entries take 1 to 4096 segments");
    const InpassLayout L = inpass_layout(h, ws, n, n_segments);
    DAP_REQUIRE((long long)L.capacity * dap::kPage < (1ll << 31), DAP_UNSUPPORTED, "too many tokens for one call");
    DAP_REQUIRE(ws && ws_bytes >= L.bytes && aligned16(ws), DAP_WORKSPACE_TOO_SMALL,
                "workspace must be 16-byte aligned and at least dap_inpass_workspace_bytes()");
    const bool generated = positions == nullptr;     // dap_forward
    if (generated) {
        DAP_REQUIRE(seq <= h->m.max_position, DAP_INVALID_ARG, "seq must be <= the model's max_position");
        dap::LayoutPrep lp;
        lp.mode = dap::kLayoutSpan;
        lp.n_tokens = (int)n;
        lp.per_group = seq;
        lp.base_pos = 0;
        lp.row_map = nullptr;
        lp.positions = L.positions;
        lp.rows = L.segments;
        lp.table = nullptr;
        lp.table_rows = 0;
        lp.table_ld = 0;
        hipError_t e = dap::launch_layout_prep(lp, s, h->profiler());
        if (e != hipSuccess) return hip_fail(e, "index preparation launch");
        positions = L.positions;
        segments = L.segments;
    } else {
        DAP_REQUIRE(aligned4(positions) && segments && aligned4(segments), DAP_INVALID_ARG,
                    "positions and segments must be non-null aligned pointers");
        if (h->validate) {
            std::vector<int32_t> hp, hs;
            if (!to_host(hp, positions, n, s) || !to_host(hs, segments, n, s))
                return fail(DAP_HIP_ERROR, "copying index arrays");
            if (int rc = check_inpass(hp, hs, n_segments)) return rc;
        }
    }
    dap::InpassPrep ip;
    ip.positions = positions;
    ip.segments = segments;
    ip.n_tokens = (int)n;
    ip.n_segments = n_segments;
    ip.table = L.table;
    ip.table_ld = L.table_ld;
    ip.capacity = L.capacity;
    ip.slots = L.slots;
    ip.rel_positions = L.rel;
    ip.seg_lo = L.seg_lo;
    ip.seg_hi = L.seg_hi;
    ip.seg_first = L.seg_first;
    ip.err = h->d_err;
    hipError_t e = dap::launch_inpass_prep(ip, s, h->profiler());
    if (e != hipSuccess) return hip_fail(e, "in-pass preparation launch");
    const int64_t wq = (int64_t)h->m.n_q_heads * h->m.head_dim;
    int rc = do_write(h, q, k, v, ld_in, (int)n, positions, nullptr, L.slots, nullptr, 0, 0, q_gain, k_gain, L.q_rope,
                      wq, L.k_pool, L.v_pool, L.capacity, s);
    if (rc) return rc;
    return do_prefill(h, L.q_rope, wq, (int)n, L.rel, segments, n_segments, L.table, L.table_ld, n_segments,
                      L.k_pool, L.v_pool, L.capacity, out, ld_out, L.prefill,
                      ws_bytes - (size_t)(L.prefill - static_cast<char*>(ws)), s);
}

}  // namespace

extern "C" {

const char* dap_last_error(void) { return g_last_error.c_str(); }

int dap_create(const dap_model* mp, dap_handle** out) {
    DAP_REQUIRE(mp && out, DAP_INVALID_ARG, "null argument");
    *out = nullptr;
    const dap_model& m = *mp;
    DAP_REQUIRE(m.n_q_heads > 0 && m.n_kv_heads > 0 && m.n_q_heads % m.n_kv_heads == 0, DAP_INVALID_ARG,
                "need Hq > 0, Hkv > 0 and Hq % Hkv == 0");
    DAP_REQUIRE(m.n_q_heads / m.n_kv_heads <= 16, DAP_UNSUPPORTED, "Hq / Hkv must be at most 16");
    DAP_REQUIRE(m.head_dim == 64 || m.head_dim == 96 || m.head_dim == 128, DAP_UNSUPPORTED,
                "head_dim must be 64, 96 or 128");
    DAP_REQUIRE(m.page_size == dap::kPage, DAP_UNSUPPORTED, "page_size must be 64");
    DAP_REQUIRE(m.window >= 0, DAP_INVALID_ARG, "window must be >= 0 (0 = none)");
    DAP_REQUIRE(m.max_position > 0, DAP_INVALID_ARG, "max_position must be positive");
    DAP_REQUIRE(m.max_position <= dap::kMaxPosition, DAP_UNSUPPORTED, "max_position must be at most 4194304");
    DAP_REQUIRE(m.rope_theta > 0 && std::isfinite(m.rope_theta), DAP_INVALID_ARG, "rope_theta must be positive");
    if (m.llama3) {
        DAP_REQUIRE(m.llama3_factor > 0 && m.llama3_low_freq_factor > 0 &&
                        m.llama3_high_freq_factor > m.llama3_low_freq_factor && m.llama3_original_max_position > 0,
                    DAP_INVALID_ARG, "llama3 needs factor > 0, high_freq_factor > low_freq_factor > 0, original > 0");
    }
    if (m.qk_norm) DAP_REQUIRE(m.qk_norm_eps > 0, DAP_INVALID_ARG, "qk_norm_eps must be positive");

    dap_handle* h = new (std::nothrow) dap_handle();
    if (!h) return fail(DAP_INVALID_ARG, "out of host memory");
    h->m = m;
    h->group = m.n_q_heads / m.n_kv_heads;
    h->validate = 0;
    {
        const char* env = std::getenv("DAP_FUSED_STEP");
        h->one_pass_step = !(env && env[0] == '0');
    }
    h->d_inv_freq = nullptr;
    h->d_err = nullptr;
    h->prof_state = nullptr;
    h->prof.st = nullptr;
    h->h_inv_freq = build_inv_freq(m);
    h->scratch = nullptr;
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess) e = scratch_address(h->device, &h->scratch);
    if (e == hipSuccess) e = hipMalloc(&h->d_inv_freq, h->h_inv_freq.size() * sizeof(double));
    if (e == hipSuccess) e = hipMalloc(&h->d_err, 256);
    if (e == hipSuccess)
        e = hipMemcpy(h->d_inv_freq, h->h_inv_freq.data(), h->h_inv_freq.size() * sizeof(double), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(h->d_err, 0, 256);
    if (e != hipSuccess) {
        dap_destroy(h);
        return hip_fail(e, "dap_create");
    }
    *out = h;
    return DAP_OK;
}

void dap_destroy(dap_handle* h) {
    if (!h) return;
    delete h->prof_state;
    if (h->d_inv_freq) (void)hipFree(h->d_inv_freq);
    if (h->d_err) (void)hipFree(h->d_err);
    delete h;
}

int dap_set_validate(dap_handle* h, int on) {
    if (int rc = check_handle(h)) return rc;
    h->validate = on ? 1 : 0;
    return DAP_OK;
}

int dap_set_profiling(dap_handle* h, int on) {
    if (int rc = check_handle(h)) return rc;
    if (on && !h->prof_state) {
        auto* st = new (std::nothrow) dap::ProfilerState();
        if (!st) return fail(DAP_INVALID_ARG, "out of host memory");
        hipError_t e = st->init();
        if (e != hipSuccess) {
            delete st;
            return hip_fail(e, "creating timing events");
        }
        h->prof_state = st;
        h->prof.st = st;
    } else if (!on && h->prof_state) {
        while (h->prof_state->count > 0)
            if (h->prof_state->drain_one() != hipSuccess) break;
        delete h->prof_state;
        h->prof_state = nullptr;
        h->prof.st = nullptr;
    }
    return DAP_OK;
}

int dap_profile_read(dap_handle* h, double* total_ms, int64_t* launches, int reset) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(h->prof_state, DAP_INVALID_ARG, "profiling is off");
    dap::ProfilerState* st = h->prof_state;
    while (st->count > 0) {
        hipError_t e = st->drain_one();
        if (e != hipSuccess) return hip_fail(e, "reading timing events");
    }
    for (int k = 0; k < DAP_N_KERNELS; ++k) {
        if (total_ms) total_ms[k] = st->total_ms[k];
        if (launches) launches[k] = st->launches[k];
        if (reset) {
            st->total_ms[k] = 0.0;
            st->launches[k] = 0;
        }
    }
    return DAP_OK;
}

int dap_inv_freq(const dap_handle* h, double* out, int32_t n) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(out && n == (int32_t)h->h_inv_freq.size(), DAP_INVALID_ARG, "n must equal head_dim / 2");
    std::memcpy(out, h->h_inv_freq.data(), n * sizeof(double));
    return DAP_OK;
}

int dap_rope_qknorm_write_pages(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                                int32_t n_tokens, const int32_t* positions, const int32_t* rows, const int32_t* slots,
                                const int32_t* table, int32_t table_ld, int32_t n_table_rows, const uint16_t* q_gain,
                                const uint16_t* k_gain, uint16_t* q_out, int64_t ld_q_out, uint16_t* k_pool,
                                uint16_t* v_pool, int32_t n_pages, void* stream) {
    if (int rc = check_handle(h)) return rc;
    return do_write(h, q, k, v, ld_in, n_tokens, positions, rows, slots, table, table_ld, n_table_rows, q_gain, k_gain,
                    q_out, ld_q_out, k_pool, v_pool, n_pages, static_cast<hipStream_t>(stream));
}

size_t dap_prefill_workspace_bytes(const dap_handle* h, int32_t n_tokens, int32_t n_segments) {
    if (!h || n_tokens < 0 || n_segments < 0) return 0;
    return dap::prefill_workspace(n_tokens, std::max(n_segments, 1), h->group, h->m.head_dim);
}

int dap_attn_prefill_packed(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_tokens, const int32_t* positions,
                            const int32_t* segments, int32_t n_segments, const int32_t* table, int32_t table_ld,
                            int32_t n_table_rows, const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
                            uint16_t* out, int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_handle(h)) return rc;
    return do_prefill(h, q, ld_q, n_tokens, positions, segments, n_segments, table, table_ld, n_table_rows, k_pool,
                      v_pool, n_pages, out, ld_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t dap_decode_workspace_bytes(const dap_handle* h, int32_t n_rows) {
    if (!h || n_rows < 0) return 0;
    return dap::decode_plan(n_rows, h->m.n_q_heads, h->m.n_kv_heads, h->m.head_dim, h->m.window, h->m.max_position)
        .workspace_bytes;
}

int dap_attn_decode_paged(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_rows, const int32_t* positions,
                          const int32_t* rows, const int32_t* table, int32_t table_ld, int32_t n_table_rows,
                          const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages, uint16_t* out,
                          int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_handle(h)) return rc;
    return do_decode(h, q, ld_q, n_rows, positions, rows, table, table_ld, n_table_rows, k_pool, v_pool, n_pages, out,
                     ld_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int dap_attn_decode_paged_noalloc(dap_handle* h, const uint16_t* q, int64_t ld_q, int32_t n_rows,
                                  const int32_t* positions, const int32_t* rows, const int32_t* table,
                                  int32_t table_ld, int32_t n_table_rows, const uint16_t* k_pool,
                                  const uint16_t* v_pool, int32_t n_pages, uint16_t* out, int64_t ld_out,
                                  void* stream) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(h->scratch, DAP_HIP_ERROR, "the handle has no static scratch address");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DAP_REQUIRE(dev == h->device, DAP_INVALID_ARG, "the handle's device must be current");
    DAP_REQUIRE(n_rows >= 0 && n_rows <= dap::kMaxDecodeRows, n_rows < 0 ? DAP_INVALID_ARG : DAP_UNSUPPORTED,
                "n_rows must lie in [0, 65535]");
    const size_t need = dap_decode_workspace_bytes(h, n_rows);
    if (need > kScratchBytes)
        return fail(DAP_WORKSPACE_TOO_SMALL, "the decode's partials for " + std::to_string(n_rows) + " rows need " +
                                                 std::to_string(need) + " bytes, above the static scratch of " +
                                                 std::to_string(kScratchBytes) +
                                                 " bytes; call dap_attn_decode_paged with a workspace");
    return do_decode(h, q, ld_q, n_rows, positions, rows, table, table_ld, n_table_rows, k_pool, v_pool, n_pages, out,
                     ld_out, h->scratch, kScratchBytes, static_cast<hipStream_t>(stream));
}

// Step workspace: the decode's partials, then the prefill's tile list.
size_t dap_step_workspace_bytes(const dap_handle* h, int32_t n_prompt, int32_t n_segments, int32_t n_step) {
    if (!h || n_prompt < 0 || n_step < 0) return 0;
    return align256(dap_decode_workspace_bytes(h, n_step)) + dap_prefill_workspace_bytes(h, n_prompt, n_segments);
}

int dap_step_paged(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                   int32_t n_prompt, int32_t n_segments, int32_t n_step, const int32_t* positions, const int32_t* rows,
                   const int32_t* slots, const int32_t* table, int32_t table_ld, int32_t n_table_rows,
                   const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* q_out, int64_t ld_q_out,
                   uint16_t* k_pool, uint16_t* v_pool, int32_t n_pages, uint16_t* out, int64_t ld_out,
                   void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(n_prompt >= 0 && n_step >= 0, DAP_INVALID_ARG, "counts must be >= 0");
    DAP_REQUIRE(rows && aligned4(rows), DAP_INVALID_ARG, "step_paged needs rows");
    const size_t need = dap_step_workspace_bytes(h, n_prompt, n_segments, n_step);
    DAP_REQUIRE(workspace && workspace_bytes >= need && aligned16(workspace), DAP_WORKSPACE_TOO_SMALL,
                "workspace must be 16-byte aligned and at least dap_step_workspace_bytes()");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t dec_bytes = align256(dap_decode_workspace_bytes(h, n_step));
    char* pre_ws = static_cast<char*>(workspace) + dec_bytes;
    const size_t pre_bytes = workspace_bytes - dec_bytes;
    const uint16_t* q_step = q_out + (int64_t)n_prompt * ld_q_out;
    uint16_t* out_step = out + (int64_t)n_prompt * ld_out;
    dap::WriteArgs wa;
    if (int rc = write_args(h, q, k, v, ld_in, n_prompt + n_step, positions, rows, slots, table, table_ld,
                            n_table_rows, q_gain, k_gain, q_out, ld_q_out, k_pool, v_pool, n_pages, wa, s))
        return rc;
    // With both prompt tokens (up to kOnePassMaxPrompt) and decode rows: the
    // write, then the prompts' tiles and the rows' chunks in one launch.
    // Otherwise in order on `stream`: every token's write, the prompts'
    // prefill, then the decode. A call with no prompt tokens skips the write
    // launch: the decode writes each row's token itself (K, V and q_out,
    // from the workgroup that reads the token's page) before reading it.
    // That needs q_out apart from q (the decode's workgroups read q while
    // q_out is written).
    if (h->one_pass_step && n_prompt > 0 && n_step > 0 && n_prompt <= kOnePassMaxPrompt &&
        (h->group == 1 || h->group == 2 || h->group == 4))
        return do_step_one_pass(h, wa, n_prompt, n_segments, n_step, positions, rows, table, table_ld, n_table_rows,
                                k_pool, v_pool, n_pages, out, ld_out, workspace, dec_bytes, s);
    const bool fused = n_prompt == 0 && n_step > 0 && q_out != q && fuse_decode(h, n_step);
    if (fused && h->validate) {
        std::vector<int32_t> hr;
        if (!to_host(hr, rows, n_step, s)) return fail(DAP_HIP_ERROR, "copying rows");
        std::unordered_set<int32_t> step_rows;
        for (int t = 0; t < n_step; ++t)
            if (!step_rows.insert(hr[t]).second)
                return fail(DAP_BAD_INDEX, "two step tokens in row " + std::to_string(hr[t]));
    }
    dap::WriteArgs wp = wa;
    if (fused) wp.n_tokens = n_prompt;
    int rc = launch_write_checked(h, wp, s);
    if (n_prompt > 0 && rc == DAP_OK)
        rc = do_prefill(h, q_out, ld_q_out, n_prompt, positions, rows, n_segments, table, table_ld, n_table_rows,
                        k_pool, v_pool, n_pages, out, ld_out, pre_ws, pre_bytes, s);
    if (n_step > 0 && rc == DAP_OK) {
        dap::WriteArgs wd = wa;
        wd.q += n_prompt * ld_in;
        wd.k += n_prompt * ld_in;
        wd.v += n_prompt * ld_in;
        wd.positions += n_prompt;
        wd.rows += n_prompt;
        if (wd.slots) wd.slots += n_prompt;
        wd.q_out += n_prompt * ld_q_out;
        wd.n_tokens = n_step;
        rc = do_decode(h, q_step, ld_q_out, n_step, positions + n_prompt, rows + n_prompt, table, table_ld,
                       n_table_rows, k_pool, v_pool, n_pages, out_step, ld_out, workspace, dec_bytes, s,
                       fused ? &wd : nullptr);
    }
    return rc;
}

int dap_tile_layout(int32_t head_dim, int32_t* k_offsets, int32_t* v_offsets) {
    DAP_REQUIRE(head_dim == 64 || head_dim == 96 || head_dim == 128, DAP_UNSUPPORTED, "head_dim must be 64, 96 or 128");
    DAP_REQUIRE(k_offsets && v_offsets, DAP_INVALID_ARG, "null argument");
    for (int key = 0; key < dap::kPage; ++key)
        for (int d = 0; d < head_dim; ++d) {
            k_offsets[key * head_dim + d] = dap::k_tile_offset(key, d, head_dim);
            v_offsets[key * head_dim + d] = dap::v_tile_offset(key, d, head_dim);
        }
    return DAP_OK;
}

size_t dap_cache_workspace_bytes(const dap_handle* h, int32_t n_tokens, int32_t n_groups, int32_t cache_rows,
                                 int32_t max_seq) {
    if (!h || n_tokens < 0 || n_groups < 0 || cache_rows < 0 || max_seq <= 0 || max_seq % dap::kPage) return 0;
    return cache_layout(h, nullptr, n_tokens, std::max(n_groups, 1), cache_rows, max_seq).bytes;
}

int dap_decode(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
               int32_t cache_rows, int32_t pos, int32_t max_seq, const uint16_t* q_gain, const uint16_t* k_gain,
               uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out, void* workspace,
               size_t workspace_bytes, void* stream) {
    return do_cache(h, kCacheDecode, q, k, v, ld_in, cache_rows, 1, pos, nullptr, nullptr, cache_rows, max_seq, q_gain,
                    k_gain, k_pool, v_pool, out, ld_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int dap_decode_rows(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                    int32_t cache_rows, const int32_t* positions, int32_t max_seq, const uint16_t* q_gain,
                    const uint16_t* k_gain, uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return do_cache(h, kCacheDecodeRows, q, k, v, ld_in, cache_rows, 1, 0, positions, nullptr, cache_rows, max_seq,
                    q_gain, k_gain, k_pool, v_pool, out, ld_out, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

int dap_prefill(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                int32_t cache_rows, int32_t seq, int32_t pos, int32_t max_seq, const uint16_t* q_gain,
                const uint16_t* k_gain, uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
                void* workspace, size_t workspace_bytes, void* stream) {
    return do_cache(h, kCachePrefill, q, k, v, ld_in, cache_rows, seq, pos, nullptr, nullptr, cache_rows, max_seq,
                    q_gain, k_gain, k_pool, v_pool, out, ld_out, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

int dap_prefill_slots(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                      int32_t n_prompts, int32_t seq, const int32_t* slots, int32_t cache_rows, int32_t max_seq,
                      const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* k_pool, uint16_t* v_pool,
                      uint16_t* out, int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream) {
    return do_cache(h, kCachePrefillSlots, q, k, v, ld_in, n_prompts, seq, 0, nullptr, slots, cache_rows, max_seq,
                    q_gain, k_gain, k_pool, v_pool, out, ld_out, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

size_t dap_inpass_workspace_bytes(const dap_handle* h, int32_t n_tokens, int32_t n_segments) {
    if (!h || n_tokens < 0 || n_segments <= 0) return 0;
    return inpass_layout(h, nullptr, n_tokens, n_segments).bytes;
}

int dap_packed(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
               int32_t n_tokens, const int32_t* positions, const int32_t* segments, int32_t n_segments,
               const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* out, int64_t ld_out, void* workspace,
               size_t workspace_bytes, void* stream) {
    if (n_tokens > 0 && !positions) return fail(DAP_INVALID_ARG, "positions must be a non-null aligned pointer");
    return do_inpass(h, q, k, v, ld_in, n_tokens, positions, segments, n_segments, 0, q_gain, k_gain, out, ld_out,
                     workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int dap_forward(dap_handle* h, const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
                int32_t n_seqs, int32_t seq, const uint16_t* q_gain, const uint16_t* k_gain, uint16_t* out,
                int64_t ld_out, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_handle(h)) return rc;
    DAP_REQUIRE(n_seqs >= 0 && seq >= 0, DAP_INVALID_ARG, "counts must be >= 0");
    return do_inpass(h, q, k, v, ld_in, (long long)n_seqs * seq, nullptr, nullptr, n_seqs, seq, q_gain, k_gain, out,
                     ld_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
