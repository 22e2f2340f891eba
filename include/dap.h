/*
 * dap.h -- paged decoder attention core for AMD MI355X (gfx950), C ABI.
 *
 * The attention core of a Llama / Phi-3 / Mistral / Qwen3 decoder layer:
 * pre-rope Q/K/V in, optional per-head QK-RMSNorm, rotary positions
 * (optional llama3 bands), K/V written into a pool of 64-position pages,
 * then causal (optionally windowed) grouped-query attention over each row's
 * pages, for packed prompts and for one decode token per row.
 *
 * Conventions for every call below
 *  - Pointers named q, k, v, qkv, *_pool, out, table, positions, rows,
 *    slots, segments, workspace, *_gain are DEVICE pointers; the model
 *    struct, handle and output arguments of the query functions are host.
 *  - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream) and ordered with other work on that stream. No call
 *    after dap_create allocates, frees or synchronises, except in validate
 *    mode (dap_set_validate), which adds host-side content checks (copies
 *    of the index arrays and a stream synchronisation).
 *  - The caller owns every buffer; the handle owns only its frequency
 *    table and a small device error word.
 *  - Return value: DAP_OK (0) or a negative status; dap_last_error()
 *    returns a thread-local message for the last failure. Nothing aborts
 *    and no C++ exception crosses this boundary.
 *  - Kernels bounds-check every index they read from device memory (page
 *    ids, rows, positions, slots); an out-of-range entry is skipped (its
 *    output left unspecified, no memory outside the buffers touched) and
 *    flagged in the handle's error word, which validate mode reports as
 *    DAP_BAD_INDEX.
 *
 * Page pool layout (bf16), n_pages pages of 64 positions each:
 *   K pool [n_pages][n_kv_heads][64 * head_dim]   one tile per (page, kv head)
 *   V pool [n_pages][n_kv_heads][64 * head_dim]
 * Inside a tile, K[key][d] and V[key][d] sit where dap_tile_layout says:
 * 16-byte chunks (8 dims of one key for K, 8 keys of one dim for V) in the
 * order the decode's waves load them, one contiguous kilobyte per load.
 * Position j of table row r lives in page table[r*table_ld + j/64] at index
 * j%64; its slot number is page*64 + j%64. (The pages: "Mistral 7B Instruct
 * v0.3", Entries table, decode_paged: a pool of positions in pages of
 * PageSize 64, row b's positions in the pages table[b] lists.)
 *
 * Stale slots. A slot that no query of a call attends may hold any bits,
 * NaN and Inf included (what an earlier request left there, or memory never
 * written): it changes no output. ("Phi-3 Mini 4K Instruct" files,
 * src/attention.linnet, prefill_slots: the rest of a row keeps what an
 * earlier request left, since decoding never reads past its own position.)
 * The kernels load whole pages, give such keys weight 0 and set their V
 * elements to 0 before the weighted sum. One qualification: the packed
 * prefill takes the tokens of a run of equal segment ids 32 at a time and
 * clears V only outside such a group's span (its lowest window start to its
 * highest position), so every slot inside the span must hold a finite
 * value. With consecutive positions in each run (prompts and chunks packed
 * end to end) every slot of the span is attended by some token of the
 * group, i.e. it is written history. Pools therefore need no initial
 * state, and the workspaces below may hold anything on entry.
 */
#ifndef DAP_H
#define DAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DAP_OK = 0,
    DAP_INVALID_ARG = -1,          /* bad pointer, count, stride or alignment */
    DAP_UNSUPPORTED = -2,          /* head_dim not 64/96/128, page_size not 64, ... */
    DAP_WORKSPACE_TOO_SMALL = -3,
    DAP_HIP_ERROR = -4,            /* a HIP runtime call failed */
    DAP_BAD_INDEX = -5             /* validate mode: an index array entry out of range */
};

/* Model constants, fixed for a handle's lifetime. */
typedef struct dap_model {
    int32_t n_q_heads;             /* Hq > 0 */
    int32_t n_kv_heads;            /* Hkv > 0, Hq % Hkv == 0, Hq / Hkv <= 16 */
    int32_t head_dim;              /* D: 64, 96 or 128 */
    int32_t page_size;             /* must be 64 */
    int32_t window;                /* 0: none; W > 0: a query at p sees keys p-W < j <= p */
    int32_t max_position;          /* positions lie in [0, max_position), at most 4194304 */
    double rope_theta;             /* rotary base, > 0 */
    int32_t llama3;                /* nonzero: llama3 three-band frequency rescale */
    double llama3_factor;          /* e.g. 8 */
    double llama3_low_freq_factor; /* e.g. 1 */
    double llama3_high_freq_factor;/* e.g. 4 */
    double llama3_original_max_position; /* e.g. 8192 */
    int32_t qk_norm;               /* nonzero: per-head RMSNorm of q and k before rope */
    double qk_norm_eps;            /* e.g. 1e-6 */
} dap_model;

typedef struct dap_handle dap_handle;

/* Build a handle on the current HIP device: checks the constants, builds
 * the frequency table in float64 on the host and uploads it.
 * Frequency table ("Phi-3 Mini 4K Instruct" files, src/rope.linnet, tables):
 * f[i] = theta^(-2i/D), i < D/2. llama3 ("Llama 3.1 8B Instruct", rope
 * scaling paragraph): wavelength 2*pi/f above original/low_freq_factor ->
 * f/factor; below original/high_freq_factor -> f; in between the linear
 * blend (1-s) f/factor + s f with s = (original/wavelength - low_freq_factor)
 * / (high_freq_factor - low_freq_factor). */
int dap_create(const dap_model* model, dap_handle** out);
void dap_destroy(dap_handle* handle);
const char* dap_last_error(void);

/* Validate mode (default off): see the conventions above. */
int dap_set_validate(dap_handle* handle, int on);

/* Copy the handle's float64 frequency table (n must be head_dim/2) to host memory. */
int dap_inv_freq(const dap_handle* handle, double* out, int32_t n);

/*
 * Fused QK-norm + rope + page write.
 * ("Phi-3 Mini 4K Instruct" files, src/attention.linnet: prefill_packed and
 * decode_rows slice the fused projection q, k, v, rope q and k, and write k
 * and v at each token's row and position; "Qwen3-4B": QK-norm of each
 * head's slice before rope; "Mistral 7B Instruct v0.3", Entries:
 * prefill_paged writes each token at its place in the pool.)
 *
 * q, k, v   : token t's Hq*D, Hkv*D and Hkv*D pre-rope values start at
 *             q + t*ld_in, k + t*ld_in, v + t*ld_in (for a fused qkv row:
 *             k = q + Hq*D, v = q + (Hq+Hkv)*D). Head h owns columns
 *             h*D .. h*D+D-1. ld_in >= the widest slice, multiple of 8.
 * positions : [n_tokens] int32, each in [0, max_position).
 * rows      : [n_tokens] int32 table row of each token (ignored if slots).
 * slots     : [n_tokens] int32 pool slot of each token, or NULL to use the
 *             table: slot = table[rows[t]*table_ld + p/64]*64 + p%64.
 *             Slots must be distinct within one call (else which write wins
 *             is unspecified).
 * q_gain, k_gain : [D] bf16 gains, required iff the model has qk_norm.
 * q_out     : [n_tokens][ld_q_out] bf16, roped (and normed) q; may equal q
 *             only if ld_q_out == ld_in.
 * k_pool, v_pool : the pools; roped (and normed) k and raw v are stored at
 *             each token's slot; nothing else in the pools changes.
 * Arithmetic: norm, angle p*f[i], sin/cos and rotation in float64; one
 * round-to-nearest-even to bf16 at the end.
 */
int dap_rope_qknorm_write_pages(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t n_tokens, const int32_t* positions, const int32_t* rows, const int32_t* slots,
    const int32_t* table, int32_t table_ld, int32_t n_table_rows,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* q_out, int64_t ld_q_out,
    uint16_t* k_pool, uint16_t* v_pool, int32_t n_pages, void* stream);

/*
 * Packed prefill over pages.
 * ("Phi-3 Mini 4K Instruct" files, src/attention.linnet: prefill_packed's
 * `own` mask and window_mask; "Mistral 7B Instruct v0.3", Entries:
 * prefill_paged attends each token over its row's pages up to its position.)
 *
 * Token t (row r = segments[t], position p = positions[t]) and query head h:
 *   out[t,h] = sum_{j in J} softmax_j(q[t,h] . K[r, h/g, j] / sqrt(D)) V[r, h/g, j]
 * with J = {j : max(0, p-W+1) <= j <= p} (all j <= p without a window) and
 * g = Hq/Hkv. Keys are read through table row r, so a prompt sees its own
 * row's earlier pages (chunks, shared prefixes) and nothing of other rows.
 * Tokens may come in any order; consecutive tokens with the same segment are
 * processed together (best performance: each prompt's tokens contiguous).
 * q   : [n_tokens][ld_q] bf16 (roped), out : [n_tokens][ld_out] bf16.
 * n_segments : an upper bound on the number of runs of equal consecutive
 *             segment ids (the number of prompts in the pack); it only
 *             sizes the launch.
 * workspace  : device memory of at least dap_prefill_workspace_bytes().
 * bf16 inputs, fp32 MFMA accumulation and softmax, bf16 output.
 */
size_t dap_prefill_workspace_bytes(const dap_handle* handle, int32_t n_tokens, int32_t n_segments);
int dap_attn_prefill_packed(dap_handle* handle,
    const uint16_t* q, int64_t ld_q, int32_t n_tokens,
    const int32_t* positions, const int32_t* segments, int32_t n_segments,
    const int32_t* table, int32_t table_ld, int32_t n_table_rows,
    const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
    uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over pages: one query token per row.
 * ("Mistral 7B Instruct v0.3", Entries: decode_paged is decode_rows over
 * pages; "Phi-3 Mini 4K Instruct" files, src/attention.linnet: decode_rows'
 * `seen` mask.)
 *
 * Row b (table row rows ? rows[b] : b, position p = positions[b]): the same
 * formula as the prefill for its one token. Keys are split into chunks of
 * pages processed in parallel; each chunk keeps a float32 running max,
 * sum and weighted V sum; a row that fits one chunk is finished in the
 * same kernel, the others by a small second kernel that merges the chunks
 * exactly (max-shifted rescale) and rounds to bf16.
 * q : [n_rows][ld_q] bf16 (roped), out : [n_rows][ld_out] bf16.
 * workspace : at least dap_decode_workspace_bytes(handle, n_rows) bytes of
 *             scratch (any contents; one call at a time). n_rows <= 65535.
 */
size_t dap_decode_workspace_bytes(const dap_handle* handle, int32_t n_rows);
int dap_attn_decode_paged(dap_handle* handle,
    const uint16_t* q, int64_t ld_q, int32_t n_rows,
    const int32_t* positions, const int32_t* rows,
    const int32_t* table, int32_t table_ld, int32_t n_table_rows,
    const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
    uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The decode above without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The per-chunk partials go to a static
 * device array of 32 MiB (33554432 bytes) inside the library instead; each
 * GPU the library runs on holds its own copy from the first dap_create on it
 * until the process ends. A call needing more than that
 * (dap_decode_workspace_bytes(handle, n_rows) > 33554432, e.g. 8 rows at
 * max_position 2^22 with 32 query heads) returns DAP_WORKSPACE_TOO_SMALL
 * and launches nothing. Nothing is allocated or freed; no part of the
 * scratch needs clearing (every partial is written before it is read).
 * All calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads, other handles) race and must be ordered by the
 * caller. The handle's device must be current. Arguments and results are as
 * for dap_attn_decode_paged.
 */
int dap_attn_decode_paged_noalloc(dap_handle* handle,
    const uint16_t* q, int64_t ld_q, int32_t n_rows,
    const int32_t* positions, const int32_t* rows,
    const int32_t* table, int32_t table_ld, int32_t n_table_rows,
    const uint16_t* k_pool, const uint16_t* v_pool, int32_t n_pages,
    uint16_t* out, int64_t ld_out, void* stream);

/*
 * One step over pages: packed prompts and one decode token per row in one
 * call. ("Mistral 7B Instruct v0.3", Entries: step_paged is prefill_paged
 * and decode_paged in one pass; "Phi-3 Mini 4K Instruct" files,
 * src/attention.linnet, step_packed: every token's k and v are written
 * first, then the prompts attend and each row's step attends over its row.)
 *
 * Tokens 0..n_prompt-1 are prompt tokens, tokens n_prompt..n_prompt+n_step-1
 * the decode tokens. rows[t] is every token's table row (for prompt tokens
 * also its segment); positions, rows, slots (nullable) cover all tokens.
 * Writes every token first, then runs the packed prefill on the prompt
 * tokens and the decode on the step tokens (q read from q_out), in that
 * order on `stream`; a token may attend slots any token of the call writes.
 * A call with no prompt tokens (a decode step) over a small decode grid
 * has no separate write: the decode writes each row's token (q_out, K, V)
 * itself, before it reads the token's page. Each step token must then have
 * a row of its own (one token per row; validate mode checks it), and q_out
 * must not be q (with q_out == q the call writes first, as above).
 * out : [n_prompt + n_step][ld_out] bf16.
 * workspace : at least dap_step_workspace_bytes() bytes of scratch.
 */
size_t dap_step_workspace_bytes(const dap_handle* handle, int32_t n_prompt, int32_t n_segments,
                                int32_t n_step);
int dap_step_paged(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t n_prompt, int32_t n_segments, int32_t n_step,
    const int32_t* positions, const int32_t* rows, const int32_t* slots,
    const int32_t* table, int32_t table_ld, int32_t n_table_rows,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* q_out, int64_t ld_q_out,
    uint16_t* k_pool, uint16_t* v_pool, int32_t n_pages,
    uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Page tile layout (host only; no device call). Fills, for head_dim D,
 * k_offsets[key * D + d] and v_offsets[key * D + d] (64 * D entries each)
 * with the element offset of logical K[key][d] and V[key][d] inside one
 * (page, kv head) tile. Tiles hold 64 * D bf16 each, 16-byte chunks of 8
 * elements in the order the decode's waves load them (one kilobyte, 64
 * lanes x 16 bytes, per load):
 *   K chunk f*64 + l, f = (h*2 + b)*(D/32) + s, l = 16*g + i:
 *     key 32*h + u(b, i), dims 32*s + 8*g .. +7;
 *   V chunk f*64 + l, f = h*(D/16) + e, l = 16*g + c:
 *     dim 16*e + c, keys 32*h + 8*g .. +7;
 * with u(b, i) = 8*(i/4) + 4*b + i%4. Returns DAP_UNSUPPORTED for D not in
 * {64, 96, 128}.
 */
int dap_tile_layout(int32_t head_dim, int32_t* k_offsets, int32_t* v_offsets);

/*
 * Contiguous-cache entries.
 * ("Phi-3 Mini 4K Instruct" files, src/attention.linnet: decode, prefill,
 * decode_rows and prefill_slots, the entries that keep [Batch, Heads,
 * MaxSeq, D] caches; model card, Entries.)
 *
 * A cache of cache_rows rows and max_seq positions (max_seq a positive
 * multiple of 64) is held as a page pool of cache_rows * max_seq / 64 pages
 * in the layout above, row r owning pages r*max_seq/64 .. (r+1)*max_seq/64-1;
 * k_pool and v_pool are those pools (the caller allocates and keeps them).
 * Each call writes its tokens' roped k and raw v into the cache (as
 * dap_rope_qknorm_write_pages) and returns the attention output of every
 * token (as the paged prefill/decode over that table).
 * q, k, v : the fused projection rows of the call's tokens, [n][ld_in] bf16.
 * q_gain, k_gain : as for the write (required iff the model has QK-norm).
 * out : [n][ld_out] bf16.
 *  dap_decode       : n = cache_rows tokens; token b is row b at position pos.
 *  dap_decode_rows  : n = cache_rows tokens; token b is row b at positions[b]
 *                     (device int32).
 *  dap_prefill      : n = cache_rows * seq tokens; token b*seq+i is row b at
 *                     position pos + i (each row's queries see that row up to
 *                     their own position, earlier calls' keys included).
 *  dap_prefill_slots: n = n_prompts * seq tokens; token m*seq+i is row
 *                     slots[m] (device int32, distinct, < cache_rows) at
 *                     position i, so each prompt sees only itself. Prompts
 *                     shorter than seq are padded by the caller; padding tokens
 *                     are written and attended like the rest, and real tokens
 *                     never see them (they come later).
 * workspace : at least dap_cache_workspace_bytes(handle, n, groups,
 *             cache_rows, max_seq) with groups = 1 for the decodes, cache_rows
 *             for dap_prefill and n_prompts for dap_prefill_slots.
 * Positions must be < min(max_seq, the model's max_position): the scalar pos
 * is checked on the host; device arrays in validate mode, and otherwise by
 * the kernels' bounds checks (out-of-range entries are skipped and flagged).
 */
size_t dap_cache_workspace_bytes(const dap_handle* handle, int32_t n_tokens, int32_t n_groups,
                                 int32_t cache_rows, int32_t max_seq);
int dap_decode(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t cache_rows, int32_t pos, int32_t max_seq,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);
int dap_decode_rows(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t cache_rows, const int32_t* positions, int32_t max_seq,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);
int dap_prefill(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t cache_rows, int32_t seq, int32_t pos, int32_t max_seq,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);
int dap_prefill_slots(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t n_prompts, int32_t seq, const int32_t* slots, int32_t cache_rows, int32_t max_seq,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* k_pool, uint16_t* v_pool, uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * In-pass entries: attention among the call's own tokens, no cache.
 * ("Phi-3 Mini 4K Instruct" files, src/attention.linnet: packed, the
 * training form of prefill_packed with no cache written, and forward, whole
 * sequences from position 0.)
 *
 * dap_packed : token t is position positions[t] of segment segments[t]
 *   (0 <= segments[t] < n_segments <= 4096); it attends to the tokens of its
 *   own segment whose positions are <= its own and within the window. Each
 *   segment's tokens must be one contiguous run of the pack (prompts packed
 *   end to end) and hold consecutive, distinct positions (validate mode
 *   checks both).
 * dap_forward : n_seqs sequences of seq tokens, token b*seq+i at position i
 *   of sequence b.
 * q, k, v : fused projection rows [n][ld_in]; out : [n][ld_out] bf16.
 * The tokens' roped k and v go to scratch pages inside the workspace (at
 * least dap_inpass_workspace_bytes(handle, n, n_segments), n_segments =
 * n_seqs for dap_forward), then the paged prefill runs over them with
 * positions counted from each segment's first position.
 */
size_t dap_inpass_workspace_bytes(const dap_handle* handle, int32_t n_tokens, int32_t n_segments);
int dap_packed(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t n_tokens, const int32_t* positions, const int32_t* segments, int32_t n_segments,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);
int dap_forward(dap_handle* handle,
    const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld_in,
    int32_t n_seqs, int32_t seq,
    const uint16_t* q_gain, const uint16_t* k_gain,
    uint16_t* out, int64_t ld_out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing, for measurement (default off; not one of the pages'
 * operations). While on, every kernel the library launches is bracketed by
 * a pair of hipEvents recorded on its launch stream; dap_profile_read
 * waits for the pending events and reports, per kernel kind, the summed
 * elapsed milliseconds and the number of launches since the last reset.
 * Turning it on creates the events (an allocation: do it outside timed or
 * captured code); at most 1024 launches are kept pending, beyond which the
 * oldest is waited for and folded in.
 */
enum {
    DAP_KERNEL_WRITE = 0,          /* rope_qknorm_write_pages */
    DAP_KERNEL_PREFILL_TILES = 1,  /* the prefill's tile-list pass */
    DAP_KERNEL_PREFILL = 2,        /* the prefill's attention kernel */
    DAP_KERNEL_DECODE = 3,         /* the decode kernel */
    DAP_KERNEL_DECODE_MERGE = 4,   /* the decode's cross-chunk merge */
    DAP_KERNEL_PREP = 5,           /* index preparation of the contiguous and in-pass entries */
    DAP_KERNEL_STEP = 6,           /* step_paged's fused prefill tiles and decode chunks */
    DAP_N_KERNELS = 7
};
int dap_set_profiling(dap_handle* handle, int on);
int dap_profile_read(dap_handle* handle, double* total_ms, int64_t* launches, int reset);

#ifdef __cplusplus
}
#endif

#endif /* DAP_H */
