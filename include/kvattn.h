/*
 * kvattn.h -- exact attention over a block-paged KV cache with Q8_0 keys and
 * Q4_0 values (and the Q8_0/Q8_0, Q4_0/Q4_0 and F16/F16 pairs), on AMD
 * Instinct MI355X (gfx950).
 *
 * What the library computes: for each query row, softmax attention over the
 * complete, logically ordered KV history of a layer.  Where a page lives
 * (resident pool page, caller-placed ring slot, or streamed from the pinned
 * host history through the transfer ring) changes only the physical address
 * the kernels read, never the attended history ("Adaptive KV Streaming for
 * llama.cpp", section "Adaptive KV streaming"; "troed's fork of Raymond's
 * adaptive KV streaming", sections "KV data movement and attention" and
 * "Keep the stock attention order").  Per-split partial softmax results are
 * merged by log-sum-exp in fixed logical order.
 *
 * Conventions (all entry points):
 *   - Every call returns a kvattn_status; nothing aborts.  Unsupported
 *     formats or shapes fail closed with KVATTN_E_UNSUPPORTED; there is no
 *     silent fallback to another format ("troed's fork ...", section
 *     "Required FlashAttention kernels", describes the trap of one).
 *   - A rejected call enqueues no GPU work.
 *   - All device buffers (pool, ring, workspace, q, out) and the pinned host
 *     history are owned by the caller; the library keeps raw pointers and
 *     never frees them.  They must outlive the handle.
 *   - Compute is stream-ordered on the compute stream passed to
 *     kvattn_create; outputs are valid once that stream has passed the call.
 *   - One handle is used by one host thread at a time.
 *   - Streams are passed as hipStream_t values cast to void *.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvattn *kvattn_t;

typedef enum kvattn_status {
    KVATTN_OK = 0,
    KVATTN_E_ARG = -1,         /* null pointer, zero size, W or R out of range, W > n_tokens */
    KVATTN_E_UNSUPPORTED = -2, /* K/V type pair, head_dim, page size or geometry not implemented */
    KVATTN_E_RANGE = -3,       /* layer, pool page or ring slot index out of range */
    KVATTN_E_PLAN = -4,        /* page table with a duplicate physical page, or streamed pages
                                  without a host history, or ring slots mixed with streaming */
    KVATTN_E_NOSPACE = -5,     /* a caller buffer is smaller than the sizes below require */
    KVATTN_E_STATE = -6,       /* call out of order (layer not set, handle destroyed, ...) */
    KVATTN_E_HIP = -7          /* a HIP runtime call failed; kvattn_last_error names it */
} kvattn_status;

/* Cache element types.  Q8_0 and Q4_0: blocks of 32 values with one IEEE
 * binary16 scale d; Q8_0 holds 32 int8 codes c (value d * c), Q4_0 32 4-bit
 * codes n (value d * (n - 8)).  F16: plain IEEE binary16 values.  The pages
 * qualify Q8_0 K / Q4_0 V ("troed's fork ...", section "Adaptive KV Streaming
 * for llama.cpp V2") and require the same-type pairs beside it ("Required
 * FlashAttention kernels"): the supported (k_type, v_type) pairs are
 * (Q8_0, Q4_0), (Q8_0, Q8_0), (Q4_0, Q4_0) and (F16, F16). */
enum { KVATTN_TYPE_F16 = 1, KVATTN_TYPE_Q4_0 = 2, KVATTN_TYPE_Q8_0 = 8 };

/* Page-table entries (one uint32 per logical page):
 *   id < 0x80000000       resident pool page `id`
 *   KVATTN_PT_RING(slot)  a ring slot the caller filled (kvattn_upload_pages)
 *   KVATTN_PT_HOST        not resident: the scheduler streams logical page P
 *                         from page P of the layer's pinned host history into
 *                         a ring slot before the kernels read it. */
#define KVATTN_PT_RING_FLAG 0x80000000u
#define KVATTN_PT_RING(slot) (KVATTN_PT_RING_FLAG | (uint32_t)(slot))
#define KVATTN_PT_HOST 0xFFFFFFFFu

/*
 * Page byte layout (head_dim 128, T = page_tokens, H = n_kv_heads), in
 * order.  A page is T token positions of every KV head of one layer ("troed's
 * fork ...", section "KV data movement and attention": 256 positions per
 * page, K and V page sizes follow the quant types).  The code sections are
 * tiled so that each lane of a 64-wide wavefront reads its matrix-core
 * operand with aligned 16-byte loads.  Below, j is a token's position in the
 * page, t a dimension (0..127), jj = j % 32, and a V key slot is
 * g = (jj % 16) / 4, s = (jj / 16) * 4 + jj % 4.
 *   1. K codes, H*T*kc bytes (kc = 128 for Q8_0, 64 for Q4_0, 256 for F16).
 *      Head h starts at h*T*kc; 16-token tiles of 16*kc bytes.  In a tile:
 *        Q8_0: byte (t/64)*1024 + (((t%32)/8)*16 + j%16)*16 + ((t/32)%2)*8 + t%8.
 *        Q4_0: byte (((t%32)/8)*16 + j%16)*16 + (t/32)*4 + (t%8)%4, the low
 *              nibble for t%8 < 4, else the high nibble.
 *        F16:  bytes (t/32)*1024 + (((t%32)/8)*16 + j%16)*16 + (t%8)*2, +1.
 *   2. K scales (Q8_0, Q4_0 only), binary16 [H][T][4] (one per 32-dim block).
 *   3. V codes, H*T*vc bytes (vc = 128 for Q8_0, 64 for Q4_0, 256 for F16).
 *      Head h starts at h*T*vc; 32-token tiles of 32*vc bytes.  In a tile:
 *        Q4_0: byte (t/64)*1024 + (g*16 + t%16)*16 + ((t/16)%4)*4 + jj%4,
 *              the low nibble for jj < 16, else the high nibble.
 *        Q8_0: byte (t/32)*1024 + (g*16 + t%16)*16 + ((t/16)%2)*8 + s.
 *        F16:  bytes (t/16)*1024 + (g*16 + t%16)*16 + s*2, +1.
 *   4. V scales (Q8_0, Q4_0 only), binary16, H*T*8 bytes.  Head h starts at
 *      h*T*8; 32-token tiles of 256 bytes.  In a tile, token j and block b
 *      have byte (b*4 + (jj%16)/4)*16 + ((jj/16)*4 + jj%4)*2.
 * binary16 values are little-endian.  Page size = H*T*(kc + 8 + vc + 8) for
 * quantised pairs (425,984 at Q8_0/Q4_0, H = 8, T = 256), H*T*512 for F16.
 * Pool pages, ring slots and host-history pages all use this layout, so a
 * host-to-device copy of a page is a plain memcpy.
 */

/* Parameters.  Append-only: new fields go at the end, and struct_size (the
 * caller's sizeof) tells the library which fields the caller knows. */
typedef struct kvattn_params {
    uint32_t struct_size;         /* sizeof(kvattn_params) as compiled by the caller */
    uint32_t n_layers;            /* layers with their own page table (>= 1) */
    uint32_t n_q_heads;           /* query heads; a multiple of n_kv_heads */
    uint32_t n_kv_heads;          /* KV heads; query head h reads KV head h / (n_q_heads / n_kv_heads) */
    uint32_t head_dim;            /* must be 128 */
    uint32_t page_tokens;         /* token positions per page; a multiple of 32 (256 in the workloads) */
    uint32_t k_type;              /* KVATTN_TYPE_*: one of the supported pairs (see above) */
    uint32_t v_type;
    uint32_t n_pool_pages;        /* pages in the resident pool buffer */
    uint32_t n_ring_slots;        /* pages in the ring buffer (0 = no ring) */
    uint32_t max_pages_per_layer; /* upper bound of ceil(n_tokens / page_tokens) */
    uint32_t max_rows;            /* upper bound of W (verify) and R (prefill chunk) */
    float softmax_scale;          /* 0 => 1/sqrt(head_dim) */
    uint32_t split_pages;         /* pages per split for narrow calls (rows per KV head <= 32);
                                     0 => chosen from the page count and the CU count */
    uint32_t chunk_slots;         /* ring slots per streamed chunk (clamped to the ring); 0 => three
                                     eighths of the active ring, at least 1 (24 of 64 slots) */
    uint32_t deterministic;       /* 1 => every call gives the same bits for the same history and
                                     queries (fixed chunk-to-wave order inside a split); 0 =>
                                     narrow calls over resident pages with long splits (>= 96
                                     chunks of 32 keys) let a split's waves claim chunks as their
                                     buffers free up, which balances them but changes the
                                     summation order from run to run (results stay within
                                     rounding of each other) */
} kvattn_params;

/* 1 if the K/V type pair and head_dim are implemented (the four pairs above,
 * head_dim 128), else 0: the capability a backend must advertise truthfully
 * before any attention runs ("troed's fork ...", section "Backend-neutral
 * memory and streaming contracts": the attention operations advertise the
 * supported K/V pairs, and a port advertises only real support). */
int kvattn_supported(uint32_t k_type, uint32_t v_type, uint32_t head_dim);

/* Bytes of one page (0 if the parameters are invalid; the reason is then in
 * kvattn_global_error()), computed from the
 * actual K and V types and the geometry ("troed's fork ...", section
 * "Backend-neutral memory and streaming contracts": page offsets follow the
 * quant types; section "KV data movement and attention": 256-position
 * pages).  No allocation, no GPU work. */
size_t kvattn_page_bytes(const kvattn_params *params);

/* Bytes the caller must provide as d_workspace (0 if the parameters are
 * invalid, the reason in kvattn_global_error()): device page tables, page
 * lists, one staging page, the split partials (m, l, acc[128] per split, row
 * and query head, fp32) and one uint32 per ring slot (the tags of
 * kvattn_debug_check_ring).  The attention operations expose their workspace size beside the span call so
 * the caller can budget it ("troed's fork ...", section "Backend-neutral
 * memory and streaming contracts"; "Adaptive KV Streaming for llama.cpp",
 * section "Batch and micro-batch sizes": a bounded query workspace). */
size_t kvattn_workspace_bytes(const kvattn_params *params);

/*
 * Create a handle: the backend side of the pages' streaming contract, which
 * owns no memory.  It names regions of allocations the caller already made
 * (pool, ring, workspace) without copying them, and supplies what the
 * contract leaves to the backend -- asynchronous host-to-device copies,
 * ready / consumed fences between a copy stream and a compute stream, KV
 * writes and attention over the history ("troed's fork ...", section
 * "Backend-neutral memory and streaming contracts": views of existing
 * allocations, and the backend adapter's copy, fence, write and attention
 * operations).
 * d_pool: n_pool_pages pages (pool_bytes >= that); d_ring: n_ring_slots pages
 * or NULL when n_ring_slots is 0; d_workspace: kvattn_workspace_bytes bytes;
 * all 16-byte aligned device memory, owned by the caller, outliving the
 * handle.  compute_stream runs the kernels; copy_stream runs host-to-device
 * page copies (it may equal compute_stream).  The current HIP device must be
 * the one that owns the buffers.  Errors: KVATTN_E_ARG (null or misaligned
 * buffer, null out), KVATTN_E_UNSUPPORTED / KVATTN_E_RANGE (parameters),
 * KVATTN_E_NOSPACE (a buffer smaller than the parameters need),
 * KVATTN_E_HIP; the message is in kvattn_global_error().  On error *out is
 * NULL and nothing was enqueued.
 */
int kvattn_create(const kvattn_params *params, void *d_pool, size_t pool_bytes, void *d_ring,
                  size_t ring_bytes, void *d_workspace, size_t workspace_bytes, void *compute_stream,
                  void *copy_stream, kvattn_t *out);

/*
 * Place pages: the span copy of the pages' copy-operations table, which
 * enqueues a host-to-device copy of K/V bytes into device slots and fences
 * it for the consumer ("troed's fork ...", section "Backend-neutral memory
 * and streaming contracts": the copy operations and ready / consumed fences;
 * section "KV data movement and attention": a ready fence before a read, a
 * consumed fence before a slot is reused).
 * Copy n pages from host memory h_pages (n * page_bytes, pinned for an
 * asynchronous copy) to the pool pages or ring slots named by dst[i]
 * (pool id, or KVATTN_PT_RING(slot)).  The copy runs on the copy stream,
 * after the compute stream has passed every call enqueued before it (so a
 * page that an earlier call still reads is never overwritten under it);
 * later compute on the compute stream waits for the copy.  h_pages must stay
 * valid until the compute stream has passed the next call.
 */
int kvattn_upload_pages(kvattn_t h, const void *h_pages, const uint32_t *dst, uint32_t n);

/*
 * Set layer `layer`'s history, the pages' span plan: one attention history
 * as logical pages in order, each placed in the pool, a ring slot or the
 * host history, validated so that no physical page serves two logical ones
 * and every logical page up to n_tokens is covered once ("troed's fork ...",
 * section "Backend-neutral memory and streaming contracts": the plan rejects
 * gaps, overlaps and insufficient coverage; a table with one entry per
 * logical page cannot have gaps, and an overlap is a physical page named
 * twice).
 * n_tokens positions in ceil(n_tokens / page_tokens) logical pages,
 * page_table[P] (host memory, read during the call) naming where logical
 * page P lives.  Rejects (KVATTN_E_PLAN) a table that names one physical page
 * twice, names KVATTN_PT_HOST without a host history, or mixes
 * caller-placed ring slots with streamed pages on one handle (the scheduler
 * owns the ring once any page streams).  h_history: the layer's pages in
 * logical order (ceil(n_tokens / page_tokens) pages), read for
 * KVATTN_PT_HOST entries; may be NULL when there are none.  Pinned history
 * (hipHostMalloc) is gathered into ring slots by a copy kernel on the copy
 * stream that reads it over the host link; pageable history is copied with
 * one hipMemcpyAsync per run of consecutive pages (slower).  The table is
 * copied to the device.
 */
int kvattn_set_layer(kvattn_t h, uint32_t layer, const uint32_t *page_table, uint32_t n_tokens,
                     const void *h_history);

/*
 * Attention for W query rows at the tail of the layer's history (positions
 * n_tokens - W .. n_tokens - 1, causal among themselves: row r sees keys
 * 0 .. n_tokens - W + r).  d_q: fp32 [W][n_q_heads][128]; d_out: fp32
 * [W][n_q_heads][128].  Both device memory.  Decode is W = 1
 * (TG1); verify is 1 + the draft length ("troed's fork ...", footnote 1).
 * 1 <= W <= min(max_rows, n_tokens).  On a layer with streamed pages every
 * width runs: each staged span of ring slots is consumed by all row tiles
 * of the call before its slots are released, so a wider call moves no more
 * host-to-device bytes than W = 1 ("Adaptive KV Streaming for llama.cpp",
 * section "Batch and micro-batch sizes"; the second mirror of "troed's fork
 * ...", footnotes: wide verify as consecutive row tiles over one KV span).
 * Asynchronous on the compute stream.  On a layer without streamed pages a
 * call enqueues kernel launches only (no allocation, memset, copy or host
 * wait), so it may be captured into a HIP graph on the compute stream.  On a
 * layer with streamed pages it also enqueues copies and events on the copy
 * stream, driven by the host, and drains both streams when the calls leave
 * the layer order; such calls run eagerly, not under capture.
 */
int kvattn_decode(kvattn_t h, uint32_t layer, const float *d_q, float *d_out);
int kvattn_verify(kvattn_t h, uint32_t layer, const float *d_q, uint32_t W, float *d_out);

/*
 * kvattn_verify without a workspace scratch region, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, result and
 * errors as kvattn_verify, for layers with no streamed pages
 * (KVATTN_E_UNSUPPORTED otherwise).  The split partials go to a static
 * device array of 8 MiB inside the library, one per GPU, held until the
 * process ends; a call whose split plan needs more (split count x W x
 * n_q_heads x 520 bytes, plus alignment: e.g. more than 96 rows per KV head
 * at the workloads' sizes) fails with KVATTN_E_NOSPACE before enqueuing
 * anything.  The call allocates nothing.  Every call on one GPU, from any
 * handle, uses the same array: calls that may run at the same time on one
 * GPU (different streams, or handles on different threads) race and must be
 * ordered by the caller.
 */
int kvattn_verify_noalloc(kvattn_t h, uint32_t layer, const float *d_q, uint32_t W, float *d_out);

/*
 * Prefill chunk: R query rows whose own keys are already the last R
 * positions of the history (row r sees keys 0 .. n_tokens - R + r).  Uses
 * the matrix-core path with splits sized for many rows ("Adaptive KV
 * Streaming for llama.cpp", section "Batch and micro-batch sizes").  Layers
 * with streamed pages run it as above: all row tiles consume each staged
 * span before it is released, with the split partials accumulated into a
 * fixed set of slots (the bounded query workspace of that section).
 * 1 <= R <= min(max_rows, n_tokens).
 */
int kvattn_prefill_chunk(kvattn_t h, uint32_t layer, const float *d_q, uint32_t R, float *d_out);

/*
 * KV writer: quantise R new token rows of `layer` into the page cache and
 * grow the layer's history from n_tokens to n_tokens + R (positions
 * n_tokens .. n_tokens + R - 1).  The writer runs before attention on every
 * decode, verify and prefill step and quantises the new rows into the tail
 * page ("troed's fork ...", section "KV data movement and attention").
 * d_k, d_v: fp32 [R][n_kv_heads][128], device memory, the new keys and
 * values in position order.  K becomes Q8_0: d = amax / 127 rounded to
 * binary16, code = round-half-even(x / d) clamped to [-127, 127], zero scale
 * gives codes 0.  V becomes Q4_0: m = the element of largest magnitude
 * (first on ties, sign kept), d = m / -8 rounded to binary16, code =
 * round-half-even(x / d) + 8 clamped to [0, 15], zero scale gives codes 8.
 * Every decision is taken in binary32 arithmetic.
 * new_pages / n_new: the pool pages (ids < 0x80000000, unused by the layer)
 * for the logical pages the growth adds, ceil((n_tokens + R) / page_tokens)
 * - ceil(n_tokens / page_tokens) of them (else KVATTN_E_ARG); host memory,
 * read during the call.  The pages the new rows land in must be resident
 * (pool pages or caller-placed ring slots): a streamed page there gives
 * KVATTN_E_UNSUPPORTED.  Other bytes of those pages (earlier rows, padding
 * past the new end) are left as they are.
 * h_publish: NULL, or host memory of ceil((n_tokens + R) / page_tokens)
 * pages in logical order (typically the layer's host history): after the
 * write, every page the new rows landed in is copied there (device to host
 * on the compute stream), so a host history stays authoritative.
 * Asynchronous on the compute stream, with no host wait: a call that adds
 * pages writes their device page-table and page-list entries from a launch
 * on the compute stream whose arguments carry them, ahead of the writer, so
 * a call may be captured in a graph (replays rewrite the same entries).  On
 * KVATTN_E_HIP the layer's state is undefined: set it again.
 */
int kvattn_append(kvattn_t h, uint32_t layer, const float *d_k, const float *d_v, uint32_t R,
                  const uint32_t *new_pages, uint32_t n_new, void *h_publish);

/* Completion fence: block the host until both streams have finished the
 * handle's work, so every buffer the handle's calls used may be reused or
 * freed.  Holding a buffer does not prove that queued GPU work stopped using
 * it; only such a fence does ("troed's fork ...", sections "Phase arena" and
 * "Backend-neutral memory and streaming contracts").  KVATTN_E_ARG for a null
 * handle, KVATTN_E_HIP if a stream reports an error. */
int kvattn_synchronize(kvattn_t h);

/*
 * Test aid: copy the bytes of `layer`'s logical page through the kernels'
 * own device-side page resolver into h_out (page_bytes of host memory).
 * Synchronous.  Streamed pages resolve to their most recently assigned
 * ring slot.  It shows the resolver returns the bytes of the logical page
 * wherever the page lives, which is what keeps placement out of the result
 * ("Adaptive KV Streaming for llama.cpp", section "Adaptive KV streaming").
 * Errors: KVATTN_E_RANGE, KVATTN_E_STATE (layer not set), KVATTN_E_ARG.
 */
int kvattn_debug_read_page(kvattn_t h, uint32_t layer, uint32_t logical_page, void *h_out);

/*
 * Test aid: while d_counter is non-NULL (a caller-owned device uint32, zeroed
 * by the caller), the attention kernels of later calls add one to it per
 * softmax re-reference event: a 16-row tile whose running reference exists
 * meets a score more than 8 (log2 units) above it, rescales its accumulators
 * and moves the reference (the online-softmax step that keeps the walk over
 * the ordered history exact, "troed's fork ...", section "Keep the stock
 * attention order").  NULL stops counting.  KVATTN_E_ARG if misaligned.
 */
int kvattn_debug_count_rescales(kvattn_t h, uint32_t *d_counter);

/*
 * Test aid: a device-side check of the streaming schedule's two fences (a
 * ready fence before a chunk is read, a consumed fence before its slots are
 * refilled: "troed's fork ...", section "KV data movement and attention").
 * While d_counters (two caller-owned device uint32, zeroed by the caller) is
 * non-NULL, each ring slot a streamed chunk fills is tagged with the page's
 * global ordinal (plus skew, 0 normally) on the copy stream once its copy
 * has finished, and the tags of the chunk's slots are compared with the
 * ordinals the compute expects on the compute stream just before and just
 * after the launch that reads them: d_counters[0] counts mismatches (a slot
 * read before its copy finished, or refilled before its reader finished),
 * d_counters[1] the slot checks made.  After the second check the chunk's
 * slots are filled with 0xFF bytes (NaN binary16 scales) before its consumed
 * fence, so any read of a recycled slot before its refill makes the output
 * NaN.  A nonzero skew makes every check fail, which shows the check runs.  The call drains both streams and restarts the
 * schedule, so every chunk computed afterwards was copied, and tagged, after
 * it.  NULL stops checking.  KVATTN_E_ARG if misaligned.
 */
int kvattn_debug_check_ring(kvattn_t h, uint32_t *d_counters, uint32_t skew);

/*
 * Host only (no GPU work): the page-table checks kvattn_set_layer applies
 * that need no handle state -- range of pool ids and ring slots, no physical
 * page named twice, streamed pages need a host history (has_history != 0)
 * and a ring, page count within max_pages_per_layer (the span-plan checks of
 * "troed's fork ...", section "Backend-neutral memory and streaming
 * contracts").  Returns the status kvattn_set_layer would return; the
 * message is in kvattn_global_error().
 */
int kvattn_validate_page_table(const kvattn_params *params, const uint32_t *page_table, uint32_t n_tokens,
                               int has_history);

/*
 * Test aid, host only (no GPU work): run the streaming planner (ring slots
 * filled in logical order, a ready fence before compute reads a chunk, a
 * consumed fence before its slots are refilled, prefetch one layer ahead:
 * "troed's fork ...", section "KV data movement and attention") over a
 * sequence of layer calls (call_layers[0 .. n_calls), layers with no streamed
 * pages skipped) for layers whose streamed-page counts are
 * streamed_counts[0 .. n_layers), and log the enqueue sequence the HIP path
 * issues.  Each op is 7 int64 values: kind (1 = copy a chunk on the copy
 * stream after waiting on consumed[wait] when wait >= 0, then record
 * ready[event]; 2 = wait ready[event], compute the chunk, record
 * consumed[event]; 3 = drain both streams; 4 = merge the layer; 5 =
 * compute the layer's resident pages; 6 = the layer's call has begun:
 * copies logged after it may run one streamed layer ahead of it), layer,
 * first and count (the chunk's
 * range of the layer's streamed pages, in logical order), ordinal base
 * (streamed page o sits in ring slot (base + o) mod n_slots), event, wait.
 * ops holds max_ops * 7 values; *n_ops receives the count.
 */
int kvattn_sched_simulate(uint32_t n_layers, uint32_t n_slots, uint32_t chunk_slots, const uint32_t *streamed_counts,
                          const uint32_t *call_layers, uint32_t n_calls, int64_t *ops, uint32_t max_ops,
                          uint32_t *n_ops);

/*
 * Profiling aid (device time per kernel, so a rate is measured rather than
 * read from busy time: "troed's fork ...", section "KV data movement and
 * attention", copy-busy is not bandwidth).  kvattn_profile(h, n) with n > 0
 * brackets each of the next
 * n kernel launches (split or merge) with timing events on the compute
 * stream; n = 0 stops.  kvattn_profile_read waits for the compute stream and
 * returns the summed device time (ms) and launch counts of the split and the
 * merge kernels recorded since kvattn_profile; reset != 0 starts a new count
 * (reset = 0 re-reads the same events, e.g. after each replay of a captured
 * graph that contains them).
 */
int kvattn_profile(kvattn_t h, uint32_t max_launches);
int kvattn_profile_read(kvattn_t h, int reset, double *split_ms, uint32_t *n_split, double *merge_ms,
                        uint32_t *n_merge);

/*
 * Adaptive resident/ring partition ("troed's fork ...", sections "KV data
 * movement and attention" and "Backend-neutral memory and streaming
 * contracts"): when everything fits, every page is resident; under pressure
 * resident pages are traded for ring slots, streaming one or a few whole
 * layers first, more pages as the context grows; the pool/ring split is
 * adjusted with hysteresis from sampled readiness misses, ring occupancy
 * and copy-stream busy time.  kvattn_policy_step is a pure host function:
 * it proposes a split and moves no bytes.  The caller applies a decision by
 * re-placing pages (kvattn_upload_pages, kvattn_set_layer) and sizing the
 * ring (kvattn_set_ring_slots).
 *
 * Feedback rule (the pages name the signals, not the rule):
 *   pressure  = misses / chunks > miss_rate_high with copy_busy < busy_high:
 *               the ring limits prefetch -> grow by ring_step after
 *               grow_after such samples in a row;
 *   saturated = copy_busy >= busy_high: a larger ring cannot help the link,
 *               fewer streamed pages can -> shrink by ring_step after
 *               shrink_after samples in a row;
 *   idle ring = no misses and ring_occupancy < occupancy_low -> shrink after
 *               shrink_after samples in a row.
 * Other samples reset the streaks; the ring stays in [min_ring_slots,
 * min(max_ring_slots, budget_pages - 1)] while anything streams.
 * Residency: the pool gets budget_pages - ring pages; the deficit streams
 * from whole layers in layer order (layer 0 first), one layer possibly in
 * part.
 */
enum { KVATTN_POLICY_FITS = 0,        /* the history fits: all resident, no ring */
       KVATTN_POLICY_HOLD = 1,        /* split unchanged */
       KVATTN_POLICY_CONTEXT = 2,     /* streaming started or the context length changed the residency */
       KVATTN_POLICY_GROW_RING = 3,
       KVATTN_POLICY_SHRINK_RING = 4 };

typedef struct kvattn_policy_config {
    uint32_t n_layers;
    uint32_t page_tokens;
    uint32_t budget_pages;        /* device pages for pool + ring together */
    uint32_t min_ring_slots;      /* >= 1 */
    uint32_t max_ring_slots;      /* >= min_ring_slots */
    uint32_t ring_step;           /* slots added or removed per adjustment (>= 1) */
    uint32_t grow_after;          /* consecutive pressure samples before growing (>= 1) */
    uint32_t shrink_after;        /* consecutive saturated or idle samples before shrinking (>= 1) */
    float miss_rate_high;         /* [0, 1] */
    float busy_high;              /* (0, 1] */
    float occupancy_low;          /* [0, 1] */
} kvattn_policy_config;

typedef struct kvattn_policy_state {  /* zero-initialise before the first step */
    uint32_t ring_slots;
    uint32_t pages_per_layer;
    uint32_t pressure_streak, saturated_streak, idle_streak;
} kvattn_policy_state;

typedef struct kvattn_policy_observation {
    uint32_t n_tokens;            /* current history length (every layer) */
    uint32_t chunks;              /* streamed chunks computed in the sample (0: no feedback) */
    uint32_t ready_misses;        /* of those, chunks whose compute reached the ready fence before the copy ended */
    float ring_occupancy;         /* peak fraction of ring slots holding copied, not yet consumed pages */
    float copy_busy;              /* fraction of the sampled interval the copy stream was copying */
} kvattn_policy_observation;

typedef struct kvattn_policy_decision {
    uint32_t reason;              /* KVATTN_POLICY_* */
    uint32_t changed;             /* 1 if ring size or pages per layer differ from the previous state */
    uint32_t ring_slots;
    uint32_t pages_per_layer;
    uint32_t resident_pages;      /* sum over layers */
    uint32_t streamed_pages;      /* per pass */
    uint32_t streamed_layers;     /* layers with at least one streamed page */
} kvattn_policy_decision;

/* One step: next state, decision, and resident_per_layer[n_layers] (pages of
 * each layer to keep resident).  KVATTN_E_ARG for an invalid config or null
 * pointers, KVATTN_E_NOSPACE when the budget cannot hold one page per layer
 * or a minimal ring beside the pool. */
int kvattn_policy_step(const kvattn_policy_config *config, const kvattn_policy_state *previous,
                       const kvattn_policy_observation *observation, kvattn_policy_state *next,
                       kvattn_policy_decision *decision, uint32_t *resident_per_layer);

/* Observation of streamed calls.  kvattn_observe(h, n) with n > 0 records
 * timing events around the next n streamed chunks (copy start and end on the
 * copy stream; compute reaching the ready fence and finishing the chunk on
 * the compute stream); n = 0 stops.  kvattn_observe_read waits for both
 * streams and fills chunks, ready_misses, ring_occupancy and copy_busy over
 * the recorded chunks (n_tokens is left to the caller); reset != 0 starts a
 * new sample. */
int kvattn_observe(kvattn_t h, uint32_t max_chunks);
int kvattn_observe_read(kvattn_t h, int reset, kvattn_policy_observation *out);

/* Ring slots the scheduler uses from now on (1 .. params.n_ring_slots): how
 * the policy's ring size is applied ("troed's fork ...", section "KV data
 * movement and attention": the resident/ring split is adjusted with
 * hysteresis).  Drains both streams and restarts the streaming schedule;
 * pages of caller-placed ring slots must lie below the new count
 * (KVATTN_E_RANGE otherwise). */
int kvattn_set_ring_slots(kvattn_t h, uint32_t n_slots);

/* Drain both streams (the completion fence above), release the handle's
 * events and free it; the caller's buffers are not touched.  Ending a use of
 * the memory follows the pages' order: drain the work first, then release
 * what held the memory ("troed's fork ...", sections "Phase arena" and
 * "Backend-neutral memory and streaming contracts").  NULL is a no-op;
 * KVATTN_E_HIP if draining failed (the handle is freed anyway). */
int kvattn_destroy(kvattn_t h);

/* Message of the handle's last failed call ("" if none); static text for
 * NULL.  Valid until the next call on the handle.  Failures are reported,
 * never turned into an abort ("Block KV cache streaming ...", maintainer
 * review: a too-small arena must become an error return). */
const char *kvattn_last_error(kvattn_t h);

/* Message of the last failure of a call that had no handle to report on
 * (kvattn_create, the sizing calls, kvattn_validate_page_table,
 * kvattn_sched_simulate, kvattn_policy_step).  Thread-local. */
const char *kvattn_global_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
