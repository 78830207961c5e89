// attn_kernels.h -- kernel arguments and launchers shared by the host code.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Page entries that travel with the launch: the first kPrePages entries of
// each of the first kPreSplits splits, so a workgroup's first loads need no
// page-table read (one dependent memory round trip less at the start).
constexpr uint32_t kPreSplits = 64, kPrePages = 4;

struct SplitArgs {
    const uint8_t *pool;          // resident pool pages
    const uint8_t *ring;          // ring slots
    const uint32_t *page_table;   // this layer's device entries (see resolve_page)
    const uint32_t *page_list;    // optional: logical pages, one split each (nullptr = ranges)
    uint32_t list_offset;         // first page_list entry of this launch
    uint32_t n_tokens;            // history length N
    uint32_t n_pages;             // ceil(N / T)
    uint32_t T;                   // tokens per page
    uint32_t W;                   // query rows (positions)
    uint32_t Hq, Hkv, G;          // query heads, KV heads, Hq / Hkv
    uint32_t split_chunks;        // 32-key chunks per split when page_list is null
    uint32_t ring_base;           // ring slot of streamed ordinal 0 (mod n_ring_slots)
    uint32_t n_ring_slots;
    size_t page_bytes;
    size_t sec_kd, sec_vc, sec_vd; // section offsets inside a page
    uint32_t k_type, v_type;      // element types (KVATTN_TYPE_*)
    uint32_t dynamic_order;       // split kernel: waves claim chunks as buffers free (else static order)
    float qscale;                 // softmax_scale * log2(e)
    const float *q;               // [W][Hq][128]
    float *part_o;                // [splits][W*Hq][128]
    float *part_ml;               // [splits][W*Hq][2]
    // split kernel, range splits s < n_pre_splits: pre_entries[s * kPrePages
    // + k] is the device entry of logical page (s * split_chunks * 32) / T + k
    // (0 past the last page); page-list and wide launches set n_pre_splits = 0
    uint32_t n_pre_splits;
    uint32_t pre_entries[kPreSplits * kPrePages];
    // test aid: when non-null, the kernels add one per softmax re-reference
    // event (a row tile moving a reference it already had)
    uint32_t *rescale_count;
    // partial slots (streamed calls of many rows): item i of the launch
    // writes partial slot i (else the split kernel's page-list items write
    // at their logical page); items below accum_slots combine with the
    // partial the slot already holds (log-sum-exp) instead of replacing it
    uint32_t slot_partials;
    uint32_t accum_slots;
};

struct MergeArgs {
    const float *part_o;
    const float *part_ml;
    uint32_t n_splits;
    uint32_t units;               // W * Hq
    uint32_t Hkv, G;              // KV heads, query heads per KV head
    float *out;                   // [W][Hq][128]
};

// Host-to-ring copy of `count` streamed pages: streamed page o (first <= o <
// first + count) is logical page list[o] of the pinned host history and goes
// to ring slot (ring_base + o) mod n_slots.
struct RingCopyArgs {
    const uint8_t *history;       // device-visible address of the layer's pinned host pages
    const uint32_t *list;         // the layer's streamed logical pages, in ordinal order
    uint8_t *ring;
    uint32_t first, count;
    uint32_t ring_base, n_slots;
    size_t page_bytes;
};

// Ring-slot tags (test aid): slot (ring_base + o) mod n_slots of a chunk's
// streamed page o (first <= o < first + count) is tagged with the page's
// global ordinal ord_lo + o (low 32 bits) plus skew when its copy has
// finished, and checked against ord_lo + o around the compute that reads it:
// counter[0] += mismatches, counter[1] += pages checked.
struct RingTagArgs {
    uint32_t *tags;
    uint32_t *counter;
    uint32_t ring_base, ord_lo, first, count, n_slots, skew;
    uint8_t *ring;      // poisoning: the ring and its page size
    size_t page_bytes;
};

// KV writer: quantise R new token rows (positions n_old .. n_old + R - 1) of
// one layer into their pages.  k, v: fp32 [R][Hkv][128].
struct WriterArgs {
    uint8_t *pool;
    uint8_t *ring;
    const uint32_t *page_table;   // the layer's device entries (resident pages only are written)
    const float *k, *v;
    uint32_t n_old, R, T, Hkv;
    uint32_t ring_base, n_ring_slots;
    size_t page_bytes;
    size_t sec_kd, sec_vc, sec_vd;
    uint32_t k_type, v_type;
};

// Device page-table and page-list entries written by a launch whose
// arguments carry their values: no host buffer and no host wait, so it can
// sit in a captured graph.  dst_a[i] = a[i] and, when dst_b is set,
// dst_b[i] = b[i] for i < n <= kTableWriteMax.
constexpr uint32_t kTableWriteMax = 64;
struct TableWriteArgs {
    uint32_t *dst_a, *dst_b;
    uint32_t n;
    uint32_t a[kTableWriteMax], b[kTableWriteMax];
};

size_t kvattn_split_smem_bytes(int rt, uint32_t k_type, uint32_t v_type);
hipError_t kvattn_launch_table_write(const TableWriteArgs &a, hipStream_t s);
hipError_t kvattn_launch_writer(const WriterArgs &a, hipStream_t s);
hipError_t kvattn_launch_ring_copy(const RingCopyArgs &a, hipStream_t s);
// check = false: write the chunk's tags; true: check them
hipError_t kvattn_launch_ring_tag(const RingTagArgs &a, bool check, hipStream_t s);
// fill the chunk's ring slots with 0xFF bytes (binary16 NaN scales)
hipError_t kvattn_launch_ring_poison(const RingTagArgs &a, hipStream_t s);
hipError_t kvattn_split_setup();
uint32_t kvattn_merge_max_splits();
// rt: row tiles of 16 rows per workgroup (1 or 2); n_row_blocks blocks of 16 * rt rows
hipError_t kvattn_launch_split(const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int rt, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Wide calls (> 96 rows per KV head): workgroups of `waves` (8 or 12) waves,
// n_row_blocks blocks of waves * kvattn_wide_rows_per_wave() rows, n_splits
// ranges of split_chunks chunks.
hipError_t kvattn_launch_wide(const SplitArgs &a, uint32_t n_splits, uint32_t n_row_blocks, int waves, hipStream_t s,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
uint32_t kvattn_wide_rows_per_wave();
hipError_t kvattn_launch_merge(const MergeArgs &a, hipStream_t s, hipEvent_t ev_start = nullptr,
                               hipEvent_t ev_stop = nullptr);
hipError_t kvattn_launch_read_page(const SplitArgs &a, uint32_t logical_page, uint8_t *dst, hipStream_t s);
