// kvattn.hip -- C-ABI of the paged Q8_0-K / Q4_0-V attention library.
//
// Host side: argument and page-table validation, the split plan, kernel
// launches, and the single-GPU streaming scheduler that copies non-resident
// pages from the pinned host history into ring slots on a side stream, one
// layer ahead, and recycles each slot once its consumer has run ("troed's
// fork of Raymond's adaptive KV streaming", section "KV data movement and
// attention": ready fence before a read, consumed fence before reuse;
// "Adaptive KV Streaming for llama.cpp", section "Adaptive KV streaming").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <new>
#include <string>
#include <vector>

#include "../../include/kvattn.h"
#include "attn_kernels.h"
#include "policy.h"
#include "sched.h"

namespace {

constexpr uint32_t kHeadDim = 128;
constexpr uint32_t kNarrowRows = 32;      // rows per KV head of one split-kernel workgroup
constexpr uint32_t kNarrowMaxBlocks = 3;  // split-kernel row blocks before the wide kernel takes over
constexpr uint32_t kWideMaxWorkgroups = 256;  // wide calls: workgroups one launch fills (one per compute unit)
constexpr uint32_t kClaimMinChunks = 96;  // splits at least this long use the claimed chunk order
constexpr uint32_t kEntryStream = 0xC0000000u;  // device entry tag: streamed ordinal
constexpr size_t kAlign = 256;

thread_local std::string g_error;

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (kvattn_verify_noalloc): the
// split partials of its calls live in this file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address: kvattn_create takes the address once per device, with
// that device current, from hipGetSymbolAddress.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (`device`), looked up
// on the device's first use.
hipError_t scratch_address(int device, void **out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t page_bytes, sec_kd, sec_vc, sec_vd;
};

bool pair_supported(uint32_t kt, uint32_t vt) {
    return (kt == KVATTN_TYPE_Q8_0 && vt == KVATTN_TYPE_Q4_0) || (kt == KVATTN_TYPE_Q8_0 && vt == KVATTN_TYPE_Q8_0) ||
           (kt == KVATTN_TYPE_Q4_0 && vt == KVATTN_TYPE_Q4_0) || (kt == KVATTN_TYPE_F16 && vt == KVATTN_TYPE_F16);
}

// Code bytes per (token, head) row and scale bytes (4 binary16 block scales;
// none for F16).
size_t code_bytes(uint32_t t) { return t == KVATTN_TYPE_Q8_0 ? kHeadDim : t == KVATTN_TYPE_Q4_0 ? kHeadDim / 2 : 2 * kHeadDim; }
size_t scale_bytes(uint32_t t) { return t == KVATTN_TYPE_F16 ? 0 : 8; }

// Sections of a page: K codes, K scales, V codes, V scales.
Layout page_layout(uint32_t H, uint32_t T, uint32_t kt, uint32_t vt) {
    Layout l;
    l.sec_kd = (size_t)H * T * code_bytes(kt);
    l.sec_vc = l.sec_kd + (size_t)H * T * scale_bytes(kt);
    l.sec_vd = l.sec_vc + (size_t)H * T * code_bytes(vt);
    l.page_bytes = l.sec_vd + (size_t)H * T * scale_bytes(vt);
    return l;
}

Layout page_layout(const kvattn_params &p) { return page_layout(p.n_kv_heads, p.page_tokens, p.k_type, p.v_type); }

// Reads the caller's params honouring struct_size (append-only struct).
bool read_params(const kvattn_params *in, kvattn_params *out) {
    if (!in || in->struct_size < offsetof(kvattn_params, split_pages)) return false;
    std::memset(out, 0, sizeof(*out));
    std::memcpy(out, in, std::min<size_t>(in->struct_size, sizeof(*out)));
    out->struct_size = sizeof(*out);
    return true;
}

int check_params(const kvattn_params &p, std::string &why) {
    if (p.n_layers == 0 || p.n_q_heads == 0 || p.n_kv_heads == 0 || p.max_pages_per_layer == 0 || p.max_rows == 0) {
        why = "n_layers, n_q_heads, n_kv_heads, max_pages_per_layer and max_rows must be >= 1";
        return KVATTN_E_ARG;
    }
    if (!pair_supported(p.k_type, p.v_type)) {
        why = "unsupported K/V element-type pair (supported: Q8_0/Q4_0, Q8_0/Q8_0, Q4_0/Q4_0, F16/F16)";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.head_dim != kHeadDim) {
        why = "only head_dim 128 is implemented";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.page_tokens == 0 || p.page_tokens % 32 != 0) {
        why = "page_tokens must be a positive multiple of 32";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.n_q_heads % p.n_kv_heads != 0) {
        why = "n_q_heads must be a multiple of n_kv_heads";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.n_kv_heads > 65535) {
        why = "n_kv_heads too large";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.max_pages_per_layer > kvattn_merge_max_splits()) {
        why = "max_pages_per_layer exceeds the merge kernel's split capacity (4096 pages)";
        return KVATTN_E_UNSUPPORTED;
    }
    if (p.n_pool_pages >= 0x80000000u || p.n_ring_slots >= 0x40000000u || p.max_pages_per_layer >= 0x40000000u) {
        why = "pool / ring / page counts exceed the page-table encoding";
        return KVATTN_E_RANGE;
    }
    if (!(p.softmax_scale >= 0.f) || std::isinf(p.softmax_scale)) {
        why = "softmax_scale must be finite and >= 0";
        return KVATTN_E_ARG;
    }
    return KVATTN_OK;
}

// Ring slots per streamed chunk for a ring of `ring` slots: the caller's
// chunk_slots, or three eighths of the ring (24 of 64 slots): against 16
// pages per chunk, measured 1.7 % faster at one row, 0.6 % at four and 9 % at
// 49 on the 262,144-token streamed workload (fewer, larger copy and compute
// launches, with still more than two chunks in the ring).
uint32_t chunk_for(const kvattn_params &p, uint32_t ring) {
    const uint32_t chunk = p.chunk_slots ? p.chunk_slots : std::max<uint32_t>(1, ring * 3 / 8);
    return std::max<uint32_t>(1, std::min(chunk, ring));
}

// Partial slots of streamed calls of more than 32 rows per KV head: pages
// per launch, at least the streamed chunk size.
uint32_t stream_slots(const kvattn_params &p) {
    return std::max<uint32_t>(16, chunk_for(p, std::max<uint32_t>(p.n_ring_slots, 1)));
}

// Partial-buffer capacity in (split, row, query head) units.
size_t partial_units(const kvattn_params &p) {
    const uint32_t G = p.n_q_heads / p.n_kv_heads;
    const uint64_t narrow_w = std::min<uint64_t>(p.max_rows, std::max<uint32_t>(1, kNarrowRows / G));
    const uint64_t narrow = (uint64_t)p.max_pages_per_layer * narrow_w * p.n_q_heads;
    // wide calls: splits x row blocks x KV heads <= kWideMaxWorkgroups (or one
    // split), and a row block holds at most 12 waves' rows, so splits x W x Hq
    // stays within kWideMaxWorkgroups such blocks, or W x Hq with one split
    const uint64_t block = 12ull * kvattn_wide_rows_per_wave();
    const uint64_t wide = std::min<uint64_t>((uint64_t)p.max_pages_per_layer * p.max_rows * p.n_q_heads,
                                             std::max<uint64_t>(kWideMaxWorkgroups * block,
                                                                (uint64_t)p.max_rows * p.n_q_heads));
    const uint64_t slotted = p.n_ring_slots ? (uint64_t)stream_slots(p) * p.max_rows * p.n_q_heads : 0;
    return (size_t)std::max(std::max(narrow, wide), slotted);
}

struct WsLayout {
    size_t tables, rlists, slists, staging, part_ml, part_o, ring_tags, total;
};

WsLayout workspace_layout(const kvattn_params &p) {
    WsLayout w;
    const size_t ents = (size_t)p.n_layers * p.max_pages_per_layer * sizeof(uint32_t);
    const size_t units = partial_units(p);
    w.tables = 0;
    w.rlists = align_up(ents);
    w.slists = w.rlists + align_up(ents);
    w.staging = w.slists + align_up(ents);
    w.part_ml = w.staging + align_up(page_layout(p).page_bytes);
    w.part_o = w.part_ml + align_up(units * 2 * sizeof(float));
    w.ring_tags = w.part_o + align_up(units * kHeadDim * sizeof(float));
    w.total = w.ring_tags + align_up((size_t)p.n_ring_slots * sizeof(uint32_t));
    return w;
}

// Planner plus the events the copy and compute streams exchange.
class StreamScheduler : public StreamPlanner {
   public:
    bool init(uint32_t n_layers, uint32_t n_slots, uint32_t chunk) {
        StreamPlanner::init(n_layers, n_slots, chunk);
        ready_.assign(n_events(), nullptr);
        consumed_.assign(n_events(), nullptr);
        for (int i = 0; i < n_events(); i++) {
            if (hipEventCreateWithFlags(&ready_[i], hipEventDisableTiming) != hipSuccess) return false;
            if (hipEventCreateWithFlags(&consumed_[i], hipEventDisableTiming) != hipSuccess) return false;
        }
        return true;
    }
    void destroy() {
        for (hipEvent_t e : ready_)
            if (e) (void)hipEventDestroy(e);
        for (hipEvent_t e : consumed_)
            if (e) (void)hipEventDestroy(e);
        ready_.clear();
        consumed_.clear();
    }
    hipEvent_t ready_event(int i) const { return ready_[i]; }
    hipEvent_t consumed_event(int i) const { return consumed_[i]; }

   private:
    std::vector<hipEvent_t> ready_, consumed_;
};

struct LayerState {
    bool set = false;
    uint32_t n_tokens = 0, n_pages = 0;
    uint32_t n_resident = 0, n_streamed = 0;
    bool uses_ring_slots = false;
    const uint8_t *history = nullptr;
    const uint8_t *history_dev = nullptr;  // device-visible alias when the history is pinned
    std::vector<uint32_t> resident;   // logical pages, ascending
    std::vector<uint32_t> streamed;   // logical pages, ascending (ordinal order)
    std::vector<uint32_t> table;      // the caller's entries, per logical page
    std::vector<uint32_t> dev;        // the device entries, per logical page
};

}  // namespace

struct kvattn {
    kvattn_params p{};
    Layout lay{};
    WsLayout ws{};
    uint8_t *pool = nullptr, *ring = nullptr, *wsp = nullptr;
    size_t pool_bytes = 0, ring_bytes = 0, ws_bytes = 0;
    hipStream_t compute = nullptr, copy = nullptr;
    int device = 0;
    int n_cus = 256;
    hipEvent_t upload_done = nullptr;
    hipEvent_t compute_mark = nullptr;  // compute-stream position uploads wait for
    uint32_t *dbg_rescales = nullptr;   // test aid: re-reference event counter (device)
    uint32_t *dbg_ring = nullptr;       // test aid: ring-slot tag check counters (device, 2 words)
    uint32_t dbg_ring_skew = 0;         // test aid: added to the tags written (0: none)
    void *scratch = nullptr;            // this device's static scratch (kvattn_verify_noalloc)
    hipError_t scratch_err = hipSuccess;
    std::vector<LayerState> layers;
    StreamScheduler sched;
    bool any_streamed = false, any_ring_slots = false;
    uint32_t ring_slots = 0;           // ring slots the scheduler uses (<= p.n_ring_slots)
    // optional observation of streamed chunks: per chunk, copy start / end on
    // the copy stream, compute reaching its ready wait / finishing the chunk
    bool observing = false;
    std::vector<hipEvent_t> obs_ev;    // [4i + 0..3] for chunk i
    std::vector<uint32_t> obs_pages;   // pages of chunk i
    std::vector<uint8_t> obs_marks;    // events recorded for chunk i (bit k: event 4i + k)
    std::map<std::tuple<uint32_t, uint64_t, uint32_t>, size_t> obs_of;  // (layer, ordinal base, first) -> i
    size_t obs_used = 0;
    std::string err;
    float qscale = 0.f;
    // optional per-launch timing of the split and merge kernels
    bool profiling = false;
    std::vector<hipEvent_t> prof_ev;   // pairs: [2i] before, [2i+1] after
    std::vector<uint8_t> prof_kind;    // 0 split, 1 merge
    size_t prof_used = 0;

    uint32_t *d_table(uint32_t layer) { return reinterpret_cast<uint32_t *>(wsp + ws.tables) + (size_t)layer * p.max_pages_per_layer; }
    // per layer: resident logical pages (ascending) and streamed logical
    // pages (ascending, ordinal order), in separate lists so that a grown
    // history appends resident pages without moving the streamed ones
    uint32_t *d_rlist(uint32_t layer) { return reinterpret_cast<uint32_t *>(wsp + ws.rlists) + (size_t)layer * p.max_pages_per_layer; }
    uint32_t *d_slist(uint32_t layer) { return reinterpret_cast<uint32_t *>(wsp + ws.slists) + (size_t)layer * p.max_pages_per_layer; }
    float *part_ml() { return reinterpret_cast<float *>(wsp + ws.part_ml); }
    float *part_o() { return reinterpret_cast<float *>(wsp + ws.part_o); }
    uint32_t *ring_tags() { return reinterpret_cast<uint32_t *>(wsp + ws.ring_tags); }
};

namespace {

int fail(kvattn_t h, int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    if (h)
        h->err = buf;
    else
        g_error = buf;
    return code;
}

#define HIP_TRY(h, call)                                                                            \
    do {                                                                                            \
        hipError_t e_ = (call);                                                                     \
        if (e_ != hipSuccess) return fail((h), KVATTN_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

SplitArgs base_args(kvattn_t h, uint32_t layer, uint32_t W, const float *q) {
    const LayerState &L = h->layers[layer];
    SplitArgs a{};
    a.pool = h->pool;
    a.ring = h->ring;
    a.page_table = h->d_table(layer);
    a.page_list = nullptr;
    a.list_offset = 0;
    a.n_tokens = L.n_tokens;
    a.n_pages = L.n_pages;
    a.T = h->p.page_tokens;
    a.W = W;
    a.Hq = h->p.n_q_heads;
    a.Hkv = h->p.n_kv_heads;
    a.G = h->p.n_q_heads / h->p.n_kv_heads;
    a.split_chunks = h->p.page_tokens / 32;
    a.ring_base = 0;
    a.n_ring_slots = std::max<uint32_t>(1, h->ring_slots);
    a.page_bytes = h->lay.page_bytes;
    a.sec_kd = h->lay.sec_kd;
    a.sec_vc = h->lay.sec_vc;
    a.sec_vd = h->lay.sec_vd;
    a.k_type = h->p.k_type;
    a.v_type = h->p.v_type;
    a.dynamic_order = 0;
    a.qscale = h->qscale;
    a.q = q;
    a.part_o = h->part_o();
    a.part_ml = h->part_ml();
    a.rescale_count = h->dbg_rescales;
    return a;
}

// Split plan of a call on an all-resident layer.  A split is a range of
// 32-key chunks of one KV head.  Narrow calls (rows per KV head <= 32) run
// the split kernel and aim at one workgroup per compute unit (or honour
// split_pages); calls of up to kNarrowMaxBlocks x 32 rows run the split
// kernel on that many 32-row blocks; wider calls (prefill chunks, wide
// verify) run the wide kernel on 256- or 384-row blocks.  Both multi-block
// plans take as many splits as fill the compute units once (at most
// kWideMaxWorkgroups workgroups).  The split count never exceeds the page
// count, which bounds the partial buffer.
struct Plan {
    uint32_t split_chunks, n_splits, n_row_blocks;
    int nrt;         // split kernel: 16-row tiles per workgroup
    bool wide;       // wide kernel
    int wide_waves;  // wide kernel: waves per workgroup (8 or 12)
};

Plan plan_resident(const kvattn_params &p, uint32_t n_tokens, uint32_t n_pages, uint32_t W, int n_cus) {
    const uint32_t G = p.n_q_heads / p.n_kv_heads;
    const uint32_t rows = W * G;
    const uint32_t n_chunks = (n_tokens + 31) / 32;
    const uint32_t cpp = p.page_tokens / 32;
    const uint64_t cus = (uint64_t)std::max(n_cus, 1);
    Plan pl;
    pl.wide_waves = 8;
    pl.wide = rows > kNarrowRows * kNarrowMaxBlocks;
    if (!pl.wide) {
        pl.nrt = rows <= 16 ? 1 : 2;
        pl.n_row_blocks = (rows + kNarrowRows - 1) / kNarrowRows;
        if (p.split_pages && pl.n_row_blocks == 1) {
            pl.split_chunks = p.split_pages * cpp;
        } else {
            // one row block: ceil(CUs / KV heads) splits; more: the row blocks
            // of a split share its keys, and splits x row blocks x KV heads
            // stays within kWideMaxWorkgroups (which bounds the partials)
            uint32_t splits = pl.n_row_blocks == 1
                                  ? (uint32_t)std::max<uint64_t>(1, (cus + p.n_kv_heads - 1) / p.n_kv_heads)
                                  : (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(cus, kWideMaxWorkgroups) /
                                                                        ((uint64_t)p.n_kv_heads * pl.n_row_blocks));
            splits = std::min(splits, n_pages);
            pl.split_chunks = std::max<uint32_t>((n_chunks + splits - 1) / splits, std::min<uint32_t>(8, n_chunks));
        }
    } else {
        pl.nrt = 2;
        // 12-wave workgroups (384-row blocks) run a row about 1.37x as fast as
        // 8-wave ones (256-row blocks, measured on the 1,280-row prefill
        // chunk); take them unless their partly empty last block costs more
        const uint32_t rpw = kvattn_wide_rows_per_wave();
        const uint64_t b8 = (rows + 8 * rpw - 1) / (8 * rpw), b12 = (rows + 12 * rpw - 1) / (12 * rpw);
        pl.wide_waves = b12 * 12 * 100 < b8 * 8 * 137 ? 12 : 8;
        pl.n_row_blocks = (uint32_t)(pl.wide_waves == 12 ? b12 : b8);
        const uint64_t per = (uint64_t)p.n_kv_heads * pl.n_row_blocks;
        const uint64_t slots = std::min<uint64_t>(cus, kWideMaxWorkgroups);
        uint32_t splits = (uint32_t)std::max<uint64_t>(1, slots / per);
        splits = std::min(splits, n_pages);
        pl.split_chunks = (n_chunks + splits - 1) / splits;
    }
    pl.n_splits = (n_chunks + pl.split_chunks - 1) / pl.split_chunks;
    return pl;
}

int validate_call(kvattn_t h, uint32_t layer, const float *q, uint32_t W, const float *out) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (layer >= h->p.n_layers) return fail(h, KVATTN_E_RANGE, "layer %u out of range (n_layers %u)", layer, h->p.n_layers);
    const LayerState &L = h->layers[layer];
    if (!L.set) return fail(h, KVATTN_E_STATE, "layer %u has no history (kvattn_set_layer first)", layer);
    if (!q || !out) return fail(h, KVATTN_E_ARG, "null q or out");
    if (W == 0 || W > h->p.max_rows) return fail(h, KVATTN_E_ARG, "row count %u outside 1..max_rows (%u)", W, h->p.max_rows);
    if (W > L.n_tokens) return fail(h, KVATTN_E_ARG, "row count %u exceeds the history length %u", W, L.n_tokens);
    return KVATTN_OK;
}

// Timing events for the next launch when profiling is on (recorded by the
// dispatch itself at its start and end).
void prof_slot(kvattn_t h, uint8_t kind, hipEvent_t *start, hipEvent_t *stop) {
    *start = *stop = nullptr;
    if (!h->profiling || h->prof_used >= h->prof_kind.size()) return;  // pool full: stop recording
    const size_t slot = h->prof_used++;
    h->prof_kind[slot] = kind;
    *start = h->prof_ev[2 * slot];
    *stop = h->prof_ev[2 * slot + 1];
}

int launch_split(kvattn_t h, const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int nrt) {
    hipEvent_t e0, e1;
    prof_slot(h, 0, &e0, &e1);
    HIP_TRY(h, kvattn_launch_split(a, n_items, n_row_blocks, nrt, h->compute, e0, e1));
    return KVATTN_OK;
}

int launch_wide(kvattn_t h, const SplitArgs &a, uint32_t n_splits, uint32_t n_row_blocks, int waves) {
    hipEvent_t e0, e1;
    prof_slot(h, 0, &e0, &e1);
    HIP_TRY(h, kvattn_launch_wide(a, n_splits, n_row_blocks, waves, h->compute, e0, e1));
    return KVATTN_OK;
}

// Where a call's split partials live: the workspace, or the static scratch
// of the allocation-free entry point.
struct Partials {
    float *o, *ml;
};
Partials workspace_partials(kvattn_t h) { return Partials{h->part_o(), h->part_ml()}; }

int run_merge(kvattn_t h, uint32_t W, uint32_t n_splits, float *out, Partials parts) {
    MergeArgs m;
    m.part_o = parts.o;
    m.part_ml = parts.ml;
    m.n_splits = n_splits;
    m.units = W * h->p.n_q_heads;
    m.Hkv = h->p.n_kv_heads;
    m.G = h->p.n_q_heads / h->p.n_kv_heads;
    m.out = out;
    hipEvent_t e0, e1;
    prof_slot(h, 1, &e0, &e1);
    HIP_TRY(h, kvattn_launch_merge(m, h->compute, e0, e1));
    return KVATTN_OK;
}

int n_cus_of(int device) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v <= 0) v = 256;
    return v;
}

// Attention on a layer without streamed pages: partials, then the merge (a
// separate launch measured cheaper than a device-wide release / counter /
// acquire handshake at the end of the split kernel).
int attend_resident(kvattn_t h, uint32_t layer, const float *q, uint32_t W, float *out, const Plan &pl, Partials parts) {
    const LayerState &L = h->layers[layer];
    SplitArgs a = base_args(h, layer, W, q);
    a.part_o = parts.o;
    a.part_ml = parts.ml;
    a.split_chunks = pl.split_chunks;
    // split kernel: the first page entries of the first splits travel with
    // the launch
    const uint32_t cpp = h->p.page_tokens / 32;
    a.n_pre_splits = pl.wide ? 0u : std::min<uint32_t>(pl.n_splits, kPreSplits);
    for (uint32_t s = 0; s < a.n_pre_splits; s++) {
        const uint32_t p0 = (uint32_t)((uint64_t)s * pl.split_chunks / cpp);
        for (uint32_t k = 0; k < kPrePages; k++)
            a.pre_entries[s * kPrePages + k] = p0 + k < L.n_pages ? L.dev[p0 + k] : 0u;
    }
    // long splits let waves claim chunks (balances them, measured faster);
    // short ones keep the static order, which was as fast or faster there
    a.dynamic_order = (!h->p.deterministic && pl.split_chunks >= kClaimMinChunks) ? 1u : 0u;
    const int rc = pl.wide ? launch_wide(h, a, pl.n_splits, pl.n_row_blocks, pl.wide_waves)
                           : launch_split(h, a, pl.n_splits, pl.n_row_blocks, pl.nrt);
    return rc != KVATTN_OK ? rc : run_merge(h, W, pl.n_splits, out, parts);
}

struct HipExec {
    kvattn_t h;
    uint32_t W;
    const float *q;
    float *out;
    SplitArgs a;
    int nrt;
    // Calls of more than 32 rows per KV head: every launch covers at most
    // `slots` pages, one per split, and item i of a launch accumulates into
    // partial slot i, so the partials stay slots x rows however long the
    // history; each staged ring chunk is read by all row blocks of the call
    // before its consumed fence.  Up to 96 rows per KV head run the split
    // kernel on row_blocks 32-row blocks, more the wide kernel.
    bool slotted = false, wide = false;
    uint32_t slots = 0, n_init = 0, row_blocks = 1;
    int wide_waves = 8;

    int launch_items(uint32_t n_items) {
        a.accum_slots = n_init;
        const int rc = wide ? launch_wide(h, a, n_items, row_blocks, wide_waves)
                            : launch_split(h, a, n_items, row_blocks, nrt);
        n_init = std::max(n_init, n_items);
        return rc;
    }

    int drain() {
        HIP_TRY(h, hipStreamSynchronize(h->copy));
        HIP_TRY(h, hipStreamSynchronize(h->compute));
        return KVATTN_OK;
    }
    int internal(const char *what) { return fail(h, KVATTN_E_STATE, "%s", what); }
    void begin(uint32_t) {}
    // A pinned history is gathered by the ring-copy kernel in one launch;
    // otherwise runs of consecutive logical pages landing in consecutive
    // ring slots become one hipMemcpyAsync each.
    // observation slot of a chunk (its copy and, possibly in a later call,
    // its compute), -1 when not observing or the pool is full
    long obs_slot(const ChunkRef &c, bool for_copy) {
        if (!h->observing) return -1;
        const auto key = std::make_tuple(c.layer, c.ordinal_base, c.first);
        if (for_copy) {
            if (h->obs_used >= h->obs_pages.size()) return -1;
            h->obs_of[key] = h->obs_used;
            h->obs_pages[h->obs_used] = c.count;
            h->obs_marks[h->obs_used] = 0;
            return (long)h->obs_used++;
        }
        auto it = h->obs_of.find(key);
        return it == h->obs_of.end() ? -1 : (long)it->second;
    }
    int obs_record(long ob, int k, hipStream_t s) {
        HIP_TRY(h, hipEventRecord(h->obs_ev[4 * ob + k], s));
        h->obs_marks[ob] |= (uint8_t)(1u << k);
        return KVATTN_OK;
    }

    int copy(const ChunkRef &c) {
        const LayerState &L = h->layers[c.layer];
        if (c.wait_event >= 0) HIP_TRY(h, hipStreamWaitEvent(h->copy, h->sched.consumed_event(c.wait_event), 0));
        const long ob = obs_slot(c, true);
        int rc;
        if (ob >= 0 && (rc = obs_record(ob, 0, h->copy))) return rc;
        if ((rc = copy_pages(c, L))) return rc;
        if (h->dbg_ring && (rc = ring_tags(c, false, h->copy))) return rc;
        if (ob >= 0 && (rc = obs_record(ob, 1, h->copy))) return rc;
        HIP_TRY(h, hipEventRecord(h->sched.ready_event(c.event), h->copy));
        return KVATTN_OK;
    }
    // test aid: write (after its copy) or check (around its compute) the
    // generation tags of the chunk's ring slots
    int ring_tags(const ChunkRef &c, bool check, hipStream_t s) {
        RingTagArgs t;
        t.tags = h->ring_tags();
        t.counter = h->dbg_ring;
        t.ring_base = (uint32_t)(c.ordinal_base % h->ring_slots);
        t.ord_lo = (uint32_t)c.ordinal_base;
        t.first = c.first;
        t.count = c.count;
        t.n_slots = h->ring_slots;
        t.skew = h->dbg_ring_skew;
        t.ring = h->ring;
        t.page_bytes = h->lay.page_bytes;
        HIP_TRY(h, kvattn_launch_ring_tag(t, check, s));
        return KVATTN_OK;
    }
    // test aid: once the chunk's readers are done, poison its slots
    int ring_poison(const ChunkRef &c) {
        RingTagArgs t{};
        t.ring_base = (uint32_t)(c.ordinal_base % h->ring_slots);
        t.first = c.first;
        t.count = c.count;
        t.n_slots = h->ring_slots;
        t.ring = h->ring;
        t.page_bytes = h->lay.page_bytes;
        HIP_TRY(h, kvattn_launch_ring_poison(t, h->compute));
        return KVATTN_OK;
    }
    int copy_pages(const ChunkRef &c, const LayerState &L) {
        const size_t pb = h->lay.page_bytes;
        if (L.history_dev) {
            RingCopyArgs r;
            r.history = L.history_dev;
            r.list = h->d_slist(c.layer);
            r.ring = h->ring;
            r.first = c.first;
            r.count = c.count;
            r.ring_base = (uint32_t)(c.ordinal_base % h->ring_slots);
            r.n_slots = h->ring_slots;
            r.page_bytes = pb;
            HIP_TRY(h, kvattn_launch_ring_copy(r, h->copy));
            return KVATTN_OK;
        }
        uint32_t o = c.first;
        while (o < c.first + c.count) {
            const uint32_t slot = (uint32_t)((c.ordinal_base + o) % h->ring_slots);
            uint32_t run = 1;
            while (o + run < c.first + c.count && L.streamed[o + run] == L.streamed[o] + run && slot + run < h->ring_slots) run++;
            HIP_TRY(h, hipMemcpyAsync(h->ring + (size_t)slot * pb, L.history + (size_t)L.streamed[o] * pb, (size_t)run * pb,
                                      hipMemcpyHostToDevice, h->copy));
            o += run;
        }
        return KVATTN_OK;
    }
    int resident(uint32_t layer) {
        const LayerState &L = h->layers[layer];
        if (!L.n_resident) return KVATTN_OK;
        a.page_list = h->d_rlist(layer);
        a.list_offset = 0;
        if (!slotted) return launch_split(h, a, L.n_resident, 1, nrt);
        for (uint32_t g = 0; g < L.n_resident; g += slots) {
            a.list_offset = g;
            const int rc = launch_items(std::min(slots, L.n_resident - g));
            if (rc) return rc;
        }
        return KVATTN_OK;
    }
    int compute(const ChunkRef &c) {
        const long ob = obs_slot(c, false);
        int rc;
        if (ob >= 0 && (rc = obs_record(ob, 2, h->compute))) return rc;
        HIP_TRY(h, hipStreamWaitEvent(h->compute, h->sched.ready_event(c.event), 0));
        a.page_list = h->d_slist(c.layer);
        a.list_offset = c.first;
        a.ring_base = (uint32_t)(c.ordinal_base % h->ring_slots);
        if (h->dbg_ring && (rc = ring_tags(c, true, h->compute))) return rc;
        if ((rc = slotted ? launch_items(c.count) : launch_split(h, a, c.count, 1, nrt))) return rc;
        if (h->dbg_ring && (rc = ring_tags(c, true, h->compute))) return rc;
        if (h->dbg_ring && (rc = ring_poison(c))) return rc;
        if (ob >= 0 && (rc = obs_record(ob, 3, h->compute))) return rc;
        HIP_TRY(h, hipEventRecord(h->sched.consumed_event(c.event), h->compute));
        return KVATTN_OK;
    }
    int merge(uint32_t layer) {
        return run_merge(h, W, slotted ? n_init : h->layers[layer].n_pages, out, workspace_partials(h));
    }
};

int attend_streamed(kvattn_t h, uint32_t layer, const float *q, uint32_t W, float *out) {
    const uint32_t rows = W * (h->p.n_q_heads / h->p.n_kv_heads);
    HipExec x{h, W, q, out, base_args(h, layer, W, q), rows <= 16 ? 1 : 2};
    x.a.page_list = h->d_rlist(layer);
    if (rows > kNarrowRows) {
        // the same kernels and row blocks as a resident call of this width
        const Plan pl = plan_resident(h->p, h->layers[layer].n_tokens, h->layers[layer].n_pages, W, h->n_cus);
        x.slotted = true;
        x.slots = stream_slots(h->p);
        x.wide = pl.wide;
        x.wide_waves = pl.wide_waves;
        x.row_blocks = pl.n_row_blocks;
        x.nrt = pl.nrt;
        x.a.slot_partials = 1;
    }
    return drive_streamed_layer(h->sched, layer, x);
}

// CPU simulator executor: logs the enqueue sequence.
struct SimExec {
    int64_t *ops;
    uint32_t max_ops, n = 0;
    bool overflow = false;
    void put(int64_t kind, int64_t layer, int64_t first, int64_t count, int64_t base, int64_t ev, int64_t wait) {
        if (n >= max_ops) {
            overflow = true;
            return;
        }
        int64_t *o = ops + (size_t)n * 7;
        o[0] = kind, o[1] = layer, o[2] = first, o[3] = count, o[4] = base, o[5] = ev, o[6] = wait;
        n++;
    }
    int drain() {
        put(3, -1, 0, 0, 0, -1, -1);
        return 0;
    }
    int internal(const char *) { return KVATTN_E_STATE; }
    void begin(uint32_t layer) { put(6, layer, 0, 0, 0, -1, -1); }
    int copy(const ChunkRef &c) {
        put(1, c.layer, c.first, c.count, (int64_t)c.ordinal_base, c.event, c.wait_event);
        return 0;
    }
    int resident(uint32_t layer) {
        put(5, layer, 0, 0, 0, -1, -1);
        return 0;
    }
    int compute(const ChunkRef &c) {
        put(2, c.layer, c.first, c.count, (int64_t)c.ordinal_base, c.event, -1);
        return 0;
    }
    int merge(uint32_t layer) {
        put(4, layer, 0, 0, 0, -1, -1);
        return 0;
    }
};

// Page-table checks of kvattn_set_layer that need no handle state.
int validate_table(kvattn_t h, const kvattn_params &p, const uint32_t *page_table, uint32_t n_tokens, bool has_history,
                   PlanCheck *chk, uint32_t *n_pages_out) {
    if (!page_table || n_tokens == 0) return fail(h, KVATTN_E_ARG, "null page table or zero tokens");
    const uint32_t T = p.page_tokens;
    const uint32_t n_pages = (uint32_t)(((uint64_t)n_tokens + T - 1) / T);
    if (n_pages > p.max_pages_per_layer)
        return fail(h, KVATTN_E_NOSPACE, "%u pages exceed max_pages_per_layer %u", n_pages, p.max_pages_per_layer);
    int rc = check_page_table(page_table, n_pages, p.n_pool_pages, h ? h->ring_slots : p.n_ring_slots, chk);
    if (rc == PT_BAD_POOL) return fail(h, KVATTN_E_RANGE, "page %u: pool page out of range", chk->bad_index);
    if (rc == PT_BAD_RING) return fail(h, KVATTN_E_RANGE, "page %u: ring slot out of range", chk->bad_index);
    if (rc == PT_DUPLICATE)
        return fail(h, KVATTN_E_PLAN, "page %u names a physical page already used by page %u", chk->bad_index, chk->other_index);
    if (chk->n_host && !has_history) return fail(h, KVATTN_E_PLAN, "%u streamed pages but no host history", chk->n_host);
    if (chk->n_host && p.n_ring_slots == 0) return fail(h, KVATTN_E_PLAN, "streamed pages need a ring (n_ring_slots is 0)");
    *n_pages_out = n_pages;
    return KVATTN_OK;
}

int attend(kvattn_t h, uint32_t layer, const float *q, uint32_t W, float *out) {
    int rc = validate_call(h, layer, q, W, out);
    if (rc) return rc;
    const LayerState &L = h->layers[layer];
    if (L.n_streamed) return attend_streamed(h, layer, q, W, out);
    const Plan pl = plan_resident(h->p, L.n_tokens, L.n_pages, W, h->n_cus);
    return attend_resident(h, layer, q, W, out, pl, workspace_partials(h));
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int kvattn_supported(uint32_t k_type, uint32_t v_type, uint32_t head_dim) {
    return pair_supported(k_type, v_type) && head_dim == kHeadDim;
}

// Parameters of the sizing calls, or false with the reason in the thread's
// global error message.
static bool sizing_params(const kvattn_params *params, kvattn_params *p) {
    if (!read_params(params, p)) {
        fail(nullptr, KVATTN_E_ARG, "null params or struct_size too small");
        return false;
    }
    std::string why;
    const int rc = check_params(*p, why);
    if (rc != KVATTN_OK) {
        fail(nullptr, rc, "%s", why.c_str());
        return false;
    }
    return true;
}

size_t kvattn_page_bytes(const kvattn_params *params) {
    kvattn_params p;
    if (!sizing_params(params, &p)) return 0;
    return page_layout(p).page_bytes;
}

size_t kvattn_workspace_bytes(const kvattn_params *params) {
    kvattn_params p;
    if (!sizing_params(params, &p)) return 0;
    return workspace_layout(p).total;
}

int kvattn_create(const kvattn_params *params, void *d_pool, size_t pool_bytes, void *d_ring, size_t ring_bytes,
                  void *d_workspace, size_t workspace_bytes, void *compute_stream, void *copy_stream, kvattn_t *out) {
    if (!out) return fail(nullptr, KVATTN_E_ARG, "null output handle pointer");
    *out = nullptr;
    kvattn_params p;
    if (!read_params(params, &p)) return fail(nullptr, KVATTN_E_ARG, "null params or struct_size too small");
    std::string why;
    int rc = check_params(p, why);
    if (rc) return fail(nullptr, rc, "%s", why.c_str());
    const Layout lay = page_layout(p);
    const WsLayout ws = workspace_layout(p);
    if (p.n_pool_pages && !d_pool) return fail(nullptr, KVATTN_E_ARG, "null pool with n_pool_pages > 0");
    if (p.n_ring_slots && !d_ring) return fail(nullptr, KVATTN_E_ARG, "null ring with n_ring_slots > 0");
    if (!d_workspace) return fail(nullptr, KVATTN_E_ARG, "null workspace");
    if (pool_bytes < (size_t)p.n_pool_pages * lay.page_bytes)
        return fail(nullptr, KVATTN_E_NOSPACE, "pool_bytes %zu < %u pages x %zu", pool_bytes, p.n_pool_pages, lay.page_bytes);
    if (ring_bytes < (size_t)p.n_ring_slots * lay.page_bytes)
        return fail(nullptr, KVATTN_E_NOSPACE, "ring_bytes %zu < %u slots x %zu", ring_bytes, p.n_ring_slots, lay.page_bytes);
    if (workspace_bytes < ws.total)
        return fail(nullptr, KVATTN_E_NOSPACE, "workspace_bytes %zu < required %zu", workspace_bytes, ws.total);
    if ((reinterpret_cast<uintptr_t>(d_pool) | reinterpret_cast<uintptr_t>(d_ring) | reinterpret_cast<uintptr_t>(d_workspace)) & 15)
        return fail(nullptr, KVATTN_E_ARG, "pool, ring and workspace must be 16-byte aligned");

    kvattn *h = new (std::nothrow) kvattn();
    if (!h) return fail(nullptr, KVATTN_E_NOSPACE, "out of host memory");
    h->p = p;
    h->lay = lay;
    h->ws = ws;
    h->pool = static_cast<uint8_t *>(d_pool);
    h->ring = static_cast<uint8_t *>(d_ring);
    h->wsp = static_cast<uint8_t *>(d_workspace);
    h->pool_bytes = pool_bytes;
    h->ring_bytes = ring_bytes;
    h->ws_bytes = workspace_bytes;
    h->compute = static_cast<hipStream_t>(compute_stream);
    h->copy = copy_stream ? static_cast<hipStream_t>(copy_stream) : h->compute;
    const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.0f / std::sqrt((float)kHeadDim);
    h->qscale = scale * 1.4426950408889634f;
    h->layers.resize(p.n_layers);
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->compute_mark, hipEventDisableTiming);
    if (e == hipSuccess) h->n_cus = n_cus_of(h->device);
    // the allocation-free entry point's scratch on this device (a failure
    // is reported by that entry point, not here)
    if (e == hipSuccess) {
        h->scratch_err = scratch_address(h->device, &h->scratch);
        if (h->scratch_err != hipSuccess) (void)hipGetLastError();
    }
    if (e == hipSuccess) e = kvattn_split_setup();
    if (e != hipSuccess) {
        int code = fail(nullptr, KVATTN_E_HIP, "device / event setup failed: %s", hipGetErrorString(e));
        if (h->upload_done) (void)hipEventDestroy(h->upload_done);
        if (h->compute_mark) (void)hipEventDestroy(h->compute_mark);
        delete h;
        return code;
    }
    h->ring_slots = p.n_ring_slots;
    if (p.n_ring_slots) {
        if (!h->sched.init(p.n_layers, p.n_ring_slots, chunk_for(p, p.n_ring_slots))) {
            (void)hipEventDestroy(h->upload_done);
            (void)hipEventDestroy(h->compute_mark);
            delete h;
            return fail(nullptr, KVATTN_E_HIP, "ring event setup failed");
        }
    }
    *out = h;
    return KVATTN_OK;
}

int kvattn_upload_pages(kvattn_t h, const void *h_pages, const uint32_t *dst, uint32_t n) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (n == 0) return KVATTN_OK;
    if (!h_pages || !dst) return fail(h, KVATTN_E_ARG, "null host pages or destination list");
    for (uint32_t i = 0; i < n; i++) {
        uint32_t e = dst[i];
        if (e & KVATTN_PT_RING_FLAG) {
            uint32_t s = e & ~KVATTN_PT_RING_FLAG;
            if (e == KVATTN_PT_HOST || s >= h->ring_slots) return fail(h, KVATTN_E_RANGE, "destination %u: ring slot out of range", i);
            if (h->any_streamed) return fail(h, KVATTN_E_PLAN, "the ring belongs to the streaming scheduler on this handle");
        } else if (e >= h->p.n_pool_pages) {
            return fail(h, KVATTN_E_RANGE, "destination %u: pool page %u out of range (%u pages)", i, e, h->p.n_pool_pages);
        }
    }
    const size_t pb = h->lay.page_bytes;
    const uint8_t *src = static_cast<const uint8_t *>(h_pages);
    // the copies overwrite pages that kernels already enqueued on the compute
    // stream may still read: they start once the compute stream has passed
    // everything enqueued before this call
    if (h->copy != h->compute) {
        HIP_TRY(h, hipEventRecord(h->compute_mark, h->compute));
        HIP_TRY(h, hipStreamWaitEvent(h->copy, h->compute_mark, 0));
    }
    for (uint32_t i = 0; i < n; i++) {
        uint32_t e = dst[i];
        uint8_t *d = (e & KVATTN_PT_RING_FLAG) ? h->ring + (size_t)(e & ~KVATTN_PT_RING_FLAG) * pb : h->pool + (size_t)e * pb;
        HIP_TRY(h, hipMemcpyAsync(d, src + (size_t)i * pb, pb, hipMemcpyHostToDevice, h->copy));
    }
    if (h->copy != h->compute) {
        HIP_TRY(h, hipEventRecord(h->upload_done, h->copy));
        HIP_TRY(h, hipStreamWaitEvent(h->compute, h->upload_done, 0));
    }
    return KVATTN_OK;
}

namespace {
// Install a validated table: drain both streams (copies in flight may read
// the old history or table), rebuild the layer's lists and device tables.
int install_layer(kvattn_t h, uint32_t layer, const uint32_t *page_table, uint32_t n_tokens, uint32_t n_pages,
                  const void *h_history, const PlanCheck &chk) {
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));

    LayerState &L = h->layers[layer];
    L = LayerState();
    L.n_tokens = n_tokens;
    L.n_pages = n_pages;
    L.table.assign(page_table, page_table + n_pages);
    L.history = static_cast<const uint8_t *>(h_history);
    if (h_history && chk.n_host) {
        // pinned (hipHostMalloc) history: the ring-copy kernel reads it in place
        void *dev = nullptr;
        if (hipHostGetDevicePointer(&dev, const_cast<void *>(h_history), 0) == hipSuccess)
            L.history_dev = static_cast<const uint8_t *>(dev);
        else
            (void)hipGetLastError();
    }
    L.uses_ring_slots = chk.n_ring > 0;
    std::vector<uint32_t> dev(n_pages);
    for (uint32_t P = 0; P < n_pages; P++) {
        if (page_table[P] == KVATTN_PT_HOST) {
            dev[P] = kEntryStream | (uint32_t)L.streamed.size();
            L.streamed.push_back(P);
        } else {
            dev[P] = page_table[P];
            L.resident.push_back(P);
        }
    }
    L.n_resident = (uint32_t)L.resident.size();
    L.n_streamed = (uint32_t)L.streamed.size();
    L.dev = dev;
    HIP_TRY(h, hipMemcpy(h->d_table(layer), dev.data(), n_pages * sizeof(uint32_t), hipMemcpyHostToDevice));
    if (L.n_resident)
        HIP_TRY(h, hipMemcpy(h->d_rlist(layer), L.resident.data(), L.n_resident * sizeof(uint32_t), hipMemcpyHostToDevice));
    if (L.n_streamed)
        HIP_TRY(h, hipMemcpy(h->d_slist(layer), L.streamed.data(), L.n_streamed * sizeof(uint32_t), hipMemcpyHostToDevice));
    L.set = true;
    h->any_streamed = false;
    h->any_ring_slots = false;
    std::vector<uint32_t> counts(h->p.n_layers, 0);
    for (uint32_t l = 0; l < h->p.n_layers; l++) {
        h->any_streamed |= h->layers[l].set && h->layers[l].n_streamed > 0;
        h->any_ring_slots |= h->layers[l].set && h->layers[l].uses_ring_slots;
        counts[l] = h->layers[l].set ? h->layers[l].n_streamed : 0;
    }
    if (h->p.n_ring_slots) h->sched.set_layer_counts(counts);
    return KVATTN_OK;
}

void streamed_counts(kvattn_t h, std::vector<uint32_t> &counts) {
    counts.assign(h->p.n_layers, 0);
    for (uint32_t l = 0; l < h->p.n_layers; l++) counts[l] = h->layers[l].set ? h->layers[l].n_streamed : 0;
}
}  // namespace

int kvattn_set_layer(kvattn_t h, uint32_t layer, const uint32_t *page_table, uint32_t n_tokens, const void *h_history) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (layer >= h->p.n_layers) return fail(h, KVATTN_E_RANGE, "layer %u out of range (n_layers %u)", layer, h->p.n_layers);
    PlanCheck chk;
    uint32_t n_pages = 0;
    int rc = validate_table(h, h->p, page_table, n_tokens, h_history != nullptr, &chk, &n_pages);
    if (rc) return rc;
    // the ring is either caller-placed or scheduler-owned on one handle
    bool other_ring = false, other_stream = false;
    for (uint32_t l = 0; l < h->p.n_layers; l++) {
        if (l == layer || !h->layers[l].set) continue;
        other_ring |= h->layers[l].uses_ring_slots;
        other_stream |= h->layers[l].n_streamed > 0;
    }
    if ((chk.n_ring && (chk.n_host || other_stream)) || (chk.n_host && other_ring))
        return fail(h, KVATTN_E_PLAN, "caller-placed ring slots and streamed pages cannot share the ring");

    return install_layer(h, layer, page_table, n_tokens, n_pages, h_history, chk);
}

int kvattn_append(kvattn_t h, uint32_t layer, const float *d_k, const float *d_v, uint32_t R,
                  const uint32_t *new_pages, uint32_t n_new, void *h_publish) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (layer >= h->p.n_layers) return fail(h, KVATTN_E_RANGE, "layer %u out of range (n_layers %u)", layer, h->p.n_layers);
    LayerState &L = h->layers[layer];
    if (!L.set) return fail(h, KVATTN_E_STATE, "layer %u has no history (kvattn_set_layer first)", layer);
    if (!d_k || !d_v || R == 0) return fail(h, KVATTN_E_ARG, "null rows or zero row count");
    const uint32_t T = h->p.page_tokens;
    const uint64_t n_after = (uint64_t)L.n_tokens + R;
    if (n_after > (uint64_t)h->p.max_pages_per_layer * T)
        return fail(h, KVATTN_E_NOSPACE, "%llu tokens exceed max_pages_per_layer x page_tokens", (unsigned long long)n_after);
    const uint32_t pages_after = (uint32_t)((n_after + T - 1) / T);
    const uint32_t need = pages_after - L.n_pages;
    if (n_new != need) return fail(h, KVATTN_E_ARG, "%u rows need %u new pages, %u given", R, need, n_new);
    if (need && !new_pages) return fail(h, KVATTN_E_ARG, "null new_pages");
    for (uint32_t i = 0; i < need; i++)
        if (new_pages[i] & KVATTN_PT_RING_FLAG) return fail(h, KVATTN_E_ARG, "new page %u must be a pool page", i);
    std::vector<uint32_t> table(L.table);
    table.insert(table.end(), new_pages, new_pages + need);
    const uint32_t P0 = L.n_tokens / T, P1 = (uint32_t)((n_after - 1) / T);
    for (uint32_t P = P0; P <= P1; P++)
        if (table[P] == KVATTN_PT_HOST)
            return fail(h, KVATTN_E_UNSUPPORTED, "logical page %u streams from the host; new rows go to resident pages", P);
    const uint32_t n_old = L.n_tokens;
    if (need) {
        PlanCheck chk;
        uint32_t n_pages = 0;
        int rc = validate_table(h, h->p, table.data(), (uint32_t)n_after, L.history != nullptr, &chk, &n_pages);
        if (rc) return rc;
        // the new pages enter the device table and the resident list from
        // launches on the compute stream, ahead of the writer, whose
        // arguments carry the entries: no drain, no host copy, capturable
        const uint32_t old_pages = L.n_pages, old_res = L.n_resident;
        for (uint32_t k = 0; k < need; k += kTableWriteMax) {
            TableWriteArgs tw{};
            tw.n = std::min<uint32_t>(kTableWriteMax, need - k);
            tw.dst_a = h->d_table(layer) + old_pages + k;
            tw.dst_b = h->d_rlist(layer) + old_res + k;
            for (uint32_t i = 0; i < tw.n; i++) {
                tw.a[i] = new_pages[k + i];
                tw.b[i] = old_pages + k + i;
            }
            HIP_TRY(h, kvattn_launch_table_write(tw, h->compute));
        }
        // host mirror of the grown history (the streamed pages and the
        // schedule do not change: the new pages are resident)
        for (uint32_t i = 0; i < need; i++) {
            L.table.push_back(new_pages[i]);
            L.dev.push_back(new_pages[i]);
            L.resident.push_back(old_pages + i);
        }
        L.n_pages = n_pages;
        L.n_resident = (uint32_t)L.resident.size();
    }
    L.n_tokens = (uint32_t)n_after;
    WriterArgs w;
    w.pool = h->pool;
    w.ring = h->ring;
    w.page_table = h->d_table(layer);
    w.k = d_k;
    w.v = d_v;
    w.n_old = n_old;
    w.R = R;
    w.T = T;
    w.Hkv = h->p.n_kv_heads;
    w.ring_base = 0;
    w.n_ring_slots = std::max<uint32_t>(1, h->ring_slots);
    w.page_bytes = h->lay.page_bytes;
    w.sec_kd = h->lay.sec_kd;
    w.sec_vc = h->lay.sec_vc;
    w.sec_vd = h->lay.sec_vd;
    w.k_type = h->p.k_type;
    w.v_type = h->p.v_type;
    HIP_TRY(h, kvattn_launch_writer(w, h->compute));
    if (h_publish) {
        const size_t pb = h->lay.page_bytes;
        for (uint32_t P = P0; P <= P1; P++) {
            const uint32_t e = table[P];
            const uint8_t *src = (e & KVATTN_PT_RING_FLAG) ? h->ring + (size_t)(e & 0x7FFFFFFFu) * pb : h->pool + (size_t)e * pb;
            HIP_TRY(h, hipMemcpyAsync(static_cast<uint8_t *>(h_publish) + (size_t)P * pb, src, pb, hipMemcpyDeviceToHost,
                                      h->compute));
        }
    }
    return KVATTN_OK;
}

int kvattn_decode(kvattn_t h, uint32_t layer, const float *d_q, float *d_out) { return attend(h, layer, d_q, 1, d_out); }

int kvattn_verify(kvattn_t h, uint32_t layer, const float *d_q, uint32_t W, float *d_out) {
    return attend(h, layer, d_q, W, d_out);
}

int kvattn_prefill_chunk(kvattn_t h, uint32_t layer, const float *d_q, uint32_t R, float *d_out) {
    return attend(h, layer, d_q, R, d_out);
}

int kvattn_verify_noalloc(kvattn_t h, uint32_t layer, const float *d_q, uint32_t W, float *d_out) {
    int rc = validate_call(h, layer, d_q, W, d_out);
    if (rc) return rc;
    const LayerState &L = h->layers[layer];
    if (L.n_streamed)
        return fail(h, KVATTN_E_UNSUPPORTED, "kvattn_verify_noalloc needs an all-resident layer (layer %u streams %u pages)",
                    layer, L.n_streamed);
    if (!h->scratch)
        return fail(h, KVATTN_E_HIP, "static scratch address unavailable: %s", hipGetErrorString(h->scratch_err));
    const Plan pl = plan_resident(h->p, L.n_tokens, L.n_pages, W, h->n_cus);
    const size_t units = (size_t)pl.n_splits * W * h->p.n_q_heads;
    const size_t ml_bytes = align_up(units * 2 * sizeof(float));
    const size_t need = ml_bytes + units * kHeadDim * sizeof(float);
    if (need > kScratchBytes)
        return fail(h, KVATTN_E_NOSPACE,
                    "the call's split partials need %zu bytes (%u splits x %u rows x %u query heads), more than the "
                    "static scratch's %zu",
                    need, pl.n_splits, W, h->p.n_q_heads, kScratchBytes);
    uint8_t *base = static_cast<uint8_t *>(h->scratch);
    const Partials parts{reinterpret_cast<float *>(base + ml_bytes), reinterpret_cast<float *>(base)};
    return attend_resident(h, layer, d_q, W, d_out, pl, parts);
}

int kvattn_synchronize(kvattn_t h) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    return KVATTN_OK;
}

int kvattn_debug_read_page(kvattn_t h, uint32_t layer, uint32_t logical_page, void *h_out) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (layer >= h->p.n_layers) return fail(h, KVATTN_E_RANGE, "layer %u out of range", layer);
    if (!h->layers[layer].set) return fail(h, KVATTN_E_STATE, "layer %u has no history", layer);
    if (logical_page >= h->layers[layer].n_pages) return fail(h, KVATTN_E_RANGE, "logical page %u out of range", logical_page);
    if (!h_out) return fail(h, KVATTN_E_ARG, "null output");
    SplitArgs a = base_args(h, layer, 1, nullptr);
    a.ring_base = (uint32_t)(h->sched.last_ordinal_base(layer) % std::max<uint32_t>(1, h->ring_slots));
    uint8_t *staging = h->wsp + h->ws.staging;
    HIP_TRY(h, kvattn_launch_read_page(a, logical_page, staging, h->compute));
    HIP_TRY(h, hipMemcpyAsync(h_out, staging, h->lay.page_bytes, hipMemcpyDeviceToHost, h->compute));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    return KVATTN_OK;
}

int kvattn_debug_count_rescales(kvattn_t h, uint32_t *d_counter) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (reinterpret_cast<uintptr_t>(d_counter) & 3) return fail(h, KVATTN_E_ARG, "counter must be 4-byte aligned");
    h->dbg_rescales = d_counter;
    return KVATTN_OK;
}

int kvattn_profile(kvattn_t h, uint32_t max_launches) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (max_launches == 0) {
        h->profiling = false;
        return KVATTN_OK;
    }
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    if (h->prof_kind.size() < max_launches) {
        for (hipEvent_t e : h->prof_ev) (void)hipEventDestroy(e);
        h->prof_ev.assign(2 * (size_t)max_launches, nullptr);
        h->prof_kind.assign(max_launches, 0);
        for (hipEvent_t &e : h->prof_ev) HIP_TRY(h, hipEventCreate(&e));
    }
    h->prof_used = 0;
    h->profiling = true;
    return KVATTN_OK;
}

int kvattn_profile_read(kvattn_t h, int reset, double *split_ms, uint32_t *n_split, double *merge_ms, uint32_t *n_merge) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (!split_ms || !n_split || !merge_ms || !n_merge) return fail(h, KVATTN_E_ARG, "null output");
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    *split_ms = *merge_ms = 0.0;
    *n_split = *n_merge = 0;
    for (size_t i = 0; i < h->prof_used; i++) {
        float ms = 0.f;
        HIP_TRY(h, hipEventElapsedTime(&ms, h->prof_ev[2 * i], h->prof_ev[2 * i + 1]));
        if (h->prof_kind[i] == 0) {
            *split_ms += ms;
            (*n_split)++;
        } else {
            *merge_ms += ms;
            (*n_merge)++;
        }
    }
    if (reset) h->prof_used = 0;
    return KVATTN_OK;
}

int kvattn_policy_step(const kvattn_policy_config *config, const kvattn_policy_state *previous,
                       const kvattn_policy_observation *observation, kvattn_policy_state *next,
                       kvattn_policy_decision *decision, uint32_t *resident_per_layer) {
    if (!config || !previous || !observation || !next || !decision || !resident_per_layer)
        return fail(nullptr, KVATTN_E_ARG, "null policy argument");
    const int rc = kvattn_policy::step(*config, *previous, *observation, next, decision, resident_per_layer);
    if (rc == KVATTN_E_ARG) return fail(nullptr, rc, "invalid policy config");
    if (rc == KVATTN_E_NOSPACE) return fail(nullptr, rc, "budget too small for one page per layer and a ring");
    return rc;
}

int kvattn_observe(kvattn_t h, uint32_t max_chunks) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    h->obs_used = 0;
    h->obs_of.clear();
    if (max_chunks == 0) {
        h->observing = false;
        return KVATTN_OK;
    }
    if (h->obs_ev.size() < 4 * (size_t)max_chunks) {
        for (hipEvent_t e : h->obs_ev) (void)hipEventDestroy(e);
        h->obs_ev.assign(4 * (size_t)max_chunks, nullptr);
        for (hipEvent_t &e : h->obs_ev) HIP_TRY(h, hipEventCreate(&e));
    }
    h->obs_pages.assign(max_chunks, 0);
    h->obs_marks.assign(max_chunks, 0);
    h->observing = true;
    return KVATTN_OK;
}

// Readiness misses, copy-stream busy fraction and peak ring occupancy over
// the observed chunks (times from timing events, relative to the first copy).
int kvattn_observe_read(kvattn_t h, int reset, kvattn_policy_observation *out) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (!out) return fail(h, KVATTN_E_ARG, "null output");
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    const uint32_t n_tokens = out->n_tokens;
    *out = kvattn_policy_observation{};
    out->n_tokens = n_tokens;
    struct T {
        double cs, ce, reach, done;
        uint32_t pages;
    };
    std::vector<T> t;
    hipEvent_t ref = nullptr;
    for (size_t i = 0; i < h->obs_used; i++)
        if (h->obs_marks[i] & 1u) {
            ref = h->obs_ev[4 * i];
            break;
        }
    double copy_sum = 0.0, lo = 1e300, hi = -1e300;
    for (size_t i = 0; ref && i < h->obs_used; i++) {
        if ((h->obs_marks[i] & 3u) != 3u) continue;
        float a = 0.f, b = 0.f;
        HIP_TRY(h, hipEventElapsedTime(&a, ref, h->obs_ev[4 * i]));
        HIP_TRY(h, hipEventElapsedTime(&b, ref, h->obs_ev[4 * i + 1]));
        copy_sum += b - a;
        lo = std::min(lo, (double)a);
        hi = std::max(hi, (double)b);
        if (h->obs_marks[i] != 15u) continue;  // compute not enqueued yet
        float r = 0.f, d = 0.f;
        HIP_TRY(h, hipEventElapsedTime(&r, ref, h->obs_ev[4 * i + 2]));
        HIP_TRY(h, hipEventElapsedTime(&d, ref, h->obs_ev[4 * i + 3]));
        t.push_back({a, b, r, d, h->obs_pages[i]});
    }
    out->chunks = (uint32_t)t.size();
    for (const T &x : t) out->ready_misses += x.ce > x.reach ? 1u : 0u;
    out->copy_busy = hi > lo ? (float)std::min(1.0, copy_sum / (hi - lo)) : 0.f;
    // peak of pages copied and not yet consumed: sweep the copy-end (+pages)
    // and chunk-done (-pages) times in order, releases first at equal times
    std::vector<std::pair<double, double>> steps;
    steps.reserve(2 * t.size());
    for (const T &x : t) {
        steps.emplace_back(x.ce, (double)x.pages);
        steps.emplace_back(x.done, -(double)x.pages);
    }
    std::sort(steps.begin(), steps.end());
    double peak = 0.0, held = 0.0;
    for (const auto &st : steps) {
        held += st.second;
        peak = std::max(peak, held);
    }
    out->ring_occupancy = h->ring_slots ? (float)std::min(1.0, peak / h->ring_slots) : 0.f;
    if (reset) {
        h->obs_used = 0;
        h->obs_of.clear();
    }
    return KVATTN_OK;
}

int kvattn_debug_check_ring(kvattn_t h, uint32_t *d_counters, uint32_t skew) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (reinterpret_cast<uintptr_t>(d_counters) % 4) return fail(h, KVATTN_E_ARG, "misaligned counters");
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    h->dbg_ring = d_counters;
    h->dbg_ring_skew = d_counters ? skew : 0u;
    // chunks copied from here on carry tags (nothing prefetched survives)
    if (h->p.n_ring_slots) {
        std::vector<uint32_t> counts;
        streamed_counts(h, counts);
        h->sched.set_layer_counts(counts);
    }
    return KVATTN_OK;
}

int kvattn_set_ring_slots(kvattn_t h, uint32_t n_slots) {
    if (!h) return fail(nullptr, KVATTN_E_ARG, "null handle");
    if (n_slots == 0 || n_slots > h->p.n_ring_slots)
        return fail(h, KVATTN_E_RANGE, "ring slots %u outside 1..%u", n_slots, h->p.n_ring_slots);
    for (uint32_t l = 0; l < h->p.n_layers; l++) {
        const LayerState &L = h->layers[l];
        if (!L.set || !L.uses_ring_slots) continue;
        for (uint32_t e : L.table)
            if (e != KVATTN_PT_HOST && (e & KVATTN_PT_RING_FLAG) && (e & ~KVATTN_PT_RING_FLAG) >= n_slots)
                return fail(h, KVATTN_E_RANGE, "layer %u places a page in ring slot %u >= %u", l, e & ~KVATTN_PT_RING_FLAG,
                            n_slots);
    }
    if (n_slots == h->ring_slots) return KVATTN_OK;
    HIP_TRY(h, hipStreamSynchronize(h->copy));
    HIP_TRY(h, hipStreamSynchronize(h->compute));
    h->sched.destroy();
    if (!h->sched.init(h->p.n_layers, n_slots, chunk_for(h->p, n_slots))) return fail(h, KVATTN_E_HIP, "ring event setup failed");
    std::vector<uint32_t> counts;
    streamed_counts(h, counts);
    h->sched.set_layer_counts(counts);
    h->ring_slots = n_slots;
    h->obs_of.clear();  // chunk keys of the old schedule
    h->obs_used = 0;
    return KVATTN_OK;
}

int kvattn_destroy(kvattn_t h) {
    if (!h) return KVATTN_OK;
    int rc = KVATTN_OK;
    if (hipStreamSynchronize(h->copy) != hipSuccess) rc = KVATTN_E_HIP;
    if (hipStreamSynchronize(h->compute) != hipSuccess) rc = KVATTN_E_HIP;
    h->sched.destroy();
    if (h->upload_done) (void)hipEventDestroy(h->upload_done);
    if (h->compute_mark) (void)hipEventDestroy(h->compute_mark);
    for (hipEvent_t e : h->prof_ev)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : h->obs_ev)
        if (e) (void)hipEventDestroy(e);
    delete h;
    return rc;
}

const char *kvattn_last_error(kvattn_t h) { return h ? h->err.c_str() : "null handle"; }

const char *kvattn_global_error(void) { return g_error.c_str(); }

/* Host only: the checks kvattn_set_layer applies to a page table that need
 * no handle state (see the header). */
int kvattn_validate_page_table(const kvattn_params *params, const uint32_t *page_table, uint32_t n_tokens, int has_history) {
    kvattn_params p;
    if (!read_params(params, &p)) return fail(nullptr, KVATTN_E_ARG, "null params or struct_size too small");
    std::string why;
    int rc = check_params(p, why);
    if (rc) return fail(nullptr, rc, "%s", why.c_str());
    PlanCheck chk;
    uint32_t n_pages = 0;
    return validate_table(nullptr, p, page_table, n_tokens, has_history != 0, &chk, &n_pages);
}

/* Test aid (host only, no GPU): run the streaming planner over a sequence of
 * layer calls and log the enqueue sequence the HIP path would issue.  Each op
 * is 7 int64: kind (1 copy, 2 compute, 3 drain, 4 merge, 5 resident pages,
 * 6 layer begun),
 * layer, first, count, ordinal base, event, wait event. */
int kvattn_sched_simulate(uint32_t n_layers, uint32_t n_slots, uint32_t chunk_slots, const uint32_t *streamed_counts,
                          const uint32_t *call_layers, uint32_t n_calls, int64_t *ops, uint32_t max_ops, uint32_t *n_ops) {
    if (!streamed_counts || !call_layers || !ops || !n_ops || n_layers == 0 || n_slots == 0)
        return fail(nullptr, KVATTN_E_ARG, "null argument, or no layers or no ring slots");
    StreamPlanner pl;
    pl.init(n_layers, n_slots, chunk_slots ? std::min(chunk_slots, n_slots) : std::max<uint32_t>(1, n_slots * 3 / 8));
    pl.set_layer_counts(std::vector<uint32_t>(streamed_counts, streamed_counts + n_layers));
    SimExec x{ops, max_ops};
    for (uint32_t i = 0; i < n_calls; i++) {
        if (call_layers[i] >= n_layers)
            return fail(nullptr, KVATTN_E_RANGE, "call %u names layer %u of %u", i, call_layers[i], n_layers);
        if (streamed_counts[call_layers[i]] == 0) continue;
        int rc = drive_streamed_layer(pl, call_layers[i], x);
        if (rc) return fail(nullptr, rc, "the planner failed on call %u (layer %u)", i, call_layers[i]);
    }
    *n_ops = x.n;
    if (x.overflow) return fail(nullptr, KVATTN_E_NOSPACE, "more than max_ops (%u) operations", max_ops);
    return KVATTN_OK;
}

}  // extern "C"
