// sched.h -- page-table validation and the ring streaming planner.
//
// The planner is pure host logic (no HIP calls) so that it can be driven on
// the CPU by a simulator; the HIP path pairs it with the pools of ready and
// consumed events that the copy and compute streams exchange.
//
// Streaming model ("troed's fork of Raymond's adaptive KV streaming", section
// "KV data movement and attention"): every streamed layer's non-resident
// pages, in logical order, get consecutive global ordinals; ordinal x lives in
// ring slot x mod n_slots.  A layer's streamed pages are cut into chunks of
// at most chunk_slots pages, so a chunk occupies one or two contiguous slot
// spans (before and after the wrap).  For each chunk:
//   copy stream:    wait consumed(predecessor) -> H2D copies -> record ready
//   compute stream: wait ready -> split kernel -> record consumed
// where the predecessor is the chunk that last held the newest slot the
// chunk overwrites (waiting on it covers all older holders, since the
// compute stream is in order).  A copy is enqueued only after its
// predecessor's consumed fence has been recorded, and never for a layer more
// than one streamed layer ahead of the layer being computed.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <vector>

enum { PT_OK = 0, PT_BAD_POOL = 1, PT_BAD_RING = 2, PT_DUPLICATE = 3 };

struct PlanCheck {
    uint32_t n_pool = 0, n_ring = 0, n_host = 0;
    uint32_t bad_index = 0, other_index = 0;
};

// Validates one layer's page table: pool ids in range, ring slots in range,
// no physical page named twice.  Host entries (0xFFFFFFFF) are counted.
inline int check_page_table(const uint32_t *pt, uint32_t n_pages, uint32_t n_pool, uint32_t n_ring, PlanCheck *out) {
    PlanCheck c;
    for (uint32_t P = 0; P < n_pages; P++) {
        const uint32_t e = pt[P];
        if (e == 0xFFFFFFFFu) {
            c.n_host++;
        } else if (e & 0x80000000u) {
            const uint32_t s = e & 0x7FFFFFFFu;
            if (s >= n_ring) { c.bad_index = P; *out = c; return PT_BAD_RING; }
            c.n_ring++;
        } else {
            if (e >= n_pool) { c.bad_index = P; *out = c; return PT_BAD_POOL; }
            c.n_pool++;
        }
    }
    // duplicate detection: sort (physical key, logical index) pairs
    std::vector<uint64_t> keys;
    keys.reserve(n_pages);
    for (uint32_t P = 0; P < n_pages; P++)
        if (pt[P] != 0xFFFFFFFFu) keys.push_back(((uint64_t)pt[P] << 32) | P);
    std::sort(keys.begin(), keys.end());
    for (size_t i = 1; i < keys.size(); i++)
        if ((keys[i] >> 32) == (keys[i - 1] >> 32)) {
            c.bad_index = (uint32_t)keys[i];
            c.other_index = (uint32_t)keys[i - 1];
            *out = c;
            return PT_DUPLICATE;
        }
    *out = c;
    return PT_OK;
}

struct ChunkRef {
    uint32_t layer = 0;
    uint32_t first = 0, count = 0;   // range of the layer's streamed-page indices
    uint64_t ordinal_base = 0;       // global ordinal of the layer's streamed page 0
    int event = 0;                   // index of this chunk's ready / consumed events
    int wait_event = -1;             // consumed event the copy waits on (-1 = none)
};

class StreamPlanner {
   public:
    void init(uint32_t n_layers, uint32_t n_slots, uint32_t chunk) {
        n_layers_ = n_layers;
        n_slots_ = n_slots ? n_slots : 1;
        chunk_ = chunk ? (chunk < n_slots_ ? chunk : n_slots_) : 1;
        n_events_ = 2 * (int)n_slots_ + 4;
        counts_.assign(n_layers, 0);
        last_base_.assign(n_layers, 0);
        ordinal_ = 0;
        restart_at(0);
    }
    int n_events() const { return n_events_; }
    uint32_t n_slots() const { return n_slots_; }

    void set_layer_counts(const std::vector<uint32_t> &counts) {
        counts_ = counts;
        restart_at(0);
    }

    // Compute side.  Returns false when `layer` is not the streamed layer the
    // schedule expects next; the caller then drains both streams and calls
    // restart(layer).
    bool begin_layer(uint32_t layer) {
        if (layer >= n_layers_ || counts_[layer] == 0) return false;
        if (!started_) restart(layer);
        if (seq_layer(compute_seq_) != layer) return false;
        next_compute_chunk_ = 0;
        active_seq_ = compute_seq_;
        return true;
    }
    void restart(uint32_t layer) {
        restart_at(layer);
        started_ = true;
    }
    bool next_compute(uint32_t layer, ChunkRef *out) {
        const uint32_t first = next_compute_chunk_ * chunk_;
        if (layer >= n_layers_ || first >= counts_[layer]) return false;
        for (const Rec &r : recs_)
            if (r.seq == compute_seq_ && r.ref.first == first) {
                *out = r.ref;
                next_compute_chunk_++;
                return true;
            }
        return false;  // copy not planned: cannot happen after next_copy ran dry
    }
    void mark_consumed(const ChunkRef &c) {
        for (Rec &r : recs_)
            if (r.seq == compute_seq_ && r.ref.first == c.first) r.consumed = true;
    }
    void end_layer(uint32_t layer) {
        (void)layer;
        compute_seq_++;
        next_compute_chunk_ = 0;
        while (bases_.size() > 1 && bases_seq0_ < active_seq_) {
            bases_.pop_front();
            bases_seq0_++;
        }
    }

    // Copy side: the next chunk whose copy may be enqueued now, if any.
    bool next_copy(ChunkRef *out) {
        if (!started_ || order_.empty()) return false;
        if (copy_seq_ > active_seq_ + 1) return false;  // lookahead: one layer past the one begun last
        const uint32_t layer = seq_layer(copy_seq_);
        const uint32_t n = counts_[layer];
        const uint32_t first = copy_chunk_ * chunk_;
        const uint32_t count = n - first < chunk_ ? n - first : chunk_;
        const uint64_t base = seq_base(copy_seq_);
        const uint64_t a = base + first, b = a + count;
        int wait = -1;
        if (b > epoch_ordinal_ + n_slots_) {
            const uint64_t x = b - 1 - n_slots_;  // newest ordinal whose slot this chunk overwrites
            bool found = false;
            for (const Rec &r : recs_)
                if (r.ord_start <= x && x < r.ord_end) {
                    if (!r.consumed) return false;  // its consumer is not enqueued yet
                    wait = r.ref.event;
                    found = true;
                    break;
                }
            if (!found) return false;
        }
        Rec r;
        r.ref.layer = layer;
        r.ref.first = first;
        r.ref.count = count;
        r.ref.ordinal_base = base;
        r.ref.event = next_event_;
        r.ref.wait_event = wait;
        r.ord_start = a;
        r.ord_end = b;
        r.seq = copy_seq_;
        next_event_ = (next_event_ + 1) % n_events_;
        recs_.push_back(r);
        // drop records no future copy can name as predecessor
        while (!recs_.empty() && recs_.front().consumed && recs_.front().ord_end + n_slots_ <= b) recs_.pop_front();
        last_base_[layer] = base;
        copy_chunk_++;
        if ((uint64_t)copy_chunk_ * chunk_ >= n) {
            copy_seq_++;
            copy_chunk_ = 0;
        }
        *out = r.ref;
        return true;
    }

    uint64_t last_ordinal_base(uint32_t layer) const { return layer < last_base_.size() ? last_base_[layer] : 0; }

   private:
    struct Rec {
        ChunkRef ref;
        uint64_t ord_start = 0, ord_end = 0;
        uint64_t seq = 0;
        bool consumed = false;
    };

    // sequence index -> layer: the streamed layers in cyclic order from the restart layer
    uint32_t seq_layer(uint64_t seq) const { return order_.empty() ? 0 : order_[(start_pos_ + seq) % order_.size()]; }
    uint64_t seq_base(uint64_t seq) {
        if (bases_.empty()) {
            bases_.push_back(epoch_ordinal_);
            bases_seq0_ = 0;
        }
        while (bases_seq0_ + bases_.size() <= seq) {
            const uint64_t last = bases_seq0_ + bases_.size() - 1;
            bases_.push_back(bases_.back() + counts_[seq_layer(last)]);
        }
        return bases_[seq - bases_seq0_];
    }
    void restart_at(uint32_t layer) {
        // all earlier work has completed (the caller drained both streams)
        for (const Rec &r : recs_) ordinal_ = ordinal_ > r.ord_end ? ordinal_ : r.ord_end;
        recs_.clear();
        bases_.clear();
        bases_seq0_ = 0;
        order_.clear();
        for (uint32_t l = 0; l < n_layers_; l++)
            if (counts_[l]) order_.push_back(l);
        start_pos_ = 0;
        for (size_t i = 0; i < order_.size(); i++)
            if (order_[i] == layer) start_pos_ = (uint32_t)i;
        epoch_ordinal_ = ordinal_;
        compute_seq_ = 0;
        active_seq_ = 0;
        copy_seq_ = 0;
        copy_chunk_ = 0;
        next_compute_chunk_ = 0;
        started_ = false;
    }

    uint32_t n_layers_ = 0, n_slots_ = 1, chunk_ = 1;
    int n_events_ = 1, next_event_ = 0;
    std::vector<uint32_t> counts_, order_;
    std::vector<uint64_t> last_base_;
    std::deque<uint64_t> bases_;
    uint64_t bases_seq0_ = 0;
    std::deque<Rec> recs_;
    uint64_t ordinal_ = 0, epoch_ordinal_ = 0;
    uint64_t compute_seq_ = 0, active_seq_ = 0, copy_seq_ = 0;
    uint32_t start_pos_ = 0, copy_chunk_ = 0, next_compute_chunk_ = 0;
    bool started_ = false;
};

// One streamed layer's enqueue sequence, shared by the HIP path, the CPU
// simulator (kvattn_sched_simulate) and the host checks built with
// sanitizers: resident pages first (no wait), then each ring chunk after its
// ready fence, recording its consumed fence; the copies of later chunks and
// of the next streamed layer are enqueued as soon as the fence each depends
// on has been recorded.
template <class Exec>
int drive_streamed_layer(StreamPlanner &pl, uint32_t layer, Exec &x) {
    int rc;
    if (!pl.begin_layer(layer)) {
        if ((rc = x.drain())) return rc;  // out-of-order call: restart the schedule here
        pl.restart(layer);
        if (!pl.begin_layer(layer)) return x.internal("schedule restart failed");
    }
    x.begin(layer);
    ChunkRef c;
    while (pl.next_copy(&c))
        if ((rc = x.copy(c))) return rc;
    if ((rc = x.resident(layer))) return rc;
    while (pl.next_compute(layer, &c)) {
        if ((rc = x.compute(c))) return rc;
        pl.mark_consumed(c);
        while (pl.next_copy(&c))
            if ((rc = x.copy(c))) return rc;
    }
    pl.end_layer(layer);
    while (pl.next_copy(&c))
        if ((rc = x.copy(c))) return rc;
    return x.merge(layer);
}
