// host_checks.cpp -- the library's pure host logic under AddressSanitizer and
// UndefinedBehaviorSanitizer: page-table validation, the ring streaming
// planner driven through the same enqueue sequence the HIP path issues, and
// the adaptive partition policy, over many seeded random configurations.
//
// Built and run by tests/test_host_sanitizers.py with g++ (host code only).
// Exit status 0 and a last line "ok" mean every check held; a sanitizer
// report or a failed check ends the program with a non-zero status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../long_context_attention_amd/csrc/policy.h"
#include "../../long_context_attention_amd/csrc/sched.h"

#define CHECK(cond, ...)                                              \
    do {                                                              \
        if (!(cond)) {                                                \
            std::fprintf(stderr, "check failed at line %d: ", __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                        \
            std::fprintf(stderr, "\n");                               \
            std::exit(1);                                             \
        }                                                             \
    } while (0)

static std::mt19937_64 rng(20261202);
static uint32_t rnd(uint32_t n) { return n ? (uint32_t)(rng() % n) : 0; }

// ---------------------------------------------------------------------------
// Page tables: check_page_table against a direct quadratic reading of the
// rules (pool ids below n_pool, ring slots below n_ring, no physical page
// twice, host entries counted).
// ---------------------------------------------------------------------------
static void check_tables(int cases) {
    for (int c = 0; c < cases; c++) {
        const uint32_t n = 1 + rnd(300), n_pool = rnd(400), n_ring = rnd(40);
        std::vector<uint32_t> pt(n);
        for (auto &e : pt) {
            const uint32_t k = rnd(10);
            if (k < 5)
                e = rnd(n_pool + 3);
            else if (k < 8)
                e = 0x80000000u | rnd(n_ring + 2);
            else
                e = 0xFFFFFFFFu;
        }
        if (rnd(3) == 0 && n > 1) pt[rnd(n)] = pt[rnd(n)];  // a likely duplicate
        PlanCheck got;
        const int rc = check_page_table(pt.data(), n, n_pool, n_ring, &got);
        int want = PT_OK;
        uint32_t hosts = 0;
        for (uint32_t P = 0; P < n && want == PT_OK; P++) {
            const uint32_t e = pt[P];
            if (e == 0xFFFFFFFFu) {
                hosts++;
            } else if (e & 0x80000000u) {
                if ((e & 0x7FFFFFFFu) >= n_ring) want = PT_BAD_RING;
            } else if (e >= n_pool) {
                want = PT_BAD_POOL;
            }
        }
        if (want == PT_OK)
            for (uint32_t a = 0; a < n && want == PT_OK; a++)
                for (uint32_t b = a + 1; b < n; b++)
                    if (pt[a] != 0xFFFFFFFFu && pt[a] == pt[b]) {
                        want = PT_DUPLICATE;
                        break;
                    }
        CHECK(rc == want, "table case %d: status %d, expected %d", c, rc, want);
        if (rc == PT_OK) CHECK(got.n_host == hosts, "table case %d: %u host entries, expected %u", c, got.n_host, hosts);
        if (rc == PT_DUPLICATE) CHECK(pt[got.bad_index] == pt[got.other_index] && got.bad_index != got.other_index,
                                      "table case %d: duplicate indices %u %u", c, got.bad_index, got.other_index);
    }
}

// ---------------------------------------------------------------------------
// Streaming planner: an executor that simulates the copy and compute streams
// (each in order, events carry completion times) and checks that a slot is
// refilled only after every read of its previous content finished, that a
// chunk is read only after its copy finished and from the ordinals the copy
// wrote, that every streamed page of a called layer is read exactly once per
// call, and that copies never run more than one streamed layer ahead.
// ---------------------------------------------------------------------------
struct SimStreams {
    uint32_t n_slots;
    const std::vector<uint32_t> &counts;
    double copy_t = 0, compute_t = 0;
    std::vector<double> ready, consumed;  // per event index
    std::vector<double> slot_free;        // when the last reader of a slot finished
    std::vector<uint64_t> slot_ord;       // global ordinal a slot holds (UINT64_MAX: none)
    std::vector<double> slot_filled;      // when that copy finished
    std::vector<int> layer_reads;         // pages of the current call read so far
    uint32_t cur_layer = 0;

    SimStreams(uint32_t slots, int events, const std::vector<uint32_t> &c)
        : n_slots(slots), counts(c), ready(events, -1), consumed(events, -1), slot_free(slots, 0),
          slot_ord(slots, UINT64_MAX), slot_filled(slots, 0) {}

    int drain() {
        const double t = copy_t > compute_t ? copy_t : compute_t;
        copy_t = compute_t = t;
        return 0;
    }
    int internal(const char *) { return KVATTN_E_STATE; }
    void begin(uint32_t layer) {
        cur_layer = layer;
        layer_reads.assign(counts[layer], 0);
    }
    int copy(const ChunkRef &c) {
        CHECK(c.count >= 1 && c.first + c.count <= counts[c.layer], "copy range %u+%u of %u", c.first, c.count,
              counts[c.layer]);
        double start = copy_t;
        if (c.wait_event >= 0) {
            CHECK(consumed[c.wait_event] >= 0, "copy waits on an unrecorded consumed fence");
            if (consumed[c.wait_event] > start) start = consumed[c.wait_event];
        }
        const double end = start + 1.0 + 0.25 * c.count;
        for (uint32_t o = c.first; o < c.first + c.count; o++) {
            const uint32_t s = (uint32_t)((c.ordinal_base + o) % n_slots);
            CHECK(slot_free[s] <= start, "slot %u refilled at %.2f while a read ends at %.2f", s, start, slot_free[s]);
            slot_ord[s] = c.ordinal_base + o;
            slot_filled[s] = end;
            slot_free[s] = start;
        }
        copy_t = end;
        ready[c.event] = end;
        consumed[c.event] = -1;
        // lookahead: a copy's layer is the layer being computed or the next streamed one
        CHECK(c.layer == cur_layer || next_streamed(cur_layer) == c.layer, "copy of layer %u while layer %u computes",
              c.layer, cur_layer);
        return 0;
    }
    uint32_t next_streamed(uint32_t layer) const {
        const uint32_t L = (uint32_t)counts.size();
        for (uint32_t k = 1; k <= L; k++)
            if (counts[(layer + k) % L]) return (layer + k) % L;
        return layer;
    }
    int resident(uint32_t) {
        compute_t += 0.5;
        return 0;
    }
    int compute(const ChunkRef &c) {
        CHECK(c.layer == cur_layer, "compute of layer %u inside the call of layer %u", c.layer, cur_layer);
        CHECK(ready[c.event] >= 0, "compute waits on an unrecorded ready fence");
        const double start = compute_t > ready[c.event] ? compute_t : ready[c.event];
        const double end = start + 0.3 * c.count;
        for (uint32_t o = c.first; o < c.first + c.count; o++) {
            const uint32_t s = (uint32_t)((c.ordinal_base + o) % n_slots);
            CHECK(slot_ord[s] == c.ordinal_base + o, "slot %u holds ordinal %llu, the chunk reads %llu", s,
                  (unsigned long long)slot_ord[s], (unsigned long long)(c.ordinal_base + o));
            CHECK(slot_filled[s] <= start, "slot %u read before its copy finished", s);
            if (slot_free[s] < end) slot_free[s] = end;
            layer_reads[o]++;
        }
        compute_t = end;
        consumed[c.event] = end;
        return 0;
    }
    int merge(uint32_t layer) {
        for (uint32_t o = 0; o < counts[layer]; o++)
            CHECK(layer_reads[o] == 1, "layer %u streamed page %u read %d times", layer, o, layer_reads[o]);
        compute_t += 0.2;
        return 0;
    }
};

static void check_planner(int cases) {
    for (int c = 0; c < cases; c++) {
        const uint32_t L = 1 + rnd(9), n_slots = 1 + rnd(24), chunk = 1 + rnd(n_slots + 2);
        std::vector<uint32_t> counts(L);
        for (auto &n : counts) n = rnd(4) == 0 ? 0 : 1 + rnd(60);
        StreamPlanner pl;
        pl.init(L, n_slots, chunk);
        pl.set_layer_counts(counts);
        SimStreams sim(n_slots, pl.n_events(), counts);
        const int calls = 1 + (int)rnd(4 * L + 4);
        uint32_t layer = rnd(L);
        for (int i = 0; i < calls; i++) {
            // mostly in order; sometimes a jump (the driver drains and restarts)
            layer = rnd(6) == 0 ? rnd(L) : (layer + 1) % L;
            if (!counts[layer]) continue;
            const int rc = drive_streamed_layer(pl, layer, sim);
            CHECK(rc == 0, "planner case %d call %d: status %d", c, i, rc);
        }
    }
}

// ---------------------------------------------------------------------------
// Policy: every decision keeps pool + ring within the budget, the ring within
// its bounds while anything streams, and residency within each layer's pages.
// ---------------------------------------------------------------------------
static void check_policy(int cases) {
    for (int c = 0; c < cases; c++) {
        kvattn_policy_config cfg{};
        cfg.n_layers = 1 + rnd(70);
        cfg.page_tokens = 32 * (1 + rnd(16));
        cfg.budget_pages = rnd(6000);
        cfg.min_ring_slots = rnd(5) == 0 ? 0 : 1 + rnd(40);
        cfg.max_ring_slots = cfg.min_ring_slots + rnd(200);
        cfg.ring_step = rnd(8) == 0 ? 0 : 1 + rnd(32);
        cfg.grow_after = rnd(8) == 0 ? 0 : 1 + rnd(3);
        cfg.shrink_after = 1 + rnd(3);
        cfg.miss_rate_high = (float)(rnd(1200)) / 1000.f;
        cfg.busy_high = (float)(rnd(1200)) / 1000.f;
        cfg.occupancy_low = (float)(rnd(1000)) / 1000.f;
        kvattn_policy_state st{};
        std::vector<uint32_t> res(cfg.n_layers, 0xDEADBEEFu);
        for (int it = 0; it < 12; it++) {
            kvattn_policy_observation ob{};
            ob.n_tokens = rnd(1u << 20);
            ob.chunks = rnd(200);
            ob.ready_misses = ob.chunks ? rnd(ob.chunks + 1) : 0;
            ob.ring_occupancy = (float)rnd(1001) / 1000.f;
            ob.copy_busy = (float)rnd(1001) / 1000.f;
            kvattn_policy_state next{};
            kvattn_policy_decision d{};
            const int rc = kvattn_policy::step(cfg, st, ob, &next, &d, res.data());
            if (rc != KVATTN_OK) {
                CHECK(rc == KVATTN_E_ARG || rc == KVATTN_E_NOSPACE, "policy case %d: status %d", c, rc);
                break;
            }
            const uint64_t P = ((uint64_t)ob.n_tokens + cfg.page_tokens - 1) / cfg.page_tokens;
            uint64_t resident = 0;
            for (uint32_t l = 0; l < cfg.n_layers; l++) {
                CHECK(res[l] <= P, "policy case %d: layer %u keeps %u of %llu pages", c, l, res[l],
                      (unsigned long long)P);
                resident += res[l];
            }
            CHECK(resident == d.resident_pages, "policy case %d: resident sum %llu vs %u", c,
                  (unsigned long long)resident, d.resident_pages);
            CHECK(resident + d.streamed_pages == P * cfg.n_layers, "policy case %d: pages do not add up", c);
            if (d.streamed_pages) {
                CHECK(resident + d.ring_slots <= cfg.budget_pages, "policy case %d: pool %llu + ring %u > budget %u", c,
                      (unsigned long long)resident, d.ring_slots, cfg.budget_pages);
                CHECK(d.ring_slots >= 1, "policy case %d: streaming without a ring", c);
            } else {
                CHECK(d.ring_slots == 0 && resident <= cfg.budget_pages, "policy case %d: fits but ring %u", c,
                      d.ring_slots);
            }
            st = next;
        }
    }
}

int main() {
    check_tables(4000);
    check_planner(3000);
    check_policy(3000);
    std::printf("ok\n");
    return 0;
}
