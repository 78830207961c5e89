// policy.h -- the adaptive resident/ring partition (pure host logic).
//
// "troed's fork of Raymond's adaptive KV streaming", sections "KV data
// movement and attention" and "Backend-neutral memory and streaming
// contracts": when the whole history fits, every page is resident and there
// is no ring; under memory pressure resident pages are traded for ring slots,
// first by streaming one or a few layers while the others stay fully
// resident, then more pages as the context grows.  The split between pool
// and ring is adjusted with hysteresis from sampled readiness misses, ring
// occupancy and copy-stream busy time, and proposing it moves no bytes.
//
// Reading of the feedback (the pages name the signals, not the rule):
//   - pressure: a share of the streamed chunks whose compute reached its
//     ready fence before the copy had finished (readiness misses) while the
//     copy stream still had idle time.  The ring, not the link, limits the
//     prefetch: grow the ring by one step after `grow_after` such samples in
//     a row.
//   - saturated: the copy stream was busy for at least `busy_high` of the
//     sampled interval.  A larger ring cannot help a saturated link; fewer
//     streamed pages can: shrink the ring (its pages return to residency)
//     after `shrink_after` such samples in a row.
//   - idle ring: no misses and peak ring occupancy below `occupancy_low`:
//     the ring is larger than the prefetch needs; shrink after
//     `shrink_after` samples in a row.
// Any other sample resets the streaks.  The ring stays within
// [min_ring_slots, max_ring_slots] whenever anything streams.
#pragma once
#include <stdint.h>

#include "../../include/kvattn.h"

namespace kvattn_policy {

inline uint32_t clamp_u32(uint32_t x, uint32_t lo, uint32_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

inline int validate(const kvattn_policy_config &c) {
    if (c.n_layers == 0 || c.page_tokens == 0) return KVATTN_E_ARG;
    if (c.min_ring_slots == 0 || c.max_ring_slots < c.min_ring_slots || c.ring_step == 0) return KVATTN_E_ARG;
    if (c.grow_after == 0 || c.shrink_after == 0) return KVATTN_E_ARG;
    if (!(c.miss_rate_high >= 0.f && c.miss_rate_high <= 1.f) || !(c.busy_high > 0.f && c.busy_high <= 1.f) ||
        !(c.occupancy_low >= 0.f && c.occupancy_low <= 1.f))
        return KVATTN_E_ARG;
    if (c.budget_pages < c.n_layers)  // one page per layer at least
        return KVATTN_E_NOSPACE;
    return KVATTN_OK;
}

// One policy step.  resident[n_layers] receives the resident page count of
// every layer (the rest of each layer's pages stream through the ring).
inline int step(const kvattn_policy_config &c, const kvattn_policy_state &prev, const kvattn_policy_observation &obs,
                kvattn_policy_state *next, kvattn_policy_decision *out, uint32_t *resident) {
    int rc = validate(c);
    if (rc != KVATTN_OK) return rc;
    const uint64_t P = ((uint64_t)obs.n_tokens + c.page_tokens - 1) / c.page_tokens;  // pages per layer
    const uint64_t need = P * c.n_layers;
    kvattn_policy_state s = prev;
    kvattn_policy_decision d{};
    d.pages_per_layer = (uint32_t)P;
    if (need <= c.budget_pages) {
        // everything fits: all resident, no ring
        s.ring_slots = 0;
        s.pressure_streak = s.saturated_streak = s.idle_streak = 0;
        d.reason = KVATTN_POLICY_FITS;
    } else {
        const uint32_t ring_hi = c.max_ring_slots < c.budget_pages ? c.max_ring_slots : c.budget_pages - 1;
        if (ring_hi < c.min_ring_slots) return KVATTN_E_NOSPACE;
        uint32_t R = prev.ring_slots;
        d.reason = KVATTN_POLICY_HOLD;
        if (R == 0) {  // streaming starts now
            R = c.min_ring_slots;
            s.pressure_streak = s.saturated_streak = s.idle_streak = 0;
            d.reason = KVATTN_POLICY_CONTEXT;
        } else if (obs.chunks > 0) {
            const float miss_rate = (float)obs.ready_misses / (float)obs.chunks;
            const bool saturated = obs.copy_busy >= c.busy_high;
            const bool pressure = !saturated && obs.ready_misses > 0 && miss_rate > c.miss_rate_high;
            const bool idle = obs.ready_misses == 0 && obs.ring_occupancy < c.occupancy_low;
            s.pressure_streak = pressure ? prev.pressure_streak + 1 : 0;
            s.saturated_streak = saturated ? prev.saturated_streak + 1 : 0;
            s.idle_streak = (idle && !saturated) ? prev.idle_streak + 1 : 0;
            if (s.pressure_streak >= c.grow_after && R < ring_hi) {
                R = R + c.ring_step < ring_hi ? R + c.ring_step : ring_hi;
                s.pressure_streak = 0;
                d.reason = KVATTN_POLICY_GROW_RING;
            } else if ((s.saturated_streak >= c.shrink_after || s.idle_streak >= c.shrink_after) &&
                       R > c.min_ring_slots) {
                R = R > c.min_ring_slots + c.ring_step ? R - c.ring_step : c.min_ring_slots;
                s.saturated_streak = s.idle_streak = 0;
                d.reason = KVATTN_POLICY_SHRINK_RING;
            }
        }
        s.ring_slots = clamp_u32(R, c.min_ring_slots, ring_hi);
        if (d.reason == KVATTN_POLICY_HOLD && prev.pages_per_layer != P) d.reason = KVATTN_POLICY_CONTEXT;
    }
    // residency: the pool holds budget - ring pages; the deficit streams
    // from the fewest layers (whole layers first, in layer order)
    const uint64_t pool = c.budget_pages - s.ring_slots;
    uint64_t deficit = need > pool ? need - pool : 0;
    d.streamed_layers = 0;
    d.resident_pages = 0;
    for (uint32_t l = 0; l < c.n_layers; l++) {
        const uint64_t take = deficit < P ? deficit : P;
        deficit -= take;
        resident[l] = (uint32_t)(P - take);
        d.resident_pages += resident[l];
        if (take) d.streamed_layers++;
    }
    d.ring_slots = s.ring_slots;
    d.streamed_pages = (uint32_t)(need - d.resident_pages);
    d.changed = (s.ring_slots != prev.ring_slots || (uint32_t)P != prev.pages_per_layer) ? 1u : 0u;
    s.pages_per_layer = (uint32_t)P;
    *next = s;
    *out = d;
    return KVATTN_OK;
}

}  // namespace kvattn_policy
