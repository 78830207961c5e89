"""CPU tests of the adaptive resident/ring partition (kvattn_policy_step).

The rule under test is the one include/kvattn.h states for the pages'
policy ("troed's fork of Raymond's adaptive KV streaming", sections "KV data
movement and attention" and "Backend-neutral memory and streaming
contracts"): everything resident while it fits; otherwise a ring of at least
min_ring_slots, the deficit streamed from the fewest whole layers; the ring
grows after grow_after pressure samples in a row (misses while the copy
stream has idle time) and shrinks after shrink_after saturated or idle-ring
samples in a row.
"""
import numpy as np
import pytest

import long_context_attention_amd as kv

L, T = 8, 256


def cfg(budget, **kw):
    base = dict(min_ring_slots=4, max_ring_slots=24, ring_step=4, grow_after=2, shrink_after=3, miss_rate_high=0.2,
                busy_high=0.9, occupancy_low=0.5)
    base.update(kw)
    return kv.policy_config(L, T, budget, **base)


def obs(n_tokens, chunks=0, misses=0, occupancy=0.0, busy=0.0):
    o = kv.PolicyObservation()
    o.n_tokens, o.chunks, o.ready_misses, o.ring_occupancy, o.copy_busy = n_tokens, chunks, misses, occupancy, busy
    return o


def check_invariants(c, d, res, n_tokens):
    P = -(-n_tokens // T)
    assert d.pages_per_layer == P and len(res) == L
    assert np.all(res <= P)
    assert d.resident_pages == int(res.sum())
    assert d.streamed_pages == L * P - d.resident_pages
    assert d.streamed_layers == int(np.sum(res < P))
    assert d.resident_pages + d.ring_slots <= c.budget_pages
    if d.streamed_pages:
        assert c.min_ring_slots <= d.ring_slots <= min(c.max_ring_slots, c.budget_pages - 1)
        # the deficit sits in the first layers: fully streamed ones, then at most one partial layer
        partial = [l for l in range(L) if 0 < res[l] < P]
        assert len(partial) <= 1
        streamed = np.where(res < P)[0]
        assert np.array_equal(streamed, np.arange(len(streamed)))
        assert np.all(res[:max(0, len(streamed) - 1)] == 0)
    else:
        assert d.ring_slots == 0


def test_fits_all_resident():
    c = cfg(budget=8 * 40)
    nxt, d, res = kv.policy_step(c, kv.PolicyState(), obs(40 * T))
    assert d.reason == kv.POLICY_FITS and d.ring_slots == 0 and d.streamed_pages == 0
    assert np.all(res == 40)
    check_invariants(c, d, res, 40 * T)


def test_overflow_streams_fewest_layers():
    # 8 layers x 40 pages = 320 > 300: pool 296 after a 4-slot ring, deficit 24 pages
    c = cfg(budget=300)
    nxt, d, res = kv.policy_step(c, kv.PolicyState(), obs(40 * T - 5))
    assert d.reason == kv.POLICY_CONTEXT and d.ring_slots == 4 and d.changed
    assert list(res) == [16] + [40] * 7
    assert d.streamed_layers == 1 and d.streamed_pages == 24
    check_invariants(c, d, res, 40 * T - 5)
    # larger context: more pages stream, whole layers first
    nxt2, d2, res2 = kv.policy_step(c, nxt, obs(100 * T))
    assert d2.reason == kv.POLICY_CONTEXT and d2.ring_slots == 4
    assert list(res2) == [0, 0, 0, 0, 0] + [96, 100, 100]
    check_invariants(c, d2, res2, 100 * T)
    # back below the budget: all resident again, ring released
    nxt3, d3, res3 = kv.policy_step(c, nxt2, obs(30 * T))
    assert d3.reason == kv.POLICY_FITS and d3.ring_slots == 0 and np.all(res3 == 30)


def run_seq(c, samples, n_tokens=60 * T):
    st, _, _ = kv.policy_step(c, kv.PolicyState(), obs(n_tokens))
    out = []
    for s in samples:
        st, d, res = kv.policy_step(c, st, obs(n_tokens, **s))
        check_invariants(c, d, res, n_tokens)
        out.append((d.reason, d.ring_slots))
    return out


PRESSURE = dict(chunks=40, misses=20, occupancy=0.9, busy=0.5)
SATURATED = dict(chunks=40, misses=20, occupancy=1.0, busy=0.95)
IDLE = dict(chunks=40, misses=0, occupancy=0.2, busy=0.3)
NEUTRAL = dict(chunks=40, misses=0, occupancy=0.8, busy=0.5)


def test_grow_after_consecutive_pressure():
    c = cfg(budget=400)
    seq = run_seq(c, [PRESSURE] * 5)
    assert seq == [(kv.POLICY_HOLD, 4), (kv.POLICY_GROW_RING, 8), (kv.POLICY_HOLD, 8), (kv.POLICY_GROW_RING, 12),
                   (kv.POLICY_HOLD, 12)]


def test_hysteresis_interrupted_streak_does_not_grow():
    c = cfg(budget=400)
    seq = run_seq(c, [PRESSURE, NEUTRAL, PRESSURE, IDLE, PRESSURE])
    assert all(r == kv.POLICY_HOLD and slots == 4 for r, slots in seq)


def test_low_miss_rate_is_not_pressure():
    c = cfg(budget=400)
    seq = run_seq(c, [dict(chunks=40, misses=4, occupancy=0.9, busy=0.5)] * 4)   # 10 % <= 20 %
    assert all(slots == 4 for _, slots in seq)


def test_grow_is_bounded():
    c = cfg(budget=400, max_ring_slots=10)
    seq = run_seq(c, [PRESSURE] * 8)
    assert max(s for _, s in seq) == 10
    assert [s for _, s in seq][-1] == 10


def test_saturated_link_shrinks_after_streak():
    c = cfg(budget=400)
    seq = run_seq(c, [PRESSURE] * 4 + [SATURATED] * 7)
    slots = [s for _, s in seq]
    assert slots[:4] == [4, 8, 8, 12]
    # three saturated samples in a row shrink one step, three more another
    assert slots[4:] == [12, 12, 8, 8, 8, 4, 4]
    assert seq[6][0] == kv.POLICY_SHRINK_RING and seq[9][0] == kv.POLICY_SHRINK_RING


def test_idle_ring_shrinks_to_min():
    c = cfg(budget=400)
    seq = run_seq(c, [PRESSURE] * 6 + [IDLE] * 12)
    slots = [s for _, s in seq]
    assert slots[5] == 16
    assert slots[-1] == 4 and min(slots) == 4


def test_ring_growth_moves_pages_out_of_the_pool():
    c = cfg(budget=400)
    st, d0, r0 = kv.policy_step(c, kv.PolicyState(), obs(60 * T))
    st, _, _ = kv.policy_step(c, st, obs(60 * T, **PRESSURE))
    st, d1, r1 = kv.policy_step(c, st, obs(60 * T, **PRESSURE))
    assert d1.reason == kv.POLICY_GROW_RING and d1.changed
    assert d1.resident_pages == d0.resident_pages - 4 == 400 - 8
    assert d1.streamed_pages == d0.streamed_pages + 4


def test_rejections():
    with pytest.raises(kv.KVAttnError) as e:
        kv.policy_step(cfg(budget=400, min_ring_slots=0), kv.PolicyState(), obs(60 * T))
    assert e.value.code == kv.E_ARG
    with pytest.raises(kv.KVAttnError) as e:
        kv.policy_step(cfg(budget=400, max_ring_slots=2), kv.PolicyState(), obs(60 * T))
    assert e.value.code == kv.E_ARG
    with pytest.raises(kv.KVAttnError) as e:
        kv.policy_step(cfg(budget=400, busy_high=0.0), kv.PolicyState(), obs(60 * T))
    assert e.value.code == kv.E_ARG
    with pytest.raises(kv.KVAttnError) as e:      # fewer pages than layers
        kv.policy_step(cfg(budget=7), kv.PolicyState(), obs(60 * T))
    assert e.value.code == kv.E_NOSPACE
    with pytest.raises(kv.KVAttnError) as e:      # no room for a 4-slot ring beside the pool
        kv.policy_step(cfg(budget=9, min_ring_slots=9, max_ring_slots=9), kv.PolicyState(), obs(60 * T))
    assert e.value.code == kv.E_NOSPACE


def test_random_sequences_keep_invariants():
    rng = np.random.default_rng(0)
    kinds = [PRESSURE, SATURATED, IDLE, NEUTRAL, {}]
    for trial in range(50):
        c = cfg(budget=int(rng.integers(40, 600)), ring_step=int(rng.integers(1, 9)),
                grow_after=int(rng.integers(1, 4)), shrink_after=int(rng.integers(1, 4)))
        st = kv.PolicyState()
        for _ in range(40):
            n_tokens = int(rng.integers(1, 120 * T))
            st, d, res = kv.policy_step(c, st, obs(n_tokens, **kinds[int(rng.integers(0, len(kinds)))]))
            check_invariants(c, d, res, n_tokens)
            assert st.ring_slots == d.ring_slots
