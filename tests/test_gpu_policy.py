"""GPU tests of the adaptive resident/ring partition: decisions of
kvattn_policy_step applied to a streamed handle (pages re-placed, ring
resized with kvattn_set_ring_slots) keep attention equal to the oracle, and
kvattn_observe_read returns sane readiness-miss, occupancy and copy-busy
samples from real streamed calls."""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
from gpu_util import TOL, handle, oracle_out, run, say

pytestmark = pytest.mark.gpu


def apply_residency(h, layers, res, ring_slots, hists):
    """Keep the last res[l] pages of layer l resident (the tail, where new
    rows land), stream the rest from its pinned history."""
    h.set_ring_slots(ring_slots)
    pb = kv.page_bytes(h.params)
    nxt = 0
    for l, kvl in enumerate(layers):
        n = kvl.pages.shape[0]
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        for P in range(n - int(res[l]), n):
            table[P] = nxt
            h.pool[nxt * pb:(nxt + 1) * pb].copy_(kvl.pages[P].to("cuda"))
            nxt += 1
        torch.cuda.synchronize()
        h.set_layer(l, table, kvl.kc.shape[0], hists[l])
    return nxt


def check_layers(h, layers, qs, refs, W):
    worst = 0.0
    for rep in range(2):
        for l in range(len(layers)):
            err = np.max(np.abs(run(h, l, qs[l], W, "verify") - refs[l]))
            worst = max(worst, err)
    assert worst <= TOL
    return worst


def test_policy_decisions_applied_keep_parity():
    Lr, N, Hq, Hkv, W = 4, 12 * 256 + 40, 40, 8, 4
    P = -(-N // 256)
    budget = 30                       # 4 layers x 13 pages = 52 do not fit
    say(f"case policy L={Lr} N={N} budget={budget}")
    layers = [inputs.draw_layer(N, Hkv, l, 88) for l in range(Lr)]
    qs = [inputs.draw_queries(W, Hq, l, 88) for l in range(Lr)]
    refs = [oracle_out(layers[l], qs[l], Hq, Hkv) for l in range(Lr)]
    hists = [kvl.pages.contiguous().pin_memory() for kvl in layers]
    h = handle(Hq, Hkv, budget, P, 8, n_ring=12, chunk_slots=2, n_layers=Lr)
    c = kv.policy_config(Lr, 256, budget, min_ring_slots=4, max_ring_slots=12, ring_step=4, grow_after=1,
                         shrink_after=1)
    o = kv.PolicyObservation()
    o.n_tokens = N
    st, d, res = kv.policy_step(c, kv.PolicyState(), o)
    assert d.reason == kv.POLICY_CONTEXT and d.ring_slots == 4
    used = apply_residency(h, layers, res, d.ring_slots, hists)
    assert used == d.resident_pages <= budget - d.ring_slots
    say(f"  start: ring {d.ring_slots}, resident {list(res)}, err {check_layers(h, layers, qs, refs, W):.3e}")

    # a real sample from streamed calls
    h.observe(256)
    check_layers(h, layers, qs, refs, W)
    sample = h.observe_read(N)
    say(f"  sample: chunks {sample.chunks} misses {sample.ready_misses} occupancy {sample.ring_occupancy:.2f} "
        f"busy {sample.copy_busy:.2f}")
    assert sample.chunks > 0 and 0 <= sample.ready_misses <= sample.chunks
    assert 0.0 <= sample.ring_occupancy <= 1.0 and 0.0 <= sample.copy_busy <= 1.0
    h.observe(0)

    # pressure grows the ring (pages leave the pool), saturation shrinks it back
    press = kv.PolicyObservation()
    press.n_tokens, press.chunks, press.ready_misses, press.ring_occupancy, press.copy_busy = N, 10, 8, 1.0, 0.3
    st, d, res = kv.policy_step(c, st, press)
    assert d.reason == kv.POLICY_GROW_RING and d.ring_slots == 8
    apply_residency(h, layers, res, d.ring_slots, hists)
    say(f"  grown: ring {d.ring_slots}, resident {list(res)}, err {check_layers(h, layers, qs, refs, W):.3e}")
    sat = kv.PolicyObservation()
    sat.n_tokens, sat.chunks, sat.ready_misses, sat.ring_occupancy, sat.copy_busy = N, 10, 8, 1.0, 0.97
    st, d, res = kv.policy_step(c, st, sat)
    assert d.reason == kv.POLICY_SHRINK_RING and d.ring_slots == 4
    apply_residency(h, layers, res, d.ring_slots, hists)
    say(f"  shrunk: ring {d.ring_slots}, resident {list(res)}, err {check_layers(h, layers, qs, refs, W):.3e}")
    # context shrinks below the budget: everything resident, ring unused
    h.destroy()


def test_set_ring_slots_rejections():
    h = handle(8, 2, 8, 4, 8, n_ring=6, n_layers=1)
    with pytest.raises(kv.KVAttnError) as e:
        h.set_ring_slots(0)
    assert e.value.code == kv.E_RANGE
    with pytest.raises(kv.KVAttnError) as e:
        h.set_ring_slots(7)
    assert e.value.code == kv.E_RANGE
    kvl = inputs.draw_layer(600, 2, 0, 89)
    from gpu_util import place
    place(h, 0, kvl, np.array([0, kv.PT_RING_FLAG | 5, 1], dtype=np.uint32))
    with pytest.raises(kv.KVAttnError) as e:      # a caller-placed page sits in slot 5
        h.set_ring_slots(4)
    assert e.value.code == kv.E_RANGE
    h.set_ring_slots(6)
    h.destroy()
