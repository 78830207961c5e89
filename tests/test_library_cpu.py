"""CPU tests of the HIP library's host side: exports, argument and page-table
validation, and the streaming planner under a discrete-event simulation.
No GPU work is issued (calls that would need a device are not made)."""
import ctypes
import os
import re

import numpy as np
import pytest

import long_context_attention_amd as kv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "kvattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvattn_[a-z_]+)\s*\(", src)) - {"kvattn_params"})


def test_library_exports_every_declared_symbol():
    L = kv.lib()
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"{n} declared in kvattn.h but not exported"
    assert set(names) == set(kv.kvattn.EXPORTS)


def test_probe_library_exports_and_rejects_bad_arguments():
    # the plain-read ceiling helper beside the attention library (benchmark only)
    from long_context_attention_amd import build as hipbuild
    src = open(os.path.join(ROOT, "include", "kvattn_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(kvattn_[a-z_]+)\s*\(", src)))
    assert names == ["kvattn_probe_read_ceiling"]
    P = ctypes.CDLL(hipbuild.PROBE_LIB)
    fn = P.kvattn_probe_read_ceiling
    fn.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    us = (ctypes.c_double * 8)()
    best = ctypes.c_double()
    # argument checks come before any device call
    assert fn(15, 1, 1, us, ctypes.byref(best)) == -1      # not a multiple of 16
    assert fn(1024, 0, 1, us, ctypes.byref(best)) == -1    # no buffer
    assert fn(1024, 1, 0, us, ctypes.byref(best)) == -1    # no pass
    assert fn(1024, 1, 1, None, ctypes.byref(best)) == -1  # no output


def test_supported_and_sizes():
    assert kv.supported()
    for pair in [(kv.TYPE_Q8_0, kv.TYPE_Q8_0), (kv.TYPE_Q4_0, kv.TYPE_Q4_0), (kv.TYPE_F16, kv.TYPE_F16)]:
        assert kv.supported(*pair)
        q = kv.make_params(4, 40, 8, 16, 16, 6, k_type=pair[0], v_type=pair[1])
        assert kv.page_bytes(q) == oracle.page_bytes(8, 256, *pair) > 0
        assert kv.workspace_bytes(q) > 0
    for pair in [(kv.TYPE_Q4_0, kv.TYPE_Q8_0), (kv.TYPE_F16, kv.TYPE_Q4_0), (kv.TYPE_Q8_0, kv.TYPE_F16), (3, 3)]:
        assert not kv.supported(*pair)
        assert kv.page_bytes(kv.make_params(4, 40, 8, 16, 16, 6, k_type=pair[0], v_type=pair[1])) == 0
    assert not kv.supported(kv.TYPE_Q8_0, kv.TYPE_Q4_0, 64)
    p = kv.make_params(64, 40, 8, 10240, 160, 6)
    assert kv.page_bytes(p) == 425984
    ws = kv.workspace_bytes(p)
    units = 160 * 6 * 40  # split partials at one page per split, 6 rows
    assert ws >= units * 130 * 4 + 2 * 64 * 160 * 4
    bad = kv.make_params(64, 40, 8, 10240, 160, 6, head_dim=64)
    assert kv.page_bytes(bad) == 0 and kv.workspace_bytes(bad) == 0
    assert kv.page_bytes(kv.make_params(1, 4, 1, 8, 8, 1, page_tokens=100)) == 0
    short = kv.make_params(1, 4, 1, 8, 8, 1)
    short.struct_size = 8
    assert kv.page_bytes(short) == 0


def create_status(params, pool=1 << 40, ring=0, ws=None, null_ws=False, null_out=False):
    """kvattn_create with fake (never dereferenced) pointers: every case here
    is rejected before any HIP call."""
    L = kv.lib()
    h = ctypes.c_void_p()
    wsb = kv.workspace_bytes(params) if ws is None else ws
    return L.kvattn_create(ctypes.byref(params), ctypes.c_void_p(0x1000), pool, ctypes.c_void_p(0x2000), ring,
                           None if null_ws else ctypes.c_void_p(0x3000), wsb, None, None,
                           None if null_out else ctypes.byref(h))


def test_create_rejections():
    p = kv.make_params(2, 40, 8, 4, 10, 6)
    assert create_status(p, null_out=True) == kv.E_ARG
    assert create_status(kv.make_params(2, 40, 8, 4, 10, 6, k_type=kv.TYPE_Q4_0, v_type=kv.TYPE_Q8_0)) == kv.E_UNSUPPORTED
    assert "Q8_0" in kv.global_error()
    assert create_status(kv.make_params(2, 40, 8, 4, 10, 6, head_dim=96)) == kv.E_UNSUPPORTED
    assert create_status(kv.make_params(2, 40, 6, 4, 10, 6)) == kv.E_UNSUPPORTED   # 40 % 6 != 0
    assert create_status(kv.make_params(0, 40, 8, 4, 10, 6)) == kv.E_ARG
    assert create_status(kv.make_params(2, 40, 8, 4, 10, 0)) == kv.E_ARG
    assert create_status(p, pool=10) == kv.E_NOSPACE
    assert create_status(p, ws=100) == kv.E_NOSPACE
    assert create_status(p, null_ws=True) == kv.E_ARG
    pr = kv.make_params(2, 40, 8, 4, 10, 6, n_ring_slots=3)
    assert create_status(pr, ring=100) == kv.E_NOSPACE
    assert create_status(kv.make_params(2, 40, 8, 4, 10, 6, softmax_scale=-1.0)) == kv.E_ARG


def test_page_table_validation():
    p = kv.make_params(2, 40, 8, 10, 8, 6, n_ring_slots=4)
    v = kv.validate_page_table
    assert v(p, [0, 1, 2], 700) == kv.OK
    assert v(p, [0, 1, 10], 700) == kv.E_RANGE                      # pool id out of range
    assert v(p, [0, kv.PT_RING(4), 2], 700) == kv.E_RANGE           # ring slot out of range
    assert v(p, [0, kv.PT_RING(3), 2], 700) == kv.OK
    assert v(p, [0, 1, 1], 700) == kv.E_PLAN                        # one physical page twice
    assert "already used" in kv.global_error()
    assert v(p, [kv.PT_RING(2), 1, kv.PT_RING(2)], 700) == kv.E_PLAN
    assert v(p, [0, kv.PT_HOST, 2], 700) == kv.E_PLAN               # streamed without history
    assert v(p, [0, kv.PT_HOST, kv.PT_HOST], 700, has_history=True) == kv.OK
    assert v(p, list(range(9)), 9 * 256) == kv.E_NOSPACE            # beyond max_pages_per_layer
    assert v(p, [0], 0) == kv.E_ARG
    p0 = kv.make_params(2, 40, 8, 10, 8, 6)
    assert v(p0, [0, kv.PT_HOST], 300, has_history=True) == kv.E_PLAN  # no ring to stream through


# ---------------------------------------------------------------- streaming planner
COPY, COMPUTE, DRAIN, MERGE, RESIDENT, BEGIN = 1, 2, 3, 4, 5, 6


def simulate(ops, n_slots, counts, copy_cost=10.0, compute_cost=1.0):
    """Replay the enqueue log on two in-order streams with event waits that
    bind to the most recent record at enqueue time.  Returns per-op
    (start, end) and checks slot safety and coverage."""
    t_copy = t_comp = 0.0
    rec_ready, rec_cons = {}, {}        # event -> op index of its latest record (host order)
    times = []
    slot_owner = {}                     # slot -> (call index, layer, o, copy end time)
    slot_readers_end = {}               # slot -> latest end time of a compute reading it
    call = 0
    copied = {}                         # (call_of_layer, layer) -> set of o
    seen_calls = []                     # layer of each call, in order of first compute
    layer_call = {}                     # layer -> call index currently served
    busy = 0.0
    first_copy = last_copy = None
    for i, (kind, layer, first, count, base, ev, wait) in enumerate(ops):
        if kind == BEGIN:
            times.append((t_comp, t_comp))
            continue
        if kind == DRAIN:
            t = max(t_copy, t_comp)
            t_copy = t_comp = t
            times.append((t, t))
            continue
        if kind == COPY:
            dep = times[rec_cons[wait]][1] if wait >= 0 else 0.0
            start = max(t_copy, dep)
            end = start + copy_cost * count
            t_copy = end
            busy += end - start
            first_copy = start if first_copy is None else first_copy
            last_copy = end
            for o in range(first, first + count):
                s = (base + o) % n_slots
                # the slot's previous content must have been read completely
                assert slot_readers_end.get(s, 0.0) <= start, f"op {i}: slot {s} overwritten while in use"
                slot_owner[s] = (layer, o, base, end)
                slot_readers_end[s] = 0.0
            rec_ready[ev] = i
            times.append((start, end))
            continue
        # compute-stream ops
        if kind == RESIDENT:
            seen_calls.append(layer)
            layer_call[layer] = len(seen_calls) - 1
            start = t_comp
            end = start + compute_cost
        elif kind == COMPUTE:
            dep = times[rec_ready[ev]][1]
            start = max(t_comp, dep)
            end = start + compute_cost * count
            for o in range(first, first + count):
                s = (base + o) % n_slots
                owner = slot_owner.get(s)
                assert owner is not None and owner[:3] == (layer, o, base), f"op {i}: slot {s} holds {owner}"
                assert owner[3] <= start, f"op {i}: read before the copy finished"
                slot_readers_end[s] = max(slot_readers_end[s], end)
                key = (layer_call[layer], layer)
                copied.setdefault(key, []).append(o)
            rec_cons[ev] = i
        else:  # MERGE
            start = t_comp
            end = start + compute_cost
            key = (layer_call[layer], layer)
            got = sorted(copied.get(key, []))
            assert got == list(range(counts[layer])), f"layer {layer}: pages read {got[:5]}..."
        t_comp = end
        times.append((start, end))
    util = busy / (last_copy - first_copy) if last_copy else 1.0
    return times, util, seen_calls


@pytest.mark.parametrize("n_slots,chunk,counts", [
    (64, 16, [614] * 8),          # the streamed workload's shape, 8 layers
    (5, 2, [11, 12, 0, 7]),
    (8, 3, [10, 0, 5, 7]),
    (7, 7, [3, 1, 9]),
    (16, 1, [40, 40]),
])
def test_planner_in_order_passes(n_slots, chunk, counts):
    L = len(counts)
    calls = [l for _ in range(3) for l in range(L)]
    ops = kv.sched_simulate(L, n_slots, chunk, counts, calls)
    times, util, seen = simulate(ops, n_slots, counts)
    streamed_calls = [l for l in calls if counts[l]]
    assert seen == streamed_calls
    assert not any(op[0] == DRAIN for op in ops)  # in-order calls never drain
    # copies are slower than compute, so with room for two chunks in the ring
    # the copy stream never idles (a one-chunk ring must wait for each consumer)
    if 2 * chunk <= n_slots:
        assert util >= 0.999, util
    # lookahead: a copy is enqueued at most one streamed layer past the layer
    # whose call began last (instances counted in call order)
    active = copy_seq = -1
    for op in ops:
        if op[0] == BEGIN:
            active += 1
        if op[0] == COPY:
            if op[2] == 0:
                copy_seq += 1
            assert copy_seq <= active + 1, f"copy {op} runs more than one layer ahead"


def test_planner_out_of_order_drains_and_stays_correct():
    counts = [9, 4, 6]
    calls = [0, 1, 2, 0, 2, 1, 1, 0, 2, 0]
    ops = kv.sched_simulate(3, 4, 2, counts, calls)
    simulate(ops, 4, counts)
    assert any(op[0] == DRAIN for op in ops)


def test_planner_chunks_cover_two_spans_at_wrap():
    ops = kv.sched_simulate(1, 10, 4, [13], [0, 0])
    copies = [op for op in ops if op[0] == COPY]
    spans = []
    for _, _, first, count, base, _, _ in copies:
        slots = [(base + o) % 10 for o in range(first, first + count)]
        runs = 1 + sum(1 for a, b in zip(slots, slots[1:]) if b != a + 1)
        spans.append(runs)
    assert max(spans) == 2 and min(spans) == 1
