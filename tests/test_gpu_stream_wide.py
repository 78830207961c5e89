"""GPU parity of streamed layers at widths beyond one 32-row block.

A call with more than 32 rows per KV head on a layer with streamed pages
runs the same kernels as a resident call of that width (two or three
32-row blocks of the split kernel, or the wide kernel) over every staged
span, one page per split, all row blocks reading a chunk before its ring
slots are released; the split partials accumulate into a fixed set of slots
across the launches.  Every test compares with the fp64 oracle reading the
same page bytes (all rows, or sampled rows at full size).
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
import oracle
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu

Q8, Q4, F16 = inputs.Q8_0, inputs.Q4_0, inputs.F16


def streamed_handle(layers, Hq, Hkv, max_rows, ring, chunk, frac, seed, k_type=Q8, v_type=Q4):
    """Layers whose pages are a seeded `frac` resident, the rest streamed
    from pinned histories through `ring` slots in chunks of `chunk`."""
    n = layers[0].pages.shape[0]
    n_res = int(round(frac * n))
    h = handle(Hq, Hkv, len(layers) * max(n_res, 1), n, max_rows, n_ring=ring, chunk_slots=chunk,
               n_layers=len(layers), k_type=k_type, v_type=v_type)
    for l, x in enumerate(layers):
        res = np.sort(np.random.default_rng(seed + l).choice(n, n_res, replace=False))
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        table[res] = l * max(n_res, 1) + np.arange(n_res)
        place(h, l, x, table, history=x.pages.contiguous().pin_memory())
    return h


def run_call(h, layer, q, W, kind):
    qd = q.cuda().contiguous()
    out = torch.full_like(qd, float("nan"))
    (h.prefill_chunk if kind == "prefill" else h.verify)(layer, qd, W, out)
    return out


# W, kind: 35 and 95 rows per KV head (split kernel, two and three 32-row
# blocks), 125 and 245 (wide kernel, 256-row blocks), prefill 64 rows of
# 40 heads (320 rows per KV head: a 384-row 12-wave block) and 256 rows
# (1,280 rows per KV head: four 384-row blocks)
WIDTHS = [(7, "verify"), (19, "verify"), (25, "verify"), (49, "verify"), (64, "prefill"), (256, "prefill")]


@pytest.mark.parametrize("W,kind", WIDTHS, ids=[f"{k}-{w}" for w, k in WIDTHS])
def test_streamed_wide_small(W, kind):
    """Two ragged layers (30 pages, 40 % resident) through a 6-slot ring in
    chunks of 3, called in order twice (the second pass reuses the slots and
    the accumulating partials)."""
    Hq, Hkv, N = 40, 8, 30 * 256 - 77
    say(f"case streamed wide N={N} W={W} {kind}: ring 6, chunk 3, 2 layers x 2 passes")
    layers = [inputs.draw_layer(N, Hkv, l, 140, pad="garbage") for l in range(2)]
    qs = [inputs.draw_queries(W, Hq, l, 140) for l in range(2)]
    h = streamed_handle(layers, Hq, Hkv, W, 6, 3, 0.4, 140)
    refs = [oracle_out(layers[l], qs[l], Hq, Hkv) for l in range(2)]
    for rep in range(2):
        outs = [run_call(h, l, qs[l], W, kind) for l in range(2)]
        h.synchronize()
        for l in range(2):
            got = outs[l].cpu().double().numpy()
            err = float(np.max(np.abs(got - refs[l])))
            say(f"  pass {rep} layer {l}: max-abs err {err:.3e}")
            assert np.isfinite(got).all()
            assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("kt,vt", [(Q8, Q8), (Q4, Q4), (F16, F16)], ids=["q8_0-q8_0", "q4_0-q4_0", "f16-f16"])
@pytest.mark.parametrize("W", [10, 49])
def test_streamed_wide_pairs(W, kt, vt):
    Hq, Hkv, N = 40, 8, 20 * 256 - 5
    say(f"case streamed wide pair {kt}/{vt} N={N} W={W}")
    layers = [inputs.draw_layer(N, Hkv, 0, 141, k_type=kt, v_type=vt, pad="garbage")]
    q = inputs.draw_queries(W, Hq, 0, 141)
    h = streamed_handle(layers, Hq, Hkv, W, 5, 2, 0.3, 141, k_type=kt, v_type=vt)
    got = run_call(h, 0, q, W, "verify")
    h.synchronize()
    err = float(np.max(np.abs(got.cpu().double().numpy() - oracle_out(layers[0], q, Hq, Hkv))))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


def test_streamed_width_moves_no_more_bytes():
    """The ring schedule of a streamed layer does not depend on the width:
    the same chunks are copied for W = 1 and W = 49 (observed copy events)."""
    Hq, Hkv, N = 40, 8, 24 * 256
    say(f"case streamed copies W=1 vs W=49 N={N}")
    layers = [inputs.draw_layer(N, Hkv, l, 142) for l in range(2)]
    h = streamed_handle(layers, Hq, Hkv, 49, 6, 3, 0.25, 142)
    chunks = {}
    for W in (1, 49):
        q = [inputs.draw_queries(W, Hq, l, 142) for l in range(2)]
        for l in range(2):
            run_call(h, l, q[l], W, "verify")   # warm the schedule at this width
        h.synchronize()
        h.observe(1 << 10)
        for l in range(2):
            run_call(h, l, q[l], W, "verify")
        ob = h.observe_read(N)
        h.observe(0)
        chunks[W] = int(ob.chunks)
        say(f"  W={W}: {chunks[W]} streamed chunks computed in one pass of 2 layers")
    # 18 streamed pages per layer in chunks of 3: 12 chunks per pass (copies
    # prefetched before the observation began are not counted)
    assert 0 < chunks[1] == chunks[49] <= 2 * 6
    h.destroy()


@pytest.mark.parametrize("W,kind", [(49, "verify"), (256, "prefill")], ids=["verify-49", "prefill-256"])
def test_full_size_streamed_wide(W, kind):
    """stream-256k geometry (262,144 tokens, 410 resident pages, 614 streamed
    through 64 slots, default chunk size), two layers set before the first
    call; 8 sampled rows (first, last, 6 seeded) of each layer against the
    oracle, every output finite."""
    w = inputs.WORKLOADS["stream-256k"]
    L = 2
    say(f"case full-size {w.name} W={W} {kind}: {L} layers, 8 sampled rows each")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, L * w.n_resident, n, W, n_ring=w.ring_slots, n_layers=L)
    pb = kv.page_bytes(h.params)
    hosts, qs = [], []
    for l in range(L):
        kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, l, w.wid, device="cuda")
        res = inputs.resident_subset(n, w.n_resident, l, w.wid)
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        table[res] = l * w.n_resident + np.arange(len(res))
        host = torch.empty((n, pb), dtype=torch.uint8, pin_memory=True)
        host.copy_(kvl.pages)
        place(h, l, kvl, table, history=host)
        hosts.append(host)
        qs.append(inputs.draw_queries(W, w.n_q_heads, l, w.wid, device="cuda"))
        del kvl
    outs = [run_call(h, l, qs[l], W, kind) for l in range(L)]
    h.synchronize()
    rng = np.random.default_rng(143)
    rows = sorted({0, W - 1, *rng.choice(W, 6, replace=False).tolist()})
    for l in range(L):
        got = outs[l].cpu().double().numpy()
        assert np.isfinite(got).all()
        ref, _ = oracle.attend_paged(np.arange(n, dtype=np.uint32), w.n_tokens, 256, w.n_q_heads, w.n_kv_heads,
                                     qs[l].cpu().numpy(), inputs.scale_for(), pool=hosts[l].numpy(), rows=rows)
        err = float(np.max(np.abs(got[rows] - ref)))
        say(f"  layer {l} rows {rows}: max-abs err {err:.3e}")
        assert err <= TOL
    h.destroy()
