"""GPU: the streaming schedule checked on the device by ring-slot tags.

kvattn_debug_check_ring tags every ring slot a streamed chunk fills with the
page's global ordinal once its copy has finished (copy stream), and checks
the tags of the chunk's slots just before and just after the launch that
reads them (compute stream).  A slot read before its copy finished, or
refilled before its reader finished, would hold another ordinal.  These
tests drive streamed layers through small and full-size rings, in order,
out of order and at several widths, and require no mismatch, the expected
number of checks, and outputs within the bar of the fp64 oracle; a run with
skewed tags shows that the check fires.
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu


def streamed_handle(layers, Hq, Hkv, max_rows, ring, chunk, frac, seed):
    n = layers[0].pages.shape[0]
    n_res = int(round(frac * n))
    h = handle(Hq, Hkv, len(layers) * max(n_res, 1), n, max_rows, n_ring=ring, chunk_slots=chunk,
               n_layers=len(layers))
    streamed = []
    for l, x in enumerate(layers):
        res = np.sort(np.random.default_rng(seed + l).choice(n, n_res, replace=False))
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        table[res] = l * max(n_res, 1) + np.arange(n_res)
        place(h, l, x, table, history=x.pages.contiguous().pin_memory())
        streamed.append(n - n_res)
    return h, streamed


def call(h, layer, q, W):
    qd = q.cuda().contiguous()
    out = torch.full_like(qd, float("nan"))
    h.verify(layer, qd, W, out)
    return out


def test_ring_tags_small_ring_orders_and_widths():
    """Two ragged layers (30 pages, 40 % resident, 18 streamed each) through
    a 6-slot ring in chunks of 3: three passes in order at W = 1, 4 and 49,
    then calls out of order (1, 0, 0), each output against the oracle."""
    Hq, Hkv, N = 40, 8, 30 * 256 - 77
    layers = [inputs.draw_layer(N, Hkv, l, 150, pad="garbage") for l in range(2)]
    h, streamed = streamed_handle(layers, Hq, Hkv, 49, 6, 3, 0.4, 150)
    counters = torch.zeros(2, dtype=torch.int32, device="cuda")
    h.check_ring(counters)
    pages = 0
    for W, seq in [(1, [0, 1, 0, 1, 0, 1]), (4, [0, 1, 0, 1]), (49, [0, 1, 0, 1]), (4, [1, 0, 0])]:
        say(f"case ring tags N={N} W={W} calls {seq}: ring 6, chunk 3")
        qs = [inputs.draw_queries(W, Hq, l, 150 + W) for l in range(2)]
        refs = [oracle_out(layers[l], qs[l], Hq, Hkv) for l in range(2)]
        for l in seq:
            got = call(h, l, qs[l], W)
            h.synchronize()
            err = float(np.max(np.abs(got.cpu().double().numpy() - refs[l])))
            assert err <= TOL, (W, l, err)
            pages += streamed[l]
    c = counters.cpu().numpy()
    say(f"  tag mismatches {c[0]}, slot checks {c[1]} (streamed pages computed {pages})")
    assert c[0] == 0
    assert c[1] == 2 * pages
    h.check_ring(None)
    h.destroy()


def test_ring_tags_skew_shows_the_check_fires():
    """Tags written one generation off: every check must count a mismatch."""
    Hq, Hkv, N = 40, 8, 20 * 256 - 5
    layers = [inputs.draw_layer(N, Hkv, l, 151) for l in range(2)]
    h, streamed = streamed_handle(layers, Hq, Hkv, 8, 5, 2, 0.3, 151)
    counters = torch.zeros(2, dtype=torch.int32, device="cuda")
    h.check_ring(counters, skew=1)
    qs = [inputs.draw_queries(1, Hq, l, 151) for l in range(2)]
    for l in (0, 1, 0):
        call(h, l, qs[l], 1)
    h.synchronize()
    c = counters.cpu().numpy()
    say(f"case ring tags skewed: mismatches {c[0]} of {c[1]} checks")
    assert c[1] == 2 * (streamed[0] * 2 + streamed[1])
    assert c[0] == c[1]
    h.check_ring(None)
    h.destroy()


def test_ring_tags_full_size():
    """stream-256k geometry (262,144 tokens, 410 resident pages, 614 streamed
    through 64 slots in chunks of 16), two layers, two passes in order at
    W = 4: no mismatch over 4 x 614 x 2 slot checks; sampled rows of the last
    pass against the oracle."""
    import oracle
    w = inputs.WORKLOADS["stream-256k"]
    L, W = 2, 4
    say(f"case ring tags full size {w.name} W={W}: {L} layers x 2 passes")
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
    counters = torch.zeros(2, dtype=torch.int32, device="cuda")
    h.check_ring(counters)
    outs = None
    for _ in range(2):
        outs = [call(h, l, qs[l], W) for l in range(L)]
    h.synchronize()
    c = counters.cpu().numpy()
    say(f"  tag mismatches {c[0]}, slot checks {c[1]}")
    assert c[0] == 0
    assert c[1] == 2 * 2 * L * (n - w.n_resident)
    rows = [0, W - 1]
    for l in range(L):
        ref, _ = oracle.attend_paged(np.arange(n, dtype=np.uint32), w.n_tokens, 256, w.n_q_heads, w.n_kv_heads,
                                     qs[l].cpu().numpy(), inputs.scale_for(), pool=hosts[l].numpy(), rows=rows)
        err = float(np.max(np.abs(outs[l].cpu().double().numpy()[rows] - ref)))
        say(f"  layer {l} rows {rows}: max-abs err {err:.3e}")
        assert err <= TOL
    h.check_ring(None)
    h.destroy()
