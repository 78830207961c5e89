"""GPU tests of the KV writer (kvattn_append): every code and scale of every
page it touches is compared with the oracle's quantiser (bit-exact), the rest
of those pages must be unchanged, and attention over the grown history must
match the oracle."""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
import oracle
from gpu_util import TOL, handle, oracle_out, place, run, say

pytestmark = pytest.mark.gpu


def rows(R, Hkv, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(R, Hkv, 128, generator=g) * scale
    v = torch.randn(R, Hkv, 128, generator=g) * scale
    return k, v


def unpack_all(h, layer, n_pages, Hkv):
    return [oracle.unpack_page(h.debug_read_page(layer, P), Hkv, 256) for P in range(n_pages)]


CASES = [
    # N0, R, Hkv
    (300, 1, 8),       # one row into the middle of a 32-token tile
    (31, 2, 2),        # the row pair straddles a tile boundary
    (250, 37, 4),      # crosses a page boundary: one new page
    (256, 256, 8),     # page-aligned growth by a whole page
    (1000, 600, 2),    # several tiles and pages
]


@pytest.mark.parametrize("N0,R,Hkv", CASES)
def test_append_bitexact(N0, R, Hkv):
    say(f"case append N0={N0} R={R} Hkv={Hkv}")
    kvl = inputs.draw_layer(N0, Hkv, 0, 90 + R % 7, pad="garbage")
    n0 = kvl.pages.shape[0]
    n1 = -(-(N0 + R) // 256)
    n_pool = n1 + 4
    h = handle(Hkv * 5, Hkv, n_pool, n1 + 1, 8)
    rng = np.random.default_rng(N0 + R)
    ids = rng.permutation(n_pool)[:n1].astype(np.uint32)
    place(h, 0, kvl, ids[:n0])
    # garbage in the pool pages the growth will use (the writer must not rely on zeros)
    pb = kv.page_bytes(h.params)
    for i in ids[n0:]:
        h.pool[int(i) * pb:(int(i) + 1) * pb].copy_(torch.randint(0, 256, (pb,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    before = unpack_all(h, 0, n0, Hkv)
    k, v = rows(R, Hkv, N0 * 7 + R)
    h.append(0, k.cuda(), v.cuda(), R, ids[n0:])
    h.synchronize()
    after = unpack_all(h, 0, n1, Hkv)
    ekc, ekd = oracle.quantize_q8_0(k.numpy())
    evc, evd = oracle.quantize_q4_0(v.numpy())
    for P in range(n1):
        kc, kd, vc, vd = after[P]
        for j in range(256):
            pos = P * 256 + j
            if N0 <= pos < N0 + R:
                r = pos - N0
                assert np.array_equal(kc[j], ekc[r]), (P, j)
                assert np.array_equal(kd[j], ekd[r]), (P, j)
                assert np.array_equal(vc[j], evc[r]), (P, j)
                assert np.array_equal(vd[j], evd[r]), (P, j)
            elif P < n0:
                for a, b in zip(after[P], before[P]):
                    assert np.array_equal(a[j], b[j]), ("changed", P, j)
    h.destroy()


def test_append_then_attention_and_publish():
    """Grow a 3,000-token layer by a 100-row chunk (new page included), run
    the prefill chunk over the grown history and a decode after one more
    appended row; the published host copy equals the device pages."""
    N0, R, Hq, Hkv = 3000, 100, 40, 8
    say(f"case append+attention N0={N0} R={R}")
    kvl = inputs.draw_layer(N0, Hkv, 0, 95)
    n0 = kvl.pages.shape[0]
    n1 = -(-(N0 + R + 1) // 256)
    h = handle(Hq, Hkv, n1 + 2, n1, 128)
    ids = np.arange(n1, dtype=np.uint32)[::-1].copy()
    place(h, 0, kvl, ids[:n0])
    pb = kv.page_bytes(h.params)
    hist = torch.zeros((n1, pb), dtype=torch.uint8).pin_memory()
    k, v = rows(R + 1, Hkv, 5)
    grow = -(-(N0 + R) // 256) - n0
    h.append(0, k[:R].cuda(), v[:R].cuda(), R, ids[n0:n0 + grow], publish=hist)
    q = inputs.draw_queries(R, Hq, 0, 95)
    got = run(h, 0, q, R, "prefill")
    pages = np.stack([h.debug_read_page(0, P) for P in range(n0 + grow)])
    ref, _ = oracle.attend_paged(np.arange(len(pages), dtype=np.uint32), N0 + R, 256, Hq, Hkv, q.numpy(),
                                 inputs.scale_for(), pool=pages)
    err = np.max(np.abs(got - ref))
    say(f"  prefill over grown history: max-abs err {err:.3e}")
    assert err <= TOL
    h.synchronize()
    for P in range(N0 // 256, n0 + grow):
        assert np.array_equal(hist[P].numpy(), pages[P]), P
    # one more row, then a decode step
    grow2 = n1 - (n0 + grow)
    h.append(0, k[R:].cuda(), v[R:].cuda(), 1, ids[n0 + grow:n0 + grow + grow2])
    q1 = inputs.draw_queries(1, Hq, 1, 95)
    got1 = run(h, 0, q1, 1, "decode")
    pages = np.stack([h.debug_read_page(0, P) for P in range(n1)])
    ref1, _ = oracle.attend_paged(np.arange(n1, dtype=np.uint32), N0 + R + 1, 256, Hq, Hkv, q1.numpy(),
                                  inputs.scale_for(), pool=pages)
    err1 = np.max(np.abs(got1 - ref1))
    say(f"  decode after one more row: max-abs err {err1:.3e}")
    assert err1 <= TOL
    h.destroy()


def test_append_rejections():
    Hkv = 2
    kvl = inputs.draw_layer(300, Hkv, 0, 96)
    h = handle(10, Hkv, 8, 3, 8, n_ring=4)
    place(h, 0, kvl, np.array([0, 1], dtype=np.uint32))
    k, v = rows(300, Hkv, 1)
    kd, vd = k.cuda(), v.cuda()
    with pytest.raises(kv.KVAttnError) as e:          # 300 more rows need one more page
        h.append(0, kd, vd, 300, None)
    assert e.value.code == kv.E_ARG
    with pytest.raises(kv.KVAttnError) as e:          # the new page must be a pool page
        h.append(0, kd, vd, 300, [kv.PT_RING_FLAG | 1])
    assert e.value.code == kv.E_ARG
    with pytest.raises(kv.KVAttnError) as e:          # beyond max_pages_per_layer (3)
        h.append(0, kd, vd, 600, [2, 3, 4])
    assert e.value.code == kv.E_NOSPACE
    with pytest.raises(kv.KVAttnError) as e:          # names a page the layer already uses
        h.append(0, kd, vd, 300, [1])
    assert e.value.code == kv.E_PLAN
    # a streamed tail page cannot take new rows
    host = kvl.pages.contiguous().pin_memory()
    h2 = handle(10, Hkv, 8, 3, 8, n_ring=4, n_layers=1)
    place(h2, 0, kvl, np.array([0, kv.PT_HOST], dtype=np.uint32), history=host)
    with pytest.raises(kv.KVAttnError) as e:
        h2.append(0, kd[:1], vd[:1], 1, None)
    assert e.value.code == kv.E_UNSUPPORTED
    h.destroy()
    h2.destroy()


@pytest.mark.parametrize("W", [1, 4])
def test_append_decode_loop_on_streamed_layer(W):
    """The serving loop on a layer that streams most of its history: each
    step appends W rows into the resident tail (a new pool page when a page
    fills), publishes the touched pages into the pinned host history the
    scheduler streams from, and attends over the grown history through the
    ring.  The eight steps cross a page boundary; every step's output is
    compared with the oracle over the published history."""
    N0, Hq, Hkv, T = 12 * 256 - 5, 40, 8, 256
    steps = 8
    n_max = -(-(N0 + steps * W + 256) // T)
    say(f"case append loop on a streamed layer N0={N0} W={W} steps={steps}")
    kvl = inputs.draw_layer(N0, Hkv, 0, 96)
    n0 = kvl.pages.shape[0]
    rng = np.random.default_rng(96)
    # the tail page and a third of the others resident; the rest stream
    res = np.sort(np.append(rng.choice(n0 - 1, (n0 - 1) // 3, replace=False), n0 - 1))
    table = np.full(n0, kv.PT_HOST, dtype=np.uint32)
    table[res] = np.arange(len(res))
    h = handle(Hq, Hkv, len(res) + n_max, n_max, 8, n_ring=5, chunk_slots=2)
    pb = kv.page_bytes(h.params)
    hist = torch.zeros((n_max, pb), dtype=torch.uint8).pin_memory()
    hist[:n0].copy_(kvl.pages)
    place(h, 0, kvl, table, history=hist)
    next_pool = len(res)
    n_tokens = N0
    k, v = rows(steps * W, Hkv, 97)
    for s in range(steps):
        new_pages = -(-(n_tokens + W) // T) - (-(-n_tokens // T))
        ids = np.arange(next_pool, next_pool + new_pages, dtype=np.uint32)
        next_pool += new_pages
        h.append(0, k[s * W:(s + 1) * W].cuda(), v[s * W:(s + 1) * W].cuda(), W, ids, publish=hist)
        n_tokens += W
        q = inputs.draw_queries(W, Hq, s, 96)
        got = run(h, 0, q, W, "verify")
        n_pages = -(-n_tokens // T)
        ref, _ = oracle.attend_paged(np.arange(n_pages, dtype=np.uint32), n_tokens, T, Hq, Hkv, q.numpy(),
                                     inputs.scale_for(), pool=hist[:n_pages].numpy())
        err = float(np.max(np.abs(got - ref)))
        say(f"  step {s}: {n_tokens} tokens, {new_pages} new pages, max-abs err {err:.3e}")
        assert np.isfinite(got).all()
        assert err <= TOL
    h.destroy()
