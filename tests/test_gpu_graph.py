"""GPU: attention and writer calls captured into a HIP graph and replayed.

The handle computes on a stream of its own (capture needs one other than the
default stream), and its calls enqueue only kernel launches there (no
memsets, no host round trips), so a captured pass must give, on every
replay, what the same calls give eagerly: bit for bit with a fixed chunk
order, within the fp64 oracle's tolerance with the claimed chunk order.
Each test replays several times with eager work of the library and of torch,
and synchronisations, between the replays, and checks every replay.
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
import oracle
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _queries(rows, Hq, seed):
    return inputs.draw_queries(rows, Hq, seed, 61).to("cuda").contiguous()


def _calls(h, layer, qs, outs):
    h.decode(layer, qs[0], outs[0])
    h.verify(layer, qs[1], qs[1].shape[0], outs[1])
    h.verify(layer, qs[2], qs[2].shape[0], outs[2])
    h.prefill_chunk(layer, qs[3], qs[3].shape[0], outs[3])


@pytest.mark.parametrize("deterministic", [1, 0], ids=["fixed-order", "claimed-order"])
def test_graph_replay_attention(deterministic):
    # 40 pages with 12-page splits: the long splits take the claimed chunk
    # order when the handle is not deterministic; ragged last page.
    N, Hq, Hkv, sp = 40 * 256 - 19, 8, 2, 12
    say(f"case graph attention N={N} Hq={Hq} Hkv={Hkv} split_pages={sp} deterministic={deterministic}")
    kvl = inputs.draw_layer(N, Hkv, 0, 61)
    n = kvl.pages.shape[0]
    table = np.random.default_rng(5).permutation(n).astype(np.uint32)
    h = handle(Hq, Hkv, n, n, 64, split_pages=sp, deterministic=deterministic, compute_stream=torch.cuda.Stream())
    place(h, 0, kvl, table)
    # 4, 12, 40 (two 32-row blocks) and 256 (wide kernel) rows per KV head
    qs = [_queries(1, Hq, 0), _queries(3, Hq, 1), _queries(10, Hq, 4), _queries(64, Hq, 2)]
    refs = [oracle_out(kvl, q.cpu(), Hq, Hkv) for q in qs]

    stream = h.compute_stream
    eager = [torch.full_like(q, float("nan")) for q in qs]
    with torch.cuda.stream(stream):
        _calls(h, 0, qs, eager)
    torch.cuda.synchronize()
    for e, r in zip(eager, refs):
        assert np.abs(e.cpu().double().numpy() - r).max() < TOL

    outs = [torch.full_like(q, float("nan")) for q in qs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        _calls(h, 0, qs, outs)
    torch.cuda.synchronize()

    side = [torch.empty_like(q) for q in qs]
    x = torch.randn(256, 256, device="cuda")
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for k, (o, e, r) in enumerate(zip(outs, eager, refs)):
            got = o.cpu()
            assert torch.isfinite(got).all(), f"replay {i} call {k}: unwritten outputs"
            if deterministic:
                assert torch.equal(got, e.cpu()), f"replay {i} call {k} differs from the eager call"
            else:
                assert np.abs(got.double().numpy() - e.cpu().double().numpy()).max() < TOL
            assert np.abs(got.double().numpy() - r).max() < TOL, f"replay {i} call {k}"
        # eager work between replays: the same calls into other buffers, and torch's own kernels
        with torch.cuda.stream(stream):
            _calls(h, 0, qs, side)
            x = torch.tanh(x @ x)
        torch.cuda.synchronize()
    h.destroy()


def test_graph_replay_append_then_decode():
    # Five new rows land in the slack of the last page (no new pages), then a
    # decode reads them; the graph holds both.  Before each replay the pool
    # is put back to its state before the append, so each replay redoes it.
    N, Hq, Hkv, R = 3 * 256 - 40, 8, 2, 5
    say(f"case graph append+decode N={N} R={R} Hq={Hq} Hkv={Hkv}")
    kvl = inputs.draw_layer(N, Hkv, 0, 62)
    n = kvl.pages.shape[0]
    table = np.array([2, 0, 1], dtype=np.uint32)
    h = handle(Hq, Hkv, n, n, 8, split_pages=1, deterministic=1, compute_stream=torch.cuda.Stream())
    place(h, 0, kvl, table)
    saved = h.pool.clone()
    g = torch.Generator(device="cuda").manual_seed(62)
    k = torch.randn(R, Hkv, 128, device="cuda", generator=g)
    v = torch.randn(R, Hkv, 128, device="cuda", generator=g)
    q = _queries(1, Hq, 3)
    stream = h.compute_stream

    out_e = torch.full_like(q, float("nan"))
    with torch.cuda.stream(stream):
        h.append(0, k, v, R)
        h.decode(0, q, out_e)
    torch.cuda.synchronize()
    page_e = h.debug_read_page(0, n - 1)
    out_e = out_e.cpu()

    h.pool.copy_(saved)
    h.set_layer(0, table, N)
    torch.cuda.synchronize()
    out_g = torch.full_like(q, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        h.append(0, k, v, R)
        h.decode(0, q, out_g)
    torch.cuda.synchronize()

    side = torch.empty_like(q)
    for i in range(REPLAYS):
        h.pool.copy_(saved)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h.debug_read_page(0, n - 1), page_e), f"replay {i}: written page differs"
        assert torch.equal(out_g.cpu(), out_e), f"replay {i}: decode after the append differs"
        with torch.cuda.stream(stream):
            h.decode(0, q, side)
        torch.cuda.synchronize()
        assert torch.equal(side.cpu(), out_e)
    h.destroy()


def test_graph_replay_append_crossing_page():
    """An append whose rows cross into a new page, captured with a decode:
    the new page's device entries come from a launch on the compute stream
    (no drain, no host copy: capture would reject either).  Before each
    replay the pool is restored and the layer is set with a decoy page in
    the new slot of the table, so a replay that did not write the entry
    would read the decoy; every replay must equal the eager calls bit for
    bit, and the eager result the oracle over the written pages."""
    N, Hq, Hkv, R = 2 * 256 - 3, 8, 2, 5
    say(f"case graph append across a page N={N} R={R} Hq={Hq} Hkv={Hkv}")
    kvl = inputs.draw_layer(N, Hkv, 0, 63)
    n = kvl.pages.shape[0]
    table = np.array([1, 0], dtype=np.uint32)
    new_page, decoy = 3, 2
    h = handle(Hq, Hkv, 4, 4, 8, split_pages=1, deterministic=1, compute_stream=torch.cuda.Stream())
    place(h, 0, kvl, table)
    pb = kv.page_bytes(h.params)
    h.pool[decoy * pb:(decoy + 1) * pb].copy_(inputs.draw_layer(256, Hkv, 1, 63).pages[0].cuda())
    saved = h.pool.clone()
    g = torch.Generator(device="cuda").manual_seed(63)
    k = torch.randn(R, Hkv, 128, device="cuda", generator=g)
    v = torch.randn(R, Hkv, 128, device="cuda", generator=g)
    q = _queries(1, Hq, 7)
    stream = h.compute_stream

    out_e = torch.full_like(q, float("nan"))
    with torch.cuda.stream(stream):
        h.append(0, k, v, R, new_pages=[new_page])
        h.decode(0, q, out_e)
    torch.cuda.synchronize()
    pages_e = np.stack([h.debug_read_page(0, P) for P in range(n + 1)])
    out_e = out_e.cpu()
    ref, _ = oracle.attend_paged(np.arange(n + 1, dtype=np.uint32), N + R, 256, Hq, Hkv, q.cpu().numpy(),
                                 inputs.scale_for(), pool=pages_e)
    err = float(np.max(np.abs(out_e.double().numpy() - ref)))
    say(f"  eager append + decode vs oracle: max-abs err {err:.3e}")
    assert err <= TOL

    h.pool.copy_(saved)
    h.set_layer(0, table, N)
    torch.cuda.synchronize()
    out_g = torch.full_like(q, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        h.append(0, k, v, R, new_pages=[new_page])
        h.decode(0, q, out_g)
    torch.cuda.synchronize()

    for i in range(REPLAYS):
        h.pool.copy_(saved)
        h.set_layer(0, np.append(table, decoy).astype(np.uint32), N + R)
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.cpu(), out_e), f"replay {i}: decode after the append differs"
        h.set_layer(0, np.append(table, new_page).astype(np.uint32), N + R)
        for P in range(n + 1):
            assert np.array_equal(h.debug_read_page(0, P), pages_e[P]), f"replay {i}: page {P} differs"
    h.destroy()
