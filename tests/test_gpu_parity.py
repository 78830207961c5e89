"""GPU parity: the HIP path through the C-ABI against the fp64 oracle.

Tolerance: max-abs 2e-3 over every output element (fp32 accumulation; Q and
P rounded to binary16 for the matrix cores).  Page-table and index handling
is checked bit-exactly (debug page reads, bitwise invariance across
placements at a fixed split plan).
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
import oracle
from gpu_util import TOL, handle, oracle_out, place, run, say

pytestmark = pytest.mark.gpu


def layer_kv(N, Hkv, wid=50, layer=0, pad="zero"):
    return inputs.draw_layer(N, Hkv, layer, wid, pad=pad)


def perm_table(n, seed):
    return np.random.default_rng(seed).permutation(n).astype(np.uint32)


# ------------------------------------------------------------------ tiny workload
def test_tiny_workload_decode():
    w = inputs.WORKLOADS["tiny-2k"]
    say(f"case tiny-2k decode N={w.n_tokens} Hq={w.n_q_heads} Hkv={w.n_kv_heads}")
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 0, w.wid)
    q = inputs.draw_queries(1, w.n_q_heads, 0, w.wid)
    table = inputs.seeded_permutation(w.n_pages, 0, w.wid)
    h = handle(w.n_q_heads, w.n_kv_heads, w.n_pages, w.n_pages, 8)
    # upload through the C-ABI (host pages in pool order)
    order = np.argsort(table)
    host = kvl.pages[torch.from_numpy(order)].contiguous().pin_memory()
    h.upload_pages(host, np.arange(w.n_pages, dtype=np.uint32))
    h.set_layer(0, table, w.n_tokens)
    got = run(h, 0, q, 1, "decode")
    ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


# ------------------------------------------------------------------ shape sweep
CASES = [
    # N, Hq, Hkv, W, kind, split_pages
    (2048 - 37, 4, 1, 1, "decode", 0),
    (1, 4, 1, 1, "decode", 0),
    (31, 8, 2, 1, "decode", 0),
    (33, 8, 2, 6, "verify", 0),
    (300, 40, 8, 1, "decode", 0),
    (300, 40, 8, 2, "verify", 0),
    (300, 40, 8, 3, "verify", 1),
    (300, 40, 8, 4, "verify", 2),
    (300, 40, 8, 5, "verify", 0),
    (300, 40, 8, 6, "verify", 0),
    (5000, 40, 8, 6, "verify", 3),
    (5000, 40, 8, 1, "decode", 7),
    (7 * 256, 40, 8, 4, "verify", 0),
    (6, 8, 1, 6, "verify", 0),          # every key a verify row
    (256 + 700, 40, 8, 256, "prefill", 0),
    (1000, 8, 1, 100, "prefill", 0),
    (256, 16, 2, 256, "prefill", 0),     # row 0 sees one key
    (3000, 40, 8, 37, "prefill", 0),
    (5000, 40, 8, 7, "verify", 0),      # 35 rows per KV head: two 32-row blocks of the split kernel
    (5000, 40, 8, 12, "verify", 0),     # 60 rows, two blocks
    (3000, 8, 1, 5, "verify", 0),       # 40 rows, one KV head
    (1500, 8, 8, 40, "verify", 0),      # G = 1: 40 rows of distinct positions
    (2000, 16, 2, 8, "prefill", 0),     # 64 rows as a prefill chunk
    (700, 40, 8, 7, "verify", 1),       # two blocks: split_pages applies to one-block calls only
    (5000, 40, 8, 13, "verify", 0),     # 65 rows: three blocks
    (5000, 40, 8, 19, "verify", 0),     # 95 rows: three blocks
    (5000, 40, 8, 20, "verify", 0),     # 100 rows: the wide kernel
    (100 * 256 - 17, 40, 8, 4, "verify", 1),   # 100 splits: the many-split merge
    (300 * 256, 8, 1, 1, "decode", 1),         # 300 splits
    # other GQA ratios and head counts: G = 3, 2 with 3 KV heads, 16, 7 (35
    # rows: two blocks), and a G = 3 prefill on the wide kernel
    (1000, 12, 4, 3, "verify", 0),
    (1000, 6, 3, 2, "verify", 0),
    (2000, 64, 4, 2, "verify", 0),
    (2000, 28, 4, 5, "verify", 0),
    (1500, 12, 4, 100, "prefill", 0),
]


@pytest.mark.parametrize("N,Hq,Hkv,W,kind,sp", CASES)
def test_parity_sweep(N, Hq, Hkv, W, kind, sp):
    say(f"case sweep N={N} Hq={Hq} Hkv={Hkv} W={W} {kind} split_pages={sp}")
    kvl = layer_kv(N, Hkv, wid=51 + N % 7, pad="garbage")
    q = inputs.draw_queries(W, Hq, 0, 51)
    n = kvl.pages.shape[0]
    table = perm_table(n, N + W)
    h = handle(Hq, Hkv, n + 3, n, max(W, 8), split_pages=sp)
    place(h, 0, kvl, table + 3)
    got = run(h, 0, q, W, kind)
    ref = oracle_out(kvl, q, Hq, Hkv)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL
    h.destroy()


# ------------------------------------------------------------------ placement, bitwise
@pytest.mark.parametrize("W", [4, 10, 20], ids=["one-block", "two-blocks", "wide"])
def test_placement_bitwise_invariance(W):
    # 20, 50 and 100 rows per KV head: the split kernel on one and on two row
    # blocks, and the wide kernel; each plan is fixed by the shapes alone
    N, Hq, Hkv = 3000, 40, 8
    say(f"case placement N={N} Hq={Hq} Hkv={Hkv} W={W}, 6 placements, split_pages=2")
    kvl = layer_kv(N, Hkv, wid=60)
    q = inputs.draw_queries(W, Hq, 0, 60)
    n = kvl.pages.shape[0]
    outs = []
    for seed in range(6):
        rng = np.random.default_rng(seed)
        h = handle(Hq, Hkv, 2 * n, n, max(8, W), n_ring=n + 2, split_pages=2, deterministic=1)
        table = np.empty(n, dtype=np.uint32)
        pool_ids = rng.permutation(2 * n)[:n]
        ring_ids = rng.permutation(n + 2)[:n]
        use_ring = rng.integers(0, 2, n) if seed % 3 else np.zeros(n, int)
        for P in range(n):
            table[P] = (kv.PT_RING_FLAG | int(ring_ids[P])) if use_ring[P] else pool_ids[P]
        place(h, 0, kvl, table)
        outs.append(run(h, 0, q, W, "verify"))
        # the kernels' own resolver reads back every page bit-exactly
        for P in range(n):
            assert np.array_equal(h.debug_read_page(0, P), kvl.pages[P].numpy()), P
        h.destroy()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.max(np.abs(outs[0] - oracle_out(kvl, q, Hq, Hkv))) <= TOL


def test_split_count_sweep():
    N, Hq, Hkv, W = 4000, 40, 8, 3
    say(f"case split sweep N={N} W={W}")
    kvl = layer_kv(N, Hkv, wid=61)
    q = inputs.draw_queries(W, Hq, 0, 61)
    n = kvl.pages.shape[0]
    ref = oracle_out(kvl, q, Hq, Hkv)
    for sp in (1, 2, 5, n):
        h = handle(Hq, Hkv, n, n, 8, split_pages=sp)
        place(h, 0, kvl, np.arange(n, dtype=np.uint32))
        err = np.max(np.abs(run(h, 0, q, W, "verify") - ref))
        say(f"  split_pages={sp}: max-abs err {err:.3e}")
        assert err <= TOL
        h.destroy()


@pytest.mark.parametrize("n_splits", [8, 9, 17, 33, 64, 65, 100])
def test_merge_split_ranges(n_splits):
    # one page per split: the merge instances for up to 8, 16, 32 and 64
    # splits and the many-split merge, each at its boundaries, ragged tail
    N, Hq, Hkv, W = n_splits * 256 - 13, 40, 8, 3
    say(f"case merge splits={n_splits} N={N} W={W}")
    kvl = layer_kv(N, Hkv, wid=62 + n_splits)
    q = inputs.draw_queries(W, Hq, 0, 62 + n_splits)
    n = kvl.pages.shape[0]
    assert n == n_splits
    ref = oracle_out(kvl, q, Hq, Hkv)
    h = handle(Hq, Hkv, n, n, 8, split_pages=1)
    place(h, 0, kvl, perm_table(n, n_splits))
    err = np.max(np.abs(run(h, 0, q, W, "verify") - ref))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


def test_merge_capacity_4096_splits():
    """The largest history a layer may have (4,096 pages, the many-split
    merge's capacity; ragged last page), one page per split: 4,096 partials
    per (row, query head) merged, against the oracle on every output."""
    n_pages = 4096
    N, Hq, Hkv, W = n_pages * 256 - 100, 4, 1, 2
    say(f"case merge capacity splits={n_pages} N={N} Hq={Hq} Hkv={Hkv} W={W}")
    kvl = inputs.draw_layer(N, Hkv, 0, 64, device="cuda")
    q = inputs.draw_queries(W, Hq, 0, 64)
    n = kvl.pages.shape[0]
    assert n == n_pages
    h = handle(Hq, Hkv, n, n, 8, split_pages=1)
    place(h, 0, kvl, perm_table(n, 64))
    got = run(h, 0, q, W, "verify")
    ref, _ = oracle.attend_paged(np.arange(n, dtype=np.uint32), N, 256, Hq, Hkv, q.numpy(), inputs.scale_for(),
                                 pool=kvl.pages.cpu().numpy())
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("W", [1, 6])
def test_chunk_order_modes(W):
    """Deterministic mode repeats its bits exactly; the default (waves claim
    chunks as buffers free) stays within rounding of it and of the oracle."""
    N, Hq, Hkv = 48 * 256 + 77, 40, 8
    say(f"case chunk order N={N} W={W}")
    kvl = layer_kv(N, Hkv, wid=62, pad="garbage")
    q = inputs.draw_queries(W, Hq, 0, 62)
    n = kvl.pages.shape[0]
    ref = oracle_out(kvl, q, Hq, Hkv)
    outs = {}
    for det in (1, 0):
        h = handle(Hq, Hkv, n, n, 8, split_pages=12, deterministic=det)   # 96 chunks per split
        place(h, 0, kvl, perm_table(n, 9))
        outs[det] = [run(h, 0, q, W, "verify" if W > 1 else "decode") for _ in range(3)]
        h.destroy()
    for o in outs[1][1:]:
        assert np.array_equal(o, outs[1][0])
    for o in outs[0]:
        assert np.max(np.abs(o - ref)) <= TOL
        assert np.max(np.abs(o - outs[1][0])) <= 1e-4
    say(f"  deterministic err {np.max(np.abs(outs[1][0] - ref)):.3e}; dynamic vs deterministic "
        f"{max(np.max(np.abs(o - outs[1][0])) for o in outs[0]):.3e}")


# ------------------------------------------------------------------ streaming
@pytest.mark.parametrize("pinned", [True, False], ids=["pinned-history", "pageable-history"])
def test_streamed_matches_resident_bitwise(pinned):
    """Layers whose non-resident pages stream from host memory through a small
    ring (gathered by the ring-copy kernel from pinned memory, or copied run by
    run from pageable memory) give the same bits as all-resident layers at one
    page per split, for every layer of two passes and an out-of-order call."""
    L, N, Hq, Hkv, W = 3, 20 * 256 + 100, 40, 8, 4
    say(f"case streamed L={L} N={N} W={W} ring=5 chunk=2 pinned={pinned}")
    n = -(-N // 256)
    layers = [layer_kv(N, Hkv, wid=70, layer=l) for l in range(L)]
    qs = [inputs.draw_queries(W, Hq, l, 70) for l in range(L)]
    hs = handle(Hq, Hkv, L * n, n, 8, n_ring=5, chunk_slots=2, n_layers=L)
    hr = handle(Hq, Hkv, L * n, n, 8, split_pages=1, n_layers=L, deterministic=1)
    hist = []
    for l in range(L):
        res = inputs.resident_subset(n, int(round(0.4 * n)), l, 70)
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        table[res] = l * n + np.arange(len(res))
        host = layers[l].pages.contiguous()
        host = host.pin_memory() if pinned else host.clone()
        hist.append(host)
        place(hs, l, layers[l], table, history=host)
        place(hr, l, layers[l], l * n + np.arange(n, dtype=np.uint32))
    refs = [oracle_out(layers[l], qs[l], Hq, Hkv) for l in range(L)]
    order = [0, 1, 2, 0, 1, 2, 1, 2, 0]
    for l in order:
        a = run(hs, l, qs[l], W, "verify")
        b = run(hr, l, qs[l], W, "verify")
        err = np.max(np.abs(a - refs[l]))
        say(f"  layer {l}: streamed vs oracle {err:.3e}, bitwise equal to resident: {np.array_equal(a, b)}")
        assert np.array_equal(a, b)
        assert err <= TOL
    # pipelined: all layers enqueued back to back, one sync at the end
    outs = []
    for rep in range(2):
        for l in range(L):
            qd = qs[l].cuda()
            o = torch.empty_like(qd)
            hs.verify(l, qd, W, o)
            outs.append((l, o))
    hs.synchronize()
    for l, o in outs:
        assert np.array_equal(o.cpu().double().numpy(), run(hr, l, qs[l], W, "verify"))
    hs.destroy()
    hr.destroy()


# ------------------------------------------------------------------ full size, sampled
def test_full_size_decode_sampled_layers():
    """The all-resident TG1 decode workload at full size (40,960 tokens, 40/8
    heads) in the launch configuration the benchmark times (automatic split
    plan), two seeded layers checked element by element."""
    w = inputs.WORKLOADS["decode-40k"]
    say(f"case full-size {w.name}: 2 sampled layers")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, 2 * n, n, 8, n_layers=2)
    for l in (0, 1):
        kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 17 + l, w.wid, device="cuda")
        table = l * n + inputs.seeded_permutation(n, 17 + l, w.wid)
        place(h, l, kvl, table)
        q = inputs.draw_queries(1, w.n_q_heads, 17 + l, w.wid, device="cuda")
        got = run(h, l, q, 1, "decode")
        ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads)
        err = np.max(np.abs(got - ref))
        say(f"  layer {17 + l}: max-abs err {err:.3e}")
        assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("W,layer", [(6, 5), (1, 6), (2, 7), (3, 8), (4, 9), (5, 10)])
def test_full_size_verify(W, layer):
    """The all-resident verify workload at full size (163,840 tokens, causal
    tail) with the automatic split plan the benchmark uses (160-chunk splits:
    the claimed chunk order); one seeded layer per width 1-6, every output
    element against the oracle."""
    w = inputs.WORKLOADS["verify-160k"]
    say(f"case full-size {w.name} W={W}: layer {layer}")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, n, n, 8)
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, layer, w.wid, device="cuda")
    place(h, 0, kvl, inputs.seeded_permutation(n, layer, w.wid))
    q = inputs.draw_queries(W, w.n_q_heads, layer, w.wid, device="cuda")
    got = run(h, 0, q, W, "verify")
    ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


def test_wide_verify_w49():
    """A wide speculative verify (49 rows, an n-gram draft width) over 20,000
    tokens: 245 rows per KV head run on the wide kernel; every element
    against the oracle."""
    N, Hq, Hkv, W = 20000, 40, 8, 49
    say(f"case wide verify N={N} W={W}")
    kvl = layer_kv(N, Hkv, wid=80, pad="garbage")
    q = inputs.draw_queries(W, Hq, 0, 80)
    n = kvl.pages.shape[0]
    h = handle(Hq, Hkv, n, n, W)
    place(h, 0, kvl, perm_table(n, 80))
    got = run(h, 0, q, W, "verify")
    ref = oracle_out(kvl, q, Hq, Hkv)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL
    h.destroy()


def test_full_size_prefill_sampled_rows():
    """The 256-row prefill chunk over a 123,136-token history at full size;
    eight seeded rows (first and last included) checked against the oracle,
    and every output finite."""
    w = inputs.WORKLOADS["prefill-120k"]
    R = w.prefill_rows
    say(f"case full-size {w.name} R={R}: 1 layer, 8 sampled rows")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, n, n, R)
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 3, w.wid, device="cuda")
    place(h, 0, kvl, inputs.seeded_permutation(n, 3, w.wid))
    q = inputs.draw_queries(R, w.n_q_heads, 3, w.wid, device="cuda")
    got = run(h, 0, q, R, "prefill")
    assert np.isfinite(got).all()
    rng = np.random.default_rng(11)
    rows = sorted({0, R - 1, *rng.choice(R, 6, replace=False).tolist()})
    ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads, rows=rows)
    err = np.max(np.abs(got[rows] - ref))
    say(f"  rows {rows}: max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("W", [1, 4])
def test_full_size_streamed_layer(W):
    """The streamed workload at full size: 262,144 tokens, 410 resident pages,
    614 streamed from a pinned history through a 64-slot ring (default chunk
    size), two layers.  Both layers are set before the first call, so the
    ring copies of layer 1 start while layer 0 computes (one layer ahead) and
    the ring wraps across the layer boundary; every output element of both
    layers against the oracle reading the same bytes."""
    w = inputs.WORKLOADS["stream-256k"]
    L = 2
    say(f"case full-size {w.name} W={W}: {L} layers, both set before the first call")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, L * w.n_resident, n, 8, n_ring=w.ring_slots, n_layers=L)
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
    outs = []
    for l in range(L):
        o = torch.full_like(qs[l], float("nan"))
        h.verify(l, qs[l], W, o)
        outs.append(o)
    h.synchronize()
    for l in range(L):
        ref, _ = oracle.attend_paged(np.arange(n, dtype=np.uint32), w.n_tokens, 256, w.n_q_heads, w.n_kv_heads,
                                     qs[l].cpu().numpy(), inputs.scale_for(), pool=hosts[l].numpy())
        err = np.max(np.abs(outs[l].cpu().double().numpy() - ref))
        say(f"  layer {l}: max-abs err {err:.3e}")
        assert err <= TOL
    h.destroy()


def test_upload_waits_for_compute():
    """kvattn_upload_pages into ring slots that calls already enqueued on the
    compute stream still read: the copies start only after those calls, so
    every earlier output sees the old pages and the next call the new ones
    (no synchronisation between the calls and the upload)."""
    N, Hq, Hkv, W, calls = 64 * 256, 40, 8, 4, 24
    say(f"case upload ordering N={N} W={W}: {calls} calls, then a re-upload of every slot, then one call")
    a, b = layer_kv(N, Hkv, wid=90), layer_kv(N, Hkv, wid=91)
    n = a.pages.shape[0]
    q = inputs.draw_queries(W, Hq, 0, 90)
    h = handle(Hq, Hkv, 1, n, 8, n_ring=n)
    assert h.copy_stream is not None and h.copy_stream != h.compute_stream
    slots = np.arange(n, dtype=np.uint32)
    ha, hb = a.pages.contiguous().pin_memory(), b.pages.contiguous().pin_memory()
    h.upload_pages(ha, kv.PT_RING_FLAG | slots)
    h.set_layer(0, kv.PT_RING_FLAG | slots, N)
    h.synchronize()
    qd = q.cuda()
    outs = [torch.empty_like(qd) for _ in range(calls + 1)]
    for i in range(calls):
        h.verify(0, qd, W, outs[i])
    h.upload_pages(hb, kv.PT_RING_FLAG | slots)
    h.verify(0, qd, W, outs[calls])
    h.synchronize()
    ref_a, ref_b = oracle_out(a, q, Hq, Hkv), oracle_out(b, q, Hq, Hkv)
    errs = [float(np.max(np.abs(o.cpu().double().numpy() - ref_a))) for o in outs[:calls]]
    err_b = float(np.max(np.abs(outs[calls].cpu().double().numpy() - ref_b)))
    say(f"  before the upload: worst max-abs err {max(errs):.3e}; after: {err_b:.3e}")
    assert max(errs) <= TOL and err_b <= TOL
    h.destroy()
