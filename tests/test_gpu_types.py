"""GPU parity for the K/V element-type pairs beside Q8_0 K / Q4_0 V: Q8_0 /
Q8_0, Q4_0 / Q4_0 and F16 / F16 ("Required FlashAttention kernels": a
same-type kernel for each side of the mixed pair, and an f16 pair).

Every case runs through the C-ABI against the fp64 oracle reading the same
pages (max-abs 2e-3); the writer's codes and scales are compared bit-exactly
with the oracle's quantisers.
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
import oracle
from gpu_util import TOL, handle, oracle_out, place, run, say

pytestmark = pytest.mark.gpu

PAIRS = [(kv.TYPE_Q8_0, kv.TYPE_Q8_0), (kv.TYPE_Q4_0, kv.TYPE_Q4_0), (kv.TYPE_F16, kv.TYPE_F16)]
IDS = ["q8k-q8v", "q4k-q4v", "f16k-f16v"]

CASES = [
    # N, Hq, Hkv, W, kind, split_pages
    (2048 - 37, 4, 1, 1, "decode", 0),
    (31, 8, 2, 1, "decode", 0),
    (300, 40, 8, 1, "decode", 0),
    (5000, 40, 8, 1, "decode", 7),
    (300, 40, 8, 3, "verify", 1),     # 15 rows per KV head: one row tile
    (5000, 40, 8, 6, "verify", 3),    # 30 rows: two row tiles
    (6, 8, 1, 6, "verify", 0),        # every key a verify row
    (256 + 700, 40, 8, 256, "prefill", 0),
    (3000, 40, 8, 37, "prefill", 0),
]


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("N,Hq,Hkv,W,kind,sp", CASES)
def test_pair_parity(pair, N, Hq, Hkv, W, kind, sp):
    say(f"case types k={pair[0]} v={pair[1]} N={N} Hq={Hq} Hkv={Hkv} W={W} {kind} split_pages={sp}")
    kvl = inputs.draw_layer(N, Hkv, 0, 70 + N % 5, pad="garbage", k_type=pair[0], v_type=pair[1])
    q = inputs.draw_queries(W, Hq, 0, 70)
    n = kvl.pages.shape[0]
    table = np.random.default_rng(N + W).permutation(n).astype(np.uint32)
    h = handle(Hq, Hkv, n + 3, n, max(W, 8), split_pages=sp, k_type=pair[0], v_type=pair[1])
    assert kv.page_bytes(h.params) == oracle.page_bytes(Hkv, 256, *pair)
    place(h, 0, kvl, table + 3)
    got = run(h, 0, q, W, kind)
    ref = oracle_out(kvl, q, Hq, Hkv)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL
    for P in range(n):   # the kernels' resolver reads every page back bit-exactly
        assert np.array_equal(h.debug_read_page(0, P), kvl.pages[P].numpy()), P
    h.destroy()


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
def test_pair_streamed(pair):
    """Pages split over pool pages and the pinned host history (streamed
    through the ring)."""
    N, Hq, Hkv, W = 4000, 40, 8, 4
    say(f"case types streamed k={pair[0]} v={pair[1]} N={N} W={W}")
    kvl = inputs.draw_layer(N, Hkv, 0, 77, k_type=pair[0], v_type=pair[1])
    q = inputs.draw_queries(W, Hq, 0, 77)
    n = kvl.pages.shape[0]
    rng = np.random.default_rng(3)
    table = np.where(rng.integers(0, 2, n) == 0, np.arange(n), kv.PT_HOST).astype(np.uint32)
    host = kvl.pages.contiguous().pin_memory()
    h = handle(Hq, Hkv, n, n, 8, n_ring=6, chunk_slots=2, k_type=pair[0], v_type=pair[1])
    place(h, 0, kvl, table, history=host)
    got = run(h, 0, q, W, "verify")
    err = np.max(np.abs(got - oracle_out(kvl, q, Hq, Hkv)))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


def expected_codes(x, t):
    """Oracle encoding of fp32 rows [R][H][128] for element type t, in the
    unpack_page convention (F16: binary16 bits)."""
    if t == kv.TYPE_Q8_0:
        c, d = oracle.quantize_q8_0(x)
        return c.astype(np.int32), d
    if t == kv.TYPE_Q4_0:
        c, d = oracle.quantize_q4_0(x)
        return c.astype(np.int32), d
    bits = np.array([oracle.f32_to_f16(float(v)) for v in x.reshape(-1)], dtype=np.int32).reshape(x.shape)
    return bits, None


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("N0,R,Hkv", [(300, 1, 8), (31, 2, 2), (250, 37, 4), (1000, 600, 2)])
def test_pair_append_bitexact(pair, N0, R, Hkv):
    say(f"case types append k={pair[0]} v={pair[1]} N0={N0} R={R} Hkv={Hkv}")
    kvl = inputs.draw_layer(N0, Hkv, 0, 80 + R % 7, pad="garbage", k_type=pair[0], v_type=pair[1])
    n0 = kvl.pages.shape[0]
    n1 = -(-(N0 + R) // 256)
    n_pool = n1 + 4
    h = handle(Hkv * 5, Hkv, n_pool, n1 + 1, 8, k_type=pair[0], v_type=pair[1])
    ids = np.random.default_rng(N0 + R).permutation(n_pool)[:n1].astype(np.uint32)
    place(h, 0, kvl, ids[:n0])
    pb = kv.page_bytes(h.params)
    for i in ids[n0:]:
        h.pool[int(i) * pb:(int(i) + 1) * pb].copy_(torch.randint(0, 256, (pb,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    before = [oracle.unpack_page(h.debug_read_page(0, P), Hkv, 256, *pair) for P in range(n0)]
    g = torch.Generator().manual_seed(N0 * 7 + R)
    k = torch.randn(R, Hkv, 128, generator=g)
    v = torch.randn(R, Hkv, 128, generator=g)
    h.append(0, k.cuda(), v.cuda(), R, ids[n0:])
    h.synchronize()
    after = [oracle.unpack_page(h.debug_read_page(0, P), Hkv, 256, *pair) for P in range(n1)]
    ekc, ekd = expected_codes(k.numpy(), pair[0])
    evc, evd = expected_codes(v.numpy(), pair[1])
    for P in range(n1):
        kc, kd, vc, vd = after[P]
        for j in range(256):
            pos = P * 256 + j
            if N0 <= pos < N0 + R:
                r = pos - N0
                assert np.array_equal(kc[j], ekc[r]), (P, j)
                assert np.array_equal(vc[j], evc[r]), (P, j)
                if ekd is not None:
                    assert np.array_equal(kd[j], ekd[r]), (P, j)
                if evd is not None:
                    assert np.array_equal(vd[j], evd[r]), (P, j)
            elif P < n0:
                for a, b in zip(after[P], before[P]):
                    assert np.array_equal(a[j], b[j]), ("changed", P, j)
    # attention over the grown history (decode of the last row)
    q = inputs.draw_queries(1, Hkv * 5, 0, 81)
    got = run(h, 0, q, 1, "decode")
    pages = np.stack([h.debug_read_page(0, P) for P in range(n1)])
    ref, _ = oracle.attend_paged(np.arange(n1, dtype=np.uint32), N0 + R, 256, Hkv * 5, Hkv, q.numpy(),
                                 inputs.scale_for(), pool=pages, k_type=pair[0], v_type=pair[1])
    err = np.max(np.abs(got - ref))
    say(f"  decode after append: max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


# ------------------------------------------------------------------ full size, the benchmark's launch configuration
@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("wname,W", [("decode-40k", 1), ("verify-160k", 6)])
def test_pair_full_size(pair, wname, W):
    """`bench.py --kv-types` workloads at full size with the automatic split
    plan: one seeded layer, every output element against the oracle."""
    w = inputs.WORKLOADS[wname]
    say(f"case full-size types k={pair[0]} v={pair[1]} {wname} W={W}")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, n, n, 8, k_type=pair[0], v_type=pair[1])
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 23, w.wid, device="cuda", k_type=pair[0], v_type=pair[1])
    place(h, 0, kvl, inputs.seeded_permutation(n, 23, w.wid))
    q = inputs.draw_queries(W, w.n_q_heads, 23, w.wid, device="cuda")
    got = run(h, 0, q, W, "decode" if W == 1 else "verify")
    ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads)
    err = np.max(np.abs(got - ref))
    say(f"  max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
def test_pair_full_size_prefill_rows(pair):
    """The 256-row prefill chunk over 123,136 keys per pair: four seeded rows
    (first and last included) against the oracle, every output finite."""
    w = inputs.WORKLOADS["prefill-120k"]
    R = w.prefill_rows
    say(f"case full-size types k={pair[0]} v={pair[1]} prefill R={R}")
    n = w.n_pages
    h = handle(w.n_q_heads, w.n_kv_heads, n, n, R, k_type=pair[0], v_type=pair[1])
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 4, w.wid, device="cuda", k_type=pair[0], v_type=pair[1])
    place(h, 0, kvl, inputs.seeded_permutation(n, 4, w.wid))
    q = inputs.draw_queries(R, w.n_q_heads, 4, w.wid, device="cuda")
    got = run(h, 0, q, R, "prefill")
    assert np.isfinite(got).all()
    rows = sorted({0, R - 1, *np.random.default_rng(12).choice(R, 2, replace=False).tolist()})
    ref = oracle_out(kvl, q, w.n_q_heads, w.n_kv_heads, rows=rows)
    err = np.max(np.abs(got[rows] - ref))
    say(f"  rows {rows}: max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()


@pytest.mark.parametrize("pair", PAIRS, ids=IDS)
@pytest.mark.parametrize("T", [32, 64])
def test_pair_small_pages(pair, T):
    """Pages of 32 and 64 tokens per pair: decode, 6-row verify, a 70-row
    prefill chunk and an append across page boundaries, all against the
    oracle reading the same pages."""
    N, Hq, Hkv = 1000, 16, 2
    say(f"case types k={pair[0]} v={pair[1]} page_tokens={T}")
    kvl = inputs.draw_layer(N, Hkv, 0, 71, pad="garbage", page_tokens=T, k_type=pair[0], v_type=pair[1])
    n = kvl.pages.shape[0]
    extra = 3
    h = handle(Hq, Hkv, n + extra + 2, n + extra, 80, page_tokens=T, k_type=pair[0], v_type=pair[1])
    table = np.random.default_rng(T).permutation(n + 2)[:n].astype(np.uint32)
    place(h, 0, kvl, table, page_tokens=T)
    for W, kind in [(1, "decode"), (6, "verify"), (70, "prefill")]:
        q = inputs.draw_queries(W, Hq, W, 71)
        got = run(h, 0, q, W, kind)
        err = np.max(np.abs(got - oracle_out(kvl, q, Hq, Hkv, page_tokens=T)))
        say(f"  {kind} W={W}: max-abs err {err:.3e}")
        assert err <= TOL
    # grow by 2 pages' worth of rows into fresh pool pages, then decode
    R = 2 * T - 7
    free = np.setdiff1d(np.arange(n + extra + 2), table)[: -(-(N + R) // T) - n].astype(np.uint32)
    g = torch.Generator().manual_seed(T)
    k = torch.randn(R, Hkv, 128, generator=g)
    v = torch.randn(R, Hkv, 128, generator=g)
    h.append(0, k.cuda(), v.cuda(), R, free)
    n1 = -(-(N + R) // T)
    pages = np.stack([h.debug_read_page(0, P) for P in range(n1)])
    q = inputs.draw_queries(1, Hq, 9, 71)
    got = run(h, 0, q, 1, "decode")
    ref, _ = oracle.attend_paged(np.arange(n1, dtype=np.uint32), N + R, T, Hq, Hkv, q.numpy(), inputs.scale_for(),
                                 pool=pages, k_type=pair[0], v_type=pair[1])
    err = np.max(np.abs(got - ref))
    say(f"  decode after append of {R} rows: max-abs err {err:.3e}")
    assert err <= TOL
    h.destroy()
