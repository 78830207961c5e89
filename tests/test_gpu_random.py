"""GPU parity over seeded random configurations.

Forty configurations drawn once from a fixed seed mix what the targeted
tests cover one at a time: page sizes 32 .. 512 tokens, GQA ratios 1 .. 8
with 1 .. 8 KV heads, widths across the one-tile, two-tile, multi-block and
wide plans (verify and prefill), every K/V pair, split_pages forced or
chosen, resident layers with pages in the pool and in caller-placed ring
slots, and layers that stream part of their pages through a small ring.
Every output element is compared with the fp64 oracle reading the same page
bytes.
"""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu

PAIRS = [(inputs.Q8_0, inputs.Q4_0), (inputs.Q8_0, inputs.Q8_0), (inputs.Q4_0, inputs.Q4_0),
         (inputs.F16, inputs.F16)]


def draw_cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.choice([32, 64, 128, 256, 512]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        kind = "prefill" if rng.random() < 0.25 else "verify"
        rows_kv = int(rng.choice([1, 8, 16, 17, 32, 33, 64, 96, 97, 200, 400]))
        W = max(1, rows_kv // G)
        if kind == "prefill":
            W = int(rng.integers(1, 65))
        n_pages = int(rng.integers(1, 40))
        N = max(W, n_pages * T - int(rng.integers(0, T)))
        pair = PAIRS[int(rng.integers(0, 4))]
        mode = str(rng.choice(["pool", "ring", "stream"]))
        sp = int(rng.choice([0, 0, 1, 2, 5]))
        cases.append(dict(i=i, T=T, Hkv=Hkv, G=G, kind=kind, W=W, N=N, pair=pair, mode=mode, sp=sp,
                          seed=int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("c", CASES, ids=[f"r{c['i']}-{c['mode']}-T{c['T']}-G{c['G']}-W{c['W']}" for c in CASES])
def test_random_configuration(c):
    T, Hkv, G, W, N = c["T"], c["Hkv"], c["G"], c["W"], c["N"]
    Hq = Hkv * G
    kt, vt = c["pair"]
    rng = np.random.default_rng(c["seed"])
    say(f"case random {c}")
    kvl = inputs.draw_layer(N, Hkv, 0, 170 + c["i"], page_tokens=T, k_type=kt, v_type=vt, pad="garbage")
    q = inputs.draw_queries(W, Hq, 0, 170 + c["i"])
    n = kvl.pages.shape[0]
    history = None
    if c["mode"] == "pool":
        h = handle(Hq, Hkv, n + 2, n, max(W, 8), split_pages=c["sp"], page_tokens=T, k_type=kt, v_type=vt)
        table = (rng.permutation(n + 2)[:n]).astype(np.uint32)
    elif c["mode"] == "ring":
        h = handle(Hq, Hkv, n, n, max(W, 8), n_ring=n + 1, split_pages=c["sp"], page_tokens=T, k_type=kt,
                   v_type=vt)
        use_ring = rng.integers(0, 2, n).astype(bool)
        pool_ids, ring_ids = rng.permutation(n), rng.permutation(n + 1)
        table = np.array([(kv.PT_RING_FLAG | int(ring_ids[P])) if use_ring[P] else int(pool_ids[P])
                          for P in range(n)], dtype=np.uint32)
    else:
        ring = int(rng.integers(1, 9))
        chunk = int(rng.integers(1, ring + 1))
        n_res = int(rng.integers(0, n))
        h = handle(Hq, Hkv, max(n_res, 1), n, max(W, 8), n_ring=ring, chunk_slots=chunk, page_tokens=T,
                   k_type=kt, v_type=vt)
        table = np.full(n, kv.PT_HOST, dtype=np.uint32)
        res = np.sort(rng.choice(n, n_res, replace=False)) if n_res else np.zeros(0, dtype=np.int64)
        table[res] = np.arange(n_res)
        history = kvl.pages.contiguous().pin_memory()
    place(h, 0, kvl, table, history=history, page_tokens=T)
    qd = q.cuda().contiguous()
    out = torch.full_like(qd, float("nan"))
    if c["kind"] == "prefill":
        h.prefill_chunk(0, qd, W, out)
    else:
        h.verify(0, qd, W, out)
    h.synchronize()
    got = out.cpu().double().numpy()
    ref = oracle_out(kvl, q, Hq, Hkv, page_tokens=T)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max-abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL
    h.destroy()
