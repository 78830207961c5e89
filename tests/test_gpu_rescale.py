"""GPU parity on inputs that drive the online-softmax re-reference path.

The kernels keep a lazy per-row softmax reference and rescale the running
accumulators when a score exceeds it by more than 8 (log2 units).  With the
workloads' N(0,1) queries later scores stay within that margin of a wave's
first chunk, so these tests build inputs whose scores climb far above it:

  scaled     queries alpha * N(0,1) (alpha = 8: scores spread over tens of
             log2 units);
  page-id    logical page P has score 8.25 * P (log2 units) for every key,
             so every new page a wave reaches moves its reference, and value
             (P + 1) / 128 (an fp64 closed form exists; the oracle's pins check
             it on the CPU);
  dominant   each (row, head) query points at one late key, which outweighs
             the rest by about 25 nats.

Rounding-exact construction, so the 2e-3 bar keeps its meaning at large
score magnitudes: queries lie on the f16 grid the kernels round them to
(q = h / qscale with h a binary16 value, qscale = softmax_scale * log2(e) in
binary32), and key scales are powers of two, so the f16 key view of the
wide kernel (c * d) is exact as well.  What remains is binary16 rounding on
the value side (P * d_V or V' and P), relative 2^-12 of |V|, and fp32
accumulation.

Each case runs twice: through the kernels' counting instantiation, whose
re-reference counter (a test aid of the C ABI) must show the branch ran, and
through the production instantiation (the same arithmetic without the
counter).  Every output element of both is compared with the fp64 oracle
reading the same page bytes.
"""
import math

import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu

Q8, Q4, F16 = inputs.Q8_0, inputs.Q4_0, inputs.F16
PAIRS = [(Q8, Q4), (Q8, Q8), (Q4, Q4), (F16, F16)]
PAIR_IDS = ["q8_0-q4_0", "q8_0-q8_0", "q4_0-q4_0", "f16-f16"]


def kernel_qscale():
    """softmax_scale * log2(e) as the library forms it: binary32 arithmetic on
    1/sqrt(128) and log2(e)."""
    s = np.float32(1.0) / np.sqrt(np.float32(128.0))
    return np.float32(s * np.float32(1.4426950408889634))


def on_f16_grid(h):
    """Queries q = h / qscale (binary32) whose kernel-side product q * qscale
    rounds back to the binary16 values h exactly."""
    qs = float(kernel_qscale())
    return torch.from_numpy((h.astype(np.float64) / qs).astype(np.float32))


def quant_k_pow2(x, k_type):
    """Keys with power-of-two block scales: Q8_0 d = 2^ceil(log2(amax / 127)),
    codes round(x / d) in [-127, 127]; Q4_0 d = 2^ceil(log2(amax / 8)), codes
    round(x / d) + 8 in [0, 15]; F16 the binary16 values."""
    if k_type == F16:
        return x.to(torch.float16), None
    xb = x.float().reshape(*x.shape[:-1], 4, 32)
    amax = xb.abs().amax(-1)
    top = 127.0 if k_type == Q8 else 8.0
    e = torch.ceil(torch.log2(torch.clamp(amax, min=1e-30) / top))
    d = torch.where(amax > 0, torch.exp2(e), torch.zeros_like(amax))
    safe = torch.where(d > 0, d, torch.ones_like(d)).unsqueeze(-1)
    c = torch.round(xb / safe)
    if k_type == Q8:
        c = c.clamp(-127, 127).to(torch.int8)
    else:
        c = (c + 8).clamp(0, 15).to(torch.uint8)
    return c.reshape(x.shape), d.to(torch.float16)


def build_layer(kc, kd, vc, vd, k_type, v_type, seed, page_tokens=256):
    pages = inputs.pack_pages(kc, kd, vc, vd, page_tokens, pad="garbage", pad_seed=seed, k_type=k_type,
                              v_type=v_type)
    return inputs.LayerKV(kc, kd, vc, vd, pages=pages, k_type=k_type, v_type=v_type)


def scaled_case(N, Hq, Hkv, W, k_type, v_type, alpha, seed, page_tokens=256):
    g = torch.Generator().manual_seed(seed)
    K = torch.randn((N, Hkv, 128), generator=g)
    V = torch.randn((N, Hkv, 128), generator=g)
    kc, kd = quant_k_pow2(K, k_type)
    vc, vd = inputs.quantize(V, v_type)
    q = alpha * torch.randn((W, Hq, 128), generator=g)
    h = (q.double() * float(kernel_qscale())).numpy().astype(np.float16)
    return build_layer(kc, kd, vc, vd, k_type, v_type, seed, page_tokens), on_f16_grid(h)


def page_id_case(N, Hq, Hkv, W, k_type, v_type, seed):
    """Page P: K dim 0 = P (block-0 scale P, code 1; other dims 0), V = (P +
    1) / 128 in every dim; queries h = 8.25 in dim 0 only, so a key of page P
    scores 8.25 * P (log2 units)."""
    P = torch.arange(N) // 256
    kc = torch.zeros((N, Hkv, 128), dtype=torch.int8)
    if k_type == F16:
        kc = torch.zeros((N, Hkv, 128), dtype=torch.float16)
        kc[:, :, 0] = P.to(torch.float16).unsqueeze(1)
        kd = None
    else:
        if k_type == Q4:
            kc = torch.full((N, Hkv, 128), 8, dtype=torch.uint8)
            kc[:, :, 0] = 9
        else:
            kc[:, :, 0] = 1
        kd = torch.zeros((N, Hkv, 4), dtype=torch.float16)
        kd[:, :, 0] = P.to(torch.float16).unsqueeze(1)
    val = ((P + 1).double() / 128.0).to(torch.float16)
    if v_type == F16:
        vc = val.view(N, 1, 1).expand(N, Hkv, 128).contiguous()
        vd = None
    else:
        vc = torch.full((N, Hkv, 128), 9 if v_type == Q4 else 1, dtype=torch.uint8 if v_type == Q4 else torch.int8)
        vd = val.view(N, 1, 1).expand(N, Hkv, 4).contiguous()
    h = np.zeros((W, Hq, 128), dtype=np.float16)
    h[:, :, 0] = 8.25
    return build_layer(kc, kd, vc, vd, k_type, v_type, seed), on_f16_grid(h)


def dominant_case(N, Hq, Hkv, W, k_type, v_type, seed):
    """Each (row, head) query is 40 nats along the dequantised key of one seeded
    key in the last quarter of the row's visible history."""
    g = torch.Generator().manual_seed(seed)
    K = torch.randn((N, Hkv, 128), generator=g)
    V = torch.randn((N, Hkv, 128), generator=g)
    kc, kd = quant_k_pow2(K, k_type)
    vc, vd = inputs.quantize(V, v_type)
    layer = build_layer(kc, kd, vc, vd, k_type, v_type, seed)
    Kd = kc.double() if k_type == F16 else None
    if k_type != F16:
        codes = kc.double() - (8.0 if k_type == Q4 else 0.0)
        Kd = (codes.reshape(N, Hkv, 4, 32) * kd.double().unsqueeze(-1)).reshape(N, Hkv, 128)
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    qs = float(kernel_qscale())
    h = np.zeros((W, Hq, 128), dtype=np.float16)
    scale = 1.0 / math.sqrt(128.0)
    for r in range(W):
        pos = N - W + r
        for hh in range(Hq):
            j = int(rng.integers(3 * (pos + 1) // 4, pos + 1))
            k = Kd[j, hh // G]
            q = 40.0 * k / (k.norm() ** 2 * scale)  # score of key j: 40 nats
            h[r, hh] = (q * qs).numpy().astype(np.float16)
    return layer, on_f16_grid(h)


def run_call(h, q, W, kind, counted, layer=0):
    """One call; counted: through the kernels' counting instantiation (the
    counter is read back), else the production one."""
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    if counted:
        h.count_rescales(counter)
    qd = q.to("cuda").contiguous()
    out = torch.full_like(qd, float("nan"))
    if kind == "prefill":
        h.prefill_chunk(layer, qd, W, out)
    else:
        h.verify(layer, qd, W, out)
    h.synchronize()
    h.count_rescales(None)
    return out.cpu().double().numpy(), int(counter.item())


def check(h, layer, q, W, kind, Hq, Hkv, what, page_tokens=256):
    """The counting instantiation shows the branch ran; both it and the
    production instantiation (same arithmetic) must match the oracle."""
    got, events = run_call(h, q, W, kind, True)
    plain, none = run_call(h, q, W, kind, False)
    ref = oracle_out(layer, q, Hq, Hkv, page_tokens=page_tokens)
    err = float(np.max(np.abs(got - ref)))
    err_plain = float(np.max(np.abs(plain - ref)))
    say(f"  {what}: max-abs err {err:.3e} (production kernels {err_plain:.3e}, bitwise equal "
        f"{np.array_equal(got, plain)}), re-reference events {events}")
    assert np.isfinite(got).all() and np.isfinite(plain).all()
    assert events > 0, "the inputs did not reach the re-reference branch"
    assert none == 0
    assert err <= TOL and err_plain <= TOL
    return events


# Plans (Hq 40 / Hkv 8, G = 5): W = 1 one 16-row tile, W = 5 two tiles,
# W = 10 two 32-row blocks, W = 17 three blocks, W = 25 and 49 the wide
# kernel, prefill R = 64 (320 rows per KV head: 12-wave wide blocks).  Long
# splits (split_pages, or long histories for the multi-block plans) give each
# wave several chunks.
PLANS = [
    # W, kind, N, split_pages
    (1, "verify", 6000, 8),
    (5, "verify", 6000, 8),
    (10, "verify", 20000, 0),
    (17, "verify", 20000, 0),
    (25, "verify", 6000, 0),
    (49, "verify", 6000, 0),
    (64, "prefill", 5000, 0),
]
PLAN_IDS = ["one-tile", "two-tile", "two-block", "three-block", "wide-8w", "wide-w49", "prefill-12w"]


@pytest.mark.parametrize("kt,vt", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("W,kind,N,sp", PLANS, ids=PLAN_IDS)
def test_scaled_queries(W, kind, N, sp, kt, vt):
    Hq, Hkv = 40, 8
    say(f"case rescale scaled alpha=8 N={N} W={W} {kind} split_pages={sp} pair={kt}/{vt}")
    layer, q = scaled_case(N, Hq, Hkv, W, kt, vt, 8.0, 900 + W)
    n = layer.pages.shape[0]
    h = handle(Hq, Hkv, n, n, max(W, 8), split_pages=sp, k_type=kt, v_type=vt)
    place(h, 0, layer, np.random.default_rng(W).permutation(n).astype(np.uint32))
    check(h, layer, q, W, kind, Hq, Hkv, "scaled")
    h.destroy()


@pytest.mark.parametrize("kt,vt", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("W,kind,N,sp", PLANS, ids=PLAN_IDS)
def test_page_id_staircase(W, kind, N, sp, kt, vt):
    Hq, Hkv = 40, 8
    # splits must cross pages for a wave to meet a higher page: long histories
    # (79 pages; at most 127, the largest page index a Q4_0 or Q8_0 scale of
    # this construction keeps exact is far larger)
    N = 20000 - 11
    say(f"case rescale page-id N={N} W={W} {kind} split_pages={sp} pair={kt}/{vt}")
    layer, q = page_id_case(N, Hq, Hkv, W, kt, vt, 910 + W)
    n = layer.pages.shape[0]
    h = handle(Hq, Hkv, n, n, max(W, 8), split_pages=sp, k_type=kt, v_type=vt)
    place(h, 0, layer, np.random.default_rng(W + 1).permutation(n).astype(np.uint32))
    check(h, layer, q, W, kind, Hq, Hkv, "page-id")
    h.destroy()


@pytest.mark.parametrize("W,kind,N,sp", PLANS[:5], ids=PLAN_IDS[:5])
def test_dominant_late_key(W, kind, N, sp):
    Hq, Hkv = 40, 8
    say(f"case rescale dominant N={N} W={W} {kind} split_pages={sp}")
    layer, q = dominant_case(N, Hq, Hkv, W, Q8, Q4, 920 + W)
    n = layer.pages.shape[0]
    h = handle(Hq, Hkv, n, n, max(W, 8), split_pages=sp)
    place(h, 0, layer, np.random.default_rng(W + 2).permutation(n).astype(np.uint32))
    check(h, layer, q, W, kind, Hq, Hkv, "dominant")
    h.destroy()


@pytest.mark.parametrize("kt,vt", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("W", [1, 4])
def test_streamed_scaled(W, kt, vt):
    """Streamed layers (pages through a 6-slot ring, one page per split):
    1024-token pages give every wave of a split several chunks, so the
    re-reference path runs inside a page; both split-kernel shapes."""
    Hq, Hkv, T = 40, 8, 1024
    N = 24 * T - 50
    say(f"case rescale streamed N={N} T={T} W={W} pair={kt}/{vt}")
    layer, q = scaled_case(N, Hq, Hkv, W, kt, vt, 8.0, 930 + W, page_tokens=T)
    n = layer.pages.shape[0]
    h = handle(Hq, Hkv, n, n, 8, n_ring=6, chunk_slots=3, k_type=kt, v_type=vt, page_tokens=T)
    res = np.sort(np.random.default_rng(W).choice(n, n // 3, replace=False))
    table = np.full(n, kv.PT_HOST, dtype=np.uint32)
    table[res] = np.arange(len(res))
    place(h, 0, layer, table, history=layer.pages.contiguous().pin_memory(), page_tokens=T)
    check(h, layer, q, W, "verify", Hq, Hkv, "streamed scaled", page_tokens=T)
    h.destroy()
