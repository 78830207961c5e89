"""Pins for the oracle: checks against things other than the oracle itself.

Each test names what it pins the oracle to: the binary16 definition (via
numpy's own conversion), exact rational arithmetic, a library attention
routine (torch's fp64 scaled_dot_product_attention on the quantiser's
unpaged arrays), closed forms, brute-force invariants, and byte counts the
pages print.  All CPU; no GPU and no HIP library involved.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128


# ---------------------------------------------------------------- helpers
Q8_0, Q4_0, F16 = inputs.Q8_0, inputs.Q4_0, inputs.F16
PAIRS = [(Q8_0, Q4_0), (Q8_0, Q8_0), (Q4_0, Q4_0), (F16, F16)]
PAIR_IDS = ["q8k-q4v", "q8k-q8v", "q4k-q4v", "f16k-f16v"]


def cache(n_tokens, n_kv_heads, layer=0, wid=90, page_tokens=256, pad="zero", k_type=Q8_0, v_type=Q4_0):
    return inputs.draw_layer(n_tokens, n_kv_heads, layer, wid, page_tokens=page_tokens, pad=pad, k_type=k_type,
                             v_type=v_type)


def dequant(codes, scales, t_):
    """Element values from the quantiser's unpaged arrays, by the block-format
    definitions: Q8_0 d * c, Q4_0 d * (n - 8), F16 the value itself."""
    if t_ == F16:
        return codes.double()
    d = scales.double().repeat_interleave(32, dim=-1)
    return d * (codes.double() - (8.0 if t_ == Q4_0 else 0.0))


def np_arrays(kv):
    return (kv.kc.numpy(), kv.kd.numpy().view(np.uint16), kv.vc.numpy(), kv.vd.numpy().view(np.uint16))


def sdpa_reference(kv, q, scale):
    """torch fp64 scaled_dot_product_attention on the unpaged dequantised
    arrays (library routine), causal among the W query rows at the tail."""
    N, H, _ = kv.kc.shape
    W, Hq, _ = q.shape
    G = Hq // H
    K = dequant(kv.kc, kv.kd, kv.k_type)                                         # [N][H][D]
    V = dequant(kv.vc, kv.vd, kv.v_type)
    Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0)                          # [Hq][N][D]
    Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
    Qh = q.double().permute(1, 0, 2)                                             # [Hq][W][D]
    pos = torch.arange(N - W, N).unsqueeze(1)
    mask = torch.arange(N).unsqueeze(0) <= pos                                  # [W][N]
    out = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh, attn_mask=mask, scale=scale)
    scores = (Qh @ Kh.transpose(1, 2)) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)                                        # [Hq][W]
    return out.permute(1, 0, 2).numpy(), lse.T.numpy()


def identity_paged(oracle, kv, q, scale, page_tokens=256):
    n_pages = kv.pages.shape[0]
    pt = np.arange(n_pages, dtype=np.uint32)
    N, H = kv.kc.shape[:2]
    return oracle.attend_paged(pt, N, page_tokens, q.shape[1], H, q.numpy(), scale, pool=kv.pages.numpy(),
                               k_type=kv.k_type, v_type=kv.v_type)


def scattered_paged(oracle, kv, q, scale, seed, page_tokens=256):
    """Same cache spread over pool pages, ring slots and the host history,
    in a seeded random physical order."""
    pages = kv.pages.numpy()
    n_pages, pb = pages.shape
    rng = np.random.default_rng(seed)
    where = rng.integers(0, 3, n_pages)             # 0 pool, 1 ring, 2 host
    pool = rng.integers(0, 256, (n_pages + 3, pb), dtype=np.uint8)   # unused pages hold noise
    ring = rng.integers(0, 256, (n_pages + 2, pb), dtype=np.uint8)
    pool_ids = rng.permutation(n_pages + 3)[:n_pages]
    ring_ids = rng.permutation(n_pages + 2)[:n_pages]
    history = rng.integers(0, 256, (n_pages, pb), dtype=np.uint8)
    pt = np.empty(n_pages, dtype=np.uint32)
    for p in range(n_pages):
        if where[p] == 0:
            pool[pool_ids[p]] = pages[p]
            pt[p] = pool_ids[p]
        elif where[p] == 1:
            ring[ring_ids[p]] = pages[p]
            pt[p] = inputs.RING_FLAG | int(ring_ids[p])
        else:
            history[p] = pages[p]
            pt[p] = inputs.HOST_ENTRY
    N, H = kv.kc.shape[:2]
    return oracle.attend_paged(pt, N, page_tokens, q.shape[1], H, q.numpy(), scale, pool=pool, ring=ring,
                               history=history, k_type=kv.k_type, v_type=kv.v_type)


def const_cache(n_tokens, n_kv_heads, kc, kd, vc, vd, page_tokens=256):
    """Logical arrays given as callables of (j, h, t) / (j, h, b) -> LayerKV."""
    j = torch.arange(n_tokens).view(-1, 1, 1)
    h = torch.arange(n_kv_heads).view(1, -1, 1)
    t = torch.arange(D).view(1, 1, -1)
    b = torch.arange(4).view(1, 1, -1)
    KC = kc(j, h, t).expand(n_tokens, n_kv_heads, D).to(torch.int8).contiguous()
    KD = kd(j, h, b).expand(n_tokens, n_kv_heads, 4).to(torch.float16).contiguous()
    VC = vc(j, h, t).expand(n_tokens, n_kv_heads, D).to(torch.uint8).contiguous()
    VD = vd(j, h, b).expand(n_tokens, n_kv_heads, 4).to(torch.float16).contiguous()
    kv = inputs.LayerKV(KC, KD, VC, VD)
    kv.pages = inputs.pack_pages(KC, KD, VC, VD, page_tokens)
    return kv


# ---------------------------------------------------------------- format pins
def test_f16_decode_exhaustive(oracle_mod):
    """All 65,536 binary16 patterns against numpy's float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


SCALES = [0.0, -0.0, 1.0, -1.0, 0.0234375, -0.3125, 6.1035156e-05, 5.9604645e-08, 65504.0, -2.0 ** -20, 0.1, 3.14]


def test_dequant_exhaustive_exact(oracle_mod):
    """Every int8 K code and every 4-bit V code, under a set of binary16 scales
    (normal, subnormal, signed zero, max), decoded from packed page bytes,
    equals Fraction(scale) * code exactly."""
    T, H = 256, 2
    kv = const_cache(
        T, H,
        kc=lambda j, h, t: ((j * 128 + t + 97 * h) % 256) - 128,
        kd=lambda j, h, b: torch.tensor(SCALES, dtype=torch.float64)[(j * 4 + b + 5 * h) % len(SCALES)],
        vc=lambda j, h, t: (j * 7 + t * 3 + h) % 16,
        vd=lambda j, h, b: torch.tensor(SCALES, dtype=torch.float64)[(j * 4 + b + 3 + h) % len(SCALES)])
    page = kv.pages[0].numpy()
    seen_k, seen_v = set(), set()
    for h in range(H):
        for j in range(T):
            for b in range(4):
                ks = oracle_mod.k_scale(page, H, T, h, j, b)
                vs = oracle_mod.v_scale(page, H, T, h, j, b)
                assert Fraction(ks) == Fraction(float(kv.kd[j, h, b]))
                assert Fraction(vs) == Fraction(float(kv.vd[j, h, b]))
            for t in range(D):
                kc = oracle_mod.k_code(page, H, T, h, j, t)
                vc = oracle_mod.v_code(page, H, T, h, j, t)
                assert kc == int(kv.kc[j, h, t]) and vc == int(kv.vc[j, h, t])
                seen_k.add(kc)
                seen_v.add(vc)
    assert seen_k == set(range(-128, 128)) and seen_v == set(range(16))
    # dequantised values, exact rationals
    K, V = oracle_mod.decode_page(page, H, T)
    for (j, h, t) in [(0, 0, 0), (5, 1, 77), (255, 1, 127), (128, 0, 64), (31, 0, 31), (32, 1, 32)]:
        b = t // 32
        assert Fraction(K[j, h, t]) == Fraction(float(kv.kd[j, h, b])) * int(kv.kc[j, h, t])
        assert Fraction(V[j, h, t]) == Fraction(float(kv.vd[j, h, b])) * (int(kv.vc[j, h, t]) - 8)
    kd = np.repeat(kv.kd.double().numpy(), 32, axis=-1)
    vd = np.repeat(kv.vd.double().numpy(), 32, axis=-1)
    assert np.array_equal(K, kd * kv.kc.double().numpy())
    assert np.array_equal(V, vd * (kv.vc.double().numpy() - 8))


def test_page_bytes_and_golden_geometry(oracle_mod):
    assert oracle_mod.page_bytes(8, 256) == 425984 == inputs.page_bytes(8, 256)
    with open(os.path.join(HERE, "golden", "geometry.json")) as f:
        fx = json.load(f)["fixtures"]
    per_token = oracle_mod.page_bytes(8, 256) / 256
    for case in fx:
        mib = case["tokens"] * case["layers"] * per_token / 2 ** 20
        assert abs(mib - case["mib"]) <= case["tolerance_mib"], case["cite"]


def test_quantiser_round_trip():
    """Input-encoding sanity: |x - x_hat| <= |d|/2 (Q8_0, with a hair for the
    binary16 rounding of d) and <= |d| (Q4_0, clamped at +7)."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4096, 128, generator=g) * 3
    c, d = quantize = inputs.quantize_q8_0(x)
    dd = d.float().repeat_interleave(32, -1)
    err = (x - dd * c.float()).abs()
    assert bool((err <= dd.abs() * (0.5 + 127 * 2.0 ** -11) + 1e-7).all())
    c, d = inputs.quantize_q4_0(x)
    dd = d.float().repeat_interleave(32, -1)
    err = (x - dd * (c.float() - 8)).abs()
    assert bool((err <= dd.abs() * (1 + 2.0 ** -9) + 1e-7).all())
    assert int(c.min()) >= 0 and int(c.max()) <= 15


# ---------------------------------------------------------------- attention pins
CORE_CASES = [
    # (N, Hq, Hkv, W, page_tokens)
    (2048, 4, 1, 1, 256),     # the tiny workload's shape
    (300, 6, 2, 3, 256),      # ragged last page, GQA 3:1
    (200, 8, 2, 6, 64),       # small pages, 6 verify rows
    (37, 5, 1, 5, 32),        # fewer keys than one page
]


@pytest.mark.parametrize("N,Hq,Hkv,W,T", CORE_CASES)
def test_attention_matches_library_sdpa(oracle_mod, N, Hq, Hkv, W, T):
    kv = cache(N, Hkv, page_tokens=T)
    q = inputs.draw_queries(W, Hq, 0, 90)
    scale = 1 / math.sqrt(D)
    ref, ref_lse = sdpa_reference(kv, q, scale)
    out, lse = scattered_paged(oracle_mod, kv, q, scale, seed=N, page_tokens=T)
    assert np.max(np.abs(out - ref)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


PAIR_CASES = [
    # (N, Hq, Hkv, W, page_tokens)
    (300, 6, 2, 3, 256),      # ragged last page, GQA 3:1
    (200, 8, 2, 6, 64),       # small pages, 6 verify rows
    (37, 4, 1, 2, 32),        # fewer keys than one page
]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("N,Hq,Hkv,W,T", PAIR_CASES)
def test_pair_attention_matches_library_sdpa(oracle_mod, pair, N, Hq, Hkv, W, T):
    """Every supported (K, V) element-type pair, pages scattered over pool,
    ring and host, against torch's fp64 SDPA on the quantiser's unpaged
    arrays dequantised by the block-format definitions."""
    kv = cache(N, Hkv, page_tokens=T, k_type=pair[0], v_type=pair[1], pad="garbage")
    q = inputs.draw_queries(W, Hq, 0, 91)
    scale = 1 / math.sqrt(D)
    ref, ref_lse = sdpa_reference(kv, q, scale)
    out, lse = scattered_paged(oracle_mod, kv, q, scale, seed=N + pair[0], page_tokens=T)
    assert np.max(np.abs(out - ref)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
def test_pair_page_bytes_closed_form(oracle_mod, pair):
    """Per (head, token): code bytes (128 Q8_0, 64 Q4_0, 256 F16) plus 8 scale
    bytes for each block type."""
    per = {Q8_0: 128 + 8, Q4_0: 64 + 8, F16: 256}
    for H, T in [(8, 256), (2, 64), (1, 32)]:
        want = H * T * (per[pair[0]] + per[pair[1]])
        assert oracle_mod.page_bytes(H, T, *pair) == want == inputs.page_bytes(H, T, *pair)
        assert oracle_mod.pair_supported(*pair)
    assert not oracle_mod.pair_supported(Q4_0, Q8_0) and not oracle_mod.pair_supported(F16, Q4_0)


def test_pair_codes_exhaustive():
    """Every 4-bit K code, every int8 V code and every binary16 pattern as a
    K and a V element is read back from packed pages with its own bits."""
    import oracle as om
    T, H = 256, 2
    j = torch.arange(T).view(-1, 1, 1)
    h = torch.arange(H).view(1, -1, 1)
    t = torch.arange(D).view(1, 1, -1)
    sc = torch.tensor(SCALES, dtype=torch.float16)
    kd = sc[(j * 4 + torch.arange(4).view(1, 1, -1) + h) % len(SCALES)].expand(T, H, 4).contiguous()
    vd = sc[(j * 4 + torch.arange(4).view(1, 1, -1) + 2 + h) % len(SCALES)].expand(T, H, 4).contiguous()
    # Q4_0 K / Q4_0 V
    kc4 = ((j * 5 + t * 3 + h) % 16).expand(T, H, D).to(torch.uint8).contiguous()
    vc4 = ((j * 7 + t + 2 * h) % 16).expand(T, H, D).to(torch.uint8).contiguous()
    page = inputs.pack_pages(kc4, kd, vc4, vd, T, k_type=Q4_0, v_type=Q4_0)[0].numpy()
    a, b, c, e = om.unpack_page(page, H, T, Q4_0, Q4_0)
    assert np.array_equal(a, kc4.numpy()) and np.array_equal(c, vc4.numpy())
    assert np.array_equal(b, kd.numpy().view(np.uint16)) and np.array_equal(e, vd.numpy().view(np.uint16))
    assert set(np.unique(a)) == set(range(16))
    # Q8_0 K / Q8_0 V
    kc8 = (((j * 128 + t + 97 * h) % 256) - 128).expand(T, H, D).to(torch.int8).contiguous()
    vc8 = (((j * 131 + t * 3 + 5 * h) % 256) - 128).expand(T, H, D).to(torch.int8).contiguous()
    page = inputs.pack_pages(kc8, kd, vc8, vd, T, k_type=Q8_0, v_type=Q8_0)[0].numpy()
    a, b, c, e = om.unpack_page(page, H, T, Q8_0, Q8_0)
    assert np.array_equal(a, kc8.numpy()) and np.array_equal(c, vc8.numpy())
    assert np.array_equal(e, vd.numpy().view(np.uint16))
    assert set(np.unique(c)) == set(range(-128, 128))
    K, V = om.decode_page(page, H, T, Q8_0, Q8_0)
    assert np.array_equal(V, np.repeat(vd.double().numpy(), 32, -1) * vc8.double().numpy())
    # F16 / F16: all 65,536 patterns (T * H * D = 65,536), V in another order
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, H, D)
    kf = torch.from_numpy(bits.copy()).view(torch.float16)
    vf = torch.from_numpy(bits[::-1].copy()).view(torch.float16)
    page = inputs.pack_pages(kf, None, vf, None, T, k_type=F16, v_type=F16)[0].numpy()
    assert page.size == H * T * 512
    a, _, c, _ = om.unpack_page(page, H, T, F16, F16)
    assert np.array_equal(a.astype(np.uint16), bits) and np.array_equal(c.astype(np.uint16), bits[::-1])
    K, V = om.decode_page(page, H, T, F16, F16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(K[fin], ref[fin]) and np.array_equal(np.isnan(K), np.isnan(ref))


@pytest.mark.parametrize("pair", PAIRS[1:], ids=PAIR_IDS[1:])
def test_pair_split_merge_identity(oracle_mod, pair):
    N, Hq, H, W = 700, 4, 2, 3
    kv = cache(N, H, k_type=pair[0], v_type=pair[1])
    q = inputs.draw_queries(W, Hq, 0, 92)
    s = 1 / math.sqrt(D)
    full, _ = identity_paged(oracle_mod, kv, q, s)
    bounds = [0, 100, 256, 257, 600, N + 10]
    m, l, acc = oracle_mod.split_partials(kv.pages.numpy(), 256, N, Hq, H, q.numpy(), s, bounds,
                                          k_type=pair[0], v_type=pair[1])
    assert np.max(np.abs(oracle_mod.merge(m, l, acc) - full)) <= 1e-12


def test_logical_equals_paged_bitwise(oracle_mod):
    kv = cache(700, 2)
    q = inputs.draw_queries(4, 4, 0, 90)
    s = 1 / math.sqrt(D)
    a, la = oracle_mod.attend_logical(*np_arrays(kv), 4, q.numpy(), s)
    b, lb = identity_paged(oracle_mod, kv, q, s)
    c, lc = scattered_paged(oracle_mod, kv, q, s, seed=5)
    assert np.array_equal(a, b) and np.array_equal(b, c)
    assert np.array_equal(la, lb) and np.array_equal(lb, lc)


def test_padding_bytes_never_read(oracle_mod):
    """A ragged last page filled with random bytes (NaN-able scales) gives
    the same bits as a zero-filled one."""
    a = cache(300, 2, pad="zero")
    b = cache(300, 2, pad="garbage")
    assert not np.array_equal(a.pages.numpy(), b.pages.numpy())
    q = inputs.draw_queries(2, 4, 0, 90)
    s = 1 / math.sqrt(D)
    oa, _ = identity_paged(oracle_mod, a, q, s)
    ob, _ = identity_paged(oracle_mod, b, q, s)
    assert np.array_equal(oa, ob) and np.isfinite(oa).all()


def exact_mean_visible_v(kv, rows_pos, Hq):
    """Exact rational mean of V-hat over keys 0..pos, per (row, head)."""
    H = kv.kc.shape[1]
    G = Hq // H
    vd = kv.vd.double().numpy()
    vc = kv.vc.numpy().astype(np.int64) - 8
    out = np.empty((len(rows_pos), Hq, D))
    for ri, pos in enumerate(rows_pos):
        for g in range(H):
            for t in range(0, D, 9):   # a stride of dims keeps the rational sums quick
                s = sum((Fraction(vd[j, g, t // 32]) * int(vc[j, g, t]) for j in range(pos + 1)), Fraction(0))
                for h in range(g * G, (g + 1) * G):
                    out[ri, h, t] = float(s / (pos + 1))
    return out


def test_zero_query_gives_exact_mean(oracle_mod):
    """q = 0: every visible key weighs 1, so O is the mean of the visible V-hat."""
    N, W, Hq = 300, 3, 4
    kv = cache(N, 2)
    q = torch.zeros(W, Hq, D)
    out, lse = identity_paged(oracle_mod, kv, q, 1 / math.sqrt(D))
    ref = exact_mean_visible_v(kv, [N - W + r for r in range(W)], Hq)
    assert np.max(np.abs(out[:, :, ::9] - ref[:, :, ::9])) <= 1e-15
    assert np.allclose(lse, np.log([N - W + r + 1 for r in range(W)])[:, None], rtol=0, atol=1e-13)


def test_zero_scale_and_zero_keys_give_mean(oracle_mod):
    N, Hq = 260, 4
    kv = cache(N, 1)
    q = inputs.draw_queries(1, Hq, 0, 90)
    ref = exact_mean_visible_v(kv, [N - 1], Hq)
    out0, _ = identity_paged(oracle_mod, kv, q, 0.0)
    assert np.max(np.abs(out0[:, :, ::9] - ref[:, :, ::9])) <= 1e-15
    kz = inputs.LayerKV(torch.zeros_like(kv.kc), kv.kd, kv.vc, kv.vd)
    kz.pages = inputs.pack_pages(kz.kc, kz.kd, kz.vc, kz.vd)
    outz, _ = identity_paged(oracle_mod, kz, q, 1 / math.sqrt(D))
    assert np.max(np.abs(outz[:, :, ::9] - ref[:, :, ::9])) <= 1e-15


def test_constant_values(oracle_mod):
    """V-hat == c everywhere => O == c whatever the scores."""
    c = 0.8125  # binary16-exact; codes 9 give c * (9 - 8)
    base = cache(513, 2)
    kv = inputs.LayerKV(base.kc, base.kd, torch.full_like(base.vc, 9), torch.full_like(base.vd, c))
    kv.pages = inputs.pack_pages(kv.kc, kv.kd, kv.vc, kv.vd)
    q = inputs.draw_queries(4, 6, 0, 90) * 3
    out, _ = identity_paged(oracle_mod, kv, q, 1 / math.sqrt(D))
    assert np.max(np.abs(out - c)) <= 1e-14


def test_single_visible_key(oracle_mod):
    """One key in the history: O equals its V-hat exactly."""
    kv = cache(1, 2)
    q = inputs.draw_queries(1, 4, 0, 90)
    out, lse = identity_paged(oracle_mod, kv, q, 1 / math.sqrt(D))
    V = kv.vd.double().repeat_interleave(32, -1) * (kv.vc.double() - 8)
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, h // 2].numpy())


def test_gqa_head_map(oracle_mod):
    """V-hat of KV head g set to g+1: every query head h reads floor(h/G)+1."""
    N, H, G = 600, 4, 3
    base = cache(N, H)
    vd = torch.arange(1, H + 1, dtype=torch.float16).view(1, H, 1).expand(N, H, 4).contiguous()
    kv = inputs.LayerKV(base.kc, base.kd, torch.full_like(base.vc, 9), vd)
    kv.pages = inputs.pack_pages(kv.kc, kv.kd, kv.vc, kv.vd)
    q = inputs.draw_queries(2, H * G, 0, 90)
    out, _ = identity_paged(oracle_mod, kv, q, 1 / math.sqrt(D))
    for h in range(H * G):
        assert np.max(np.abs(out[:, h] - (h // G + 1))) <= 1e-14


@pytest.mark.parametrize("N", [2048, 2048 - 37, 1000])
def test_page_id_closed_form(oracle_mod, N):
    """Logical page P: K-hat = P in dim 0 (scale 1, code P), V-hat = (P+1)/16
    everywhere (scale (P+1)/16, code 9).  With q = e0 the weights are
    n_P * e^(s*P) for the n_P visible keys of page P: an exact few-term
    closed form that any missing, doubled or misplaced page breaks."""
    T, H = 256, 1
    kv = const_cache(N, H,
                     kc=lambda j, h, t: torch.where(t == 0, j // T, torch.zeros_like(t)),
                     kd=lambda j, h, b: torch.ones_like(b, dtype=torch.float64),
                     vc=lambda j, h, t: torch.full_like(t, 9),
                     vd=lambda j, h, b: ((j // T) + 1) / 16.0 + 0 * b)
    q = torch.zeros(1, 2, D)
    q[0, :, 0] = 1.0
    s = 1 / math.sqrt(D)
    out, lse = scattered_paged(oracle_mod, kv, q, s, seed=N)
    n_pages = -(-N // T)
    counts = [min(T, N - P * T) for P in range(n_pages)]
    num = sum(c * math.exp(s * P) * (P + 1) / 16 for P, c in enumerate(counts))
    den = sum(c * math.exp(s * P) for P, c in enumerate(counts))
    assert np.max(np.abs(out - num / den)) <= 1e-13
    # drop the last page: the closed form moves far beyond any tolerance
    num2 = sum(c * math.exp(s * P) * (P + 1) / 16 for P, c in enumerate(counts[:-1]))
    den2 = sum(c * math.exp(s * P) for P, c in enumerate(counts[:-1]))
    assert abs(num2 / den2 - num / den) > 1e-2


def test_causality(oracle_mod):
    """Row r's output ignores keys after its position, and equals single-row
    attention over keys 0..p_r."""
    N, W, Hq, H = 520, 4, 4, 2
    a = cache(N, H, wid=91)
    q = inputs.draw_queries(W, Hq, 0, 90)
    s = 1 / math.sqrt(D)
    out, lse = identity_paged(oracle_mod, a, q, s)
    b = cache(N, H, wid=92)   # different keys everywhere ...
    for r in range(W):
        p = N - W + r
        kc, kd = a.kc.clone(), a.kd.clone()
        vc, vd = a.vc.clone(), a.vd.clone()
        kc[p + 1:], kd[p + 1:], vc[p + 1:], vd[p + 1:] = b.kc[p + 1:], b.kd[p + 1:], b.vc[p + 1:], b.vd[p + 1:]
        m = inputs.LayerKV(kc, kd, vc, vd)   # ... after row r's position only
        m.pages = inputs.pack_pages(kc, kd, vc, vd)
        o2, _ = identity_paged(oracle_mod, m, q, s)
        assert np.array_equal(o2[r], out[r])
        short = inputs.LayerKV(a.kc[:p + 1], a.kd[:p + 1], a.vc[:p + 1], a.vd[:p + 1])
        short.pages = inputs.pack_pages(short.kc, short.kd, short.vc, short.vd)
        o3, l3 = identity_paged(oracle_mod, short, q[r:r + 1], s)
        assert np.array_equal(o3[0], out[r]) and np.array_equal(l3[0], lse[r])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_merge_identity(oracle_mod, seed):
    """Partials over any split plan, merged by log-sum-exp in split order,
    equal the unsplit attention (empty splits included)."""
    N, W, Hq, H = 777, 3, 4, 2
    kv = cache(N, H)
    q = inputs.draw_queries(W, Hq, 0, 90)
    s = 1 / math.sqrt(D)
    full, _ = identity_paged(oracle_mod, kv, q, s)
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, N + 40), size=6, replace=False))
    bounds = np.concatenate([[0], cuts, [N + 50]])   # last splits may be empty / past the rows
    m, l, acc = oracle_mod.split_partials(kv.pages.numpy(), 256, N, Hq, H, q.numpy(), s, bounds)
    merged = oracle_mod.merge(m, l, acc)
    assert np.max(np.abs(merged - full)) <= 1e-12
    one = oracle_mod.merge(*oracle_mod.split_partials(kv.pages.numpy(), 256, N, Hq, H, q.numpy(), s,
                                                      [0, N]))
    assert np.max(np.abs(one - full)) <= 1e-13


MUTATIONS = [
    # (name, pair, text in oracle.c, planted replacement)
    ("nibble halves swapped", (Q8_0, Q4_0), "return jj < 16 ? (byte & 0x0F) : (byte >> 4);",
     "return jj >= 16 ? (byte & 0x0F) : (byte >> 4);"),
    ("Q4_0 offset wrong", (Q8_0, Q4_0), "return scale * (double)(code - 8);", "return scale * (double)(code - 7);"),
    ("K layout half-block offset dropped", (Q8_0, Q4_0), "(size_t)((t / 32) % 2) * 8 + (size_t)(t % 8);",
     "(size_t)((t / 32) % 2) * 0 + (size_t)(t % 8);"),
    ("GQA map transposed", (Q8_0, Q4_0), "attend_range(src, h / G,", "attend_range(src, h % Hkv,"),
    ("causal mask off by one", (Q8_0, Q4_0), "scale, 0, pos + 1, &m, &l, acc);", "scale, 0, pos, &m, &l, acc);"),
    ("K scale block index wrong", (Q8_0, Q4_0),
     "sec_k_scales(kt, vt, H, T) + (((size_t)head * T + j) * N_BLOCKS + block) * 2;",
     "sec_k_scales(kt, vt, H, T) + (((size_t)head * T + j) * N_BLOCKS + (block ^ 1)) * 2;"),
    ("V scale tile slot wrong", (Q8_0, Q4_0), "(size_t)((jj / 16) * 4 + jj % 4) * 2;",
     "(size_t)((jj / 16) * 4 + (jj + 1) % 4) * 2;"),
    ("V tile stride wrong", (Q8_0, Q4_0), "(size_t)(j / 32) * 32 * vc;", "(size_t)(j / 32) * 16 * vc;"),
    ("Q4_0 K nibble halves swapped", (Q4_0, Q4_0), "return (t % 8) < 4 ? (byte & 0x0F) : (byte >> 4);",
     "return (t % 8) >= 4 ? (byte & 0x0F) : (byte >> 4);"),
    ("Q8_0 V half-tile offset dropped", (Q8_0, Q8_0), "lane * 16 + (size_t)((t / 16) % 2) * 8 + (size_t)slot]",
     "lane * 16 + (size_t)((t / 16) % 2) * 0 + (size_t)slot]"),
    ("F16 K dimension-group stride wrong", (F16, F16),
     "(size_t)(t / 32) * 1024 + lane * 16 + (size_t)(t % 8) * 2);",
     "(size_t)(t / 32) * 512 + lane * 16 + (size_t)(t % 8) * 2);"),
    ("F16 V slot order wrong", (F16, F16), "(size_t)(t / 16) * 1024 + lane * 16 + (size_t)slot * 2);",
     "(size_t)(t / 16) * 1024 + lane * 16 + (size_t)(slot ^ 1) * 2);"),
]


@pytest.mark.parametrize("name,pair,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_oracle_mistake_fails_pin(oracle_mod, tmp_path, name, pair, old, new):
    """Plant a plausible mistake in a copy of the oracle's C source, build it
    on the CPU, and check that the library-routine pin rejects it."""
    import ctypes
    import subprocess
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")).read()
    assert src.count(old) == 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so),
                           str(mutated), "-lm"])
    lib = ctypes.CDLL(str(so))
    P, I, Z, Dd = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
    lib.oracle_attend_paged.argtypes = [P, Z, P, Z, P, P, I, I, I, I, I, I, P, I, Dd, P, I, P, P, I]
    N, Hq, H, W = 300, 6, 2, 3
    kv = cache(N, H, k_type=pair[0], v_type=pair[1])
    q = inputs.draw_queries(W, Hq, 0, 90)
    s = 1 / math.sqrt(D)
    ref, _ = sdpa_reference(kv, q, s)
    pool = np.ascontiguousarray(kv.pages.numpy())
    pt = np.arange(pool.shape[0], dtype=np.uint32)
    qn = np.ascontiguousarray(q.numpy())
    out = np.zeros((W, Hq, D))
    lse = np.zeros((W, Hq))
    rc = lib.oracle_attend_paged(pool.ctypes.data, pool.shape[0], None, 0, None, pt.ctypes.data, N, 256, pair[0],
                                 pair[1], Hq, H, qn.ctypes.data, W, s, None, W, out.ctypes.data, lse.ctypes.data, 1)
    assert rc == 0
    assert not np.max(np.abs(out - ref)) <= 1e-12, f"pin missed the planted mistake: {name}"
