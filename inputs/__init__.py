"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic.  It draws the pre-quantisation
keys, values and queries, encodes keys as Q8_0 and values as Q4_0 (the
workload's cache formats: 32-value blocks with one binary16 scale; int8
codes for K, 4-bit codes offset by 8 for V), packs the encoded cache into
256-token pages, and builds page tables and residency sets.  Both sides
consume the exact bytes produced here, so parity never depends on the
quantiser.

Draws use torch generators seeded from ``numpy.random.SeedSequence`` of
(seed, workload id, layer, tensor id).  A CPU draw and a GPU draw of the same
seed differ (different generator streams); every comparison is made on the
same bytes, never on a re-draw on another device.

Page layout (head_dim 128, T tokens per page, H KV heads; all offsets in
bytes; binary16 little-endian), four sections in order:
  1. K codes, int8, H*T*128: head h at h*T*128, then 16-token tiles of 2048
     bytes.  Inside a tile, byte ``off`` holds key ``off%1024//16 % 16`` of
     the tile and dim ``64*(off//1024) + 32*((off%16)//8) + 8*(off%1024//256)
     + off%8``.
  2. K scales, binary16 [H][T][4].
  3. V codes, 4-bit, H*T*64: head h at h*T*64, then 32-token tiles of 2048
     bytes.  Inside a tile, byte ``off`` holds dim ``64*(off//1024) +
     16*((off%16)//4) + (off%1024//16) % 16`` of two keys: key
     ``4*(off%1024//256) + off%4`` in the low nibble and that key + 16 in the
     high nibble.
  4. V scales, binary16: head h at h*T*8, then 32-token tiles of 256 bytes;
     inside a tile, the 2-byte scale at ``off`` is block ``off//64`` of key
     ``16*(off%16//8) + 4*(off%64//16) + (off%8)//2``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
BLOCK = 32
PAGE_TOKENS = 256
BASE_SEED = 20261202
HOST_ENTRY = 0xFFFFFFFF
RING_FLAG = 0x80000000

# tensor ids for seed derivation
T_K, T_V, T_Q, T_PERM, T_RESIDENT, T_GARBAGE = 1, 2, 3, 4, 5, 6


# --------------------------------------------------------------------------
# Workloads (the pages' geometry: 256-token pages, Q8_0 K / Q4_0 V,
# head_dim 128, 40 query heads over 8 KV heads; contexts 40k-256k)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    n_layers: int
    n_tokens: int
    n_q_heads: int
    n_kv_heads: int
    widths: tuple
    resident_fraction: float = 1.0
    ring_slots: int = 0
    prefill_rows: int = 0
    note: str = ""

    @property
    def n_pages(self) -> int:
        return -(-self.n_tokens // PAGE_TOKENS)

    @property
    def page_bytes(self) -> int:
        return page_bytes(self.n_kv_heads, PAGE_TOKENS)

    @property
    def n_resident(self) -> int:
        return int(round(self.resident_fraction * self.n_pages))


WORKLOADS = {
    "tiny-2k": Workload("tiny-2k", 0, 1, 2048, 4, 1, (1,),
                        note="1 layer, 2048 tokens in 8 pages, GQA 4:1, TG1, permuted page table"),
    "decode-40k": Workload("decode-40k", 1, 64, 40960, 40, 8, (1,),
                           note="all-resident TG1 decode, 160 pages/layer, 64 layers"),
    "verify-160k": Workload("verify-160k", 2, 64, 163840, 40, 8, (1, 2, 3, 4, 5, 6),
                            note="speculative verify widths 1-6, causal tail, 640 pages/layer"),
    "stream-256k": Workload("stream-256k", 3, 64, 262144, 40, 8, (1, 4), resident_fraction=0.4, ring_slots=64,
                            note="40% resident (seeded subset), rest streamed via a 64-slot ring"),
    "prefill-120k": Workload("prefill-120k", 4, 64, 122880 + 256, 40, 8, (256,), prefill_rows=256,
                             note="256-row chunk over a 122,880-token prefix plus itself"),
}


# --------------------------------------------------------------------------
# Seeds
# --------------------------------------------------------------------------
def derive_seed(seed: int, wid: int, layer: int, tensor: int) -> int:
    st = np.random.SeedSequence([seed, wid, layer, tensor]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def generator(seed: int, wid: int, layer: int, tensor: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, wid, layer, tensor))
    return g


# --------------------------------------------------------------------------
# Quantisers (input encoding)
# --------------------------------------------------------------------------
def quantize_q8_0(x: torch.Tensor):
    """fp32 [..., 128] -> (int8 codes [..., 128], float16 scales [..., 4]).

    d = amax / 127 rounded to binary16; code = clamp(round-half-even(x / d),
    -127, 127); a zero scale gives zero codes."""
    xb = x.float().reshape(*x.shape[:-1], -1, BLOCK)
    amax = xb.abs().amax(dim=-1)
    d16 = (amax / 127.0).to(torch.float16)
    d = d16.float().unsqueeze(-1)
    safe = torch.where(d == 0, torch.ones_like(d), d)
    c = torch.round(xb / safe).clamp_(-127, 127)
    c = torch.where(d == 0, torch.zeros_like(c), c)
    return c.to(torch.int8).reshape(x.shape), d16


def quantize_q4_0(x: torch.Tensor):
    """fp32 [..., 128] -> (uint8 codes 0..15 [..., 128], float16 scales [..., 4]).

    m = the block's element of largest magnitude (first on ties, sign kept);
    d = m / -8 rounded to binary16; code = clamp(round-half-even(x / d) + 8,
    0, 15); a zero scale gives codes 8."""
    xb = x.float().reshape(*x.shape[:-1], -1, BLOCK)
    idx = xb.abs().argmax(dim=-1, keepdim=True)  # first index of the maximum
    m = torch.gather(xb, -1, idx).squeeze(-1)
    d16 = (m / -8.0).to(torch.float16)
    d = d16.float().unsqueeze(-1)
    safe = torch.where(d == 0, torch.ones_like(d), d)
    c = (torch.round(xb / safe) + 8).clamp_(0, 15)
    c = torch.where(d == 0, torch.full_like(c, 8), c)
    return c.to(torch.uint8).reshape(x.shape), d16


# --------------------------------------------------------------------------
# Page packing
# --------------------------------------------------------------------------
F16, Q4_0, Q8_0 = 1, 2, 8   # element types


def code_bytes(t: int) -> int:
    return {Q8_0: HEAD_DIM, Q4_0: HEAD_DIM // 2, F16: 2 * HEAD_DIM}[t]


def scale_bytes(t: int) -> int:
    return 0 if t == F16 else 8


def page_bytes(n_kv_heads: int, page_tokens: int = PAGE_TOKENS, k_type: int = Q8_0, v_type: int = Q4_0) -> int:
    return n_kv_heads * page_tokens * (code_bytes(k_type) + scale_bytes(k_type) + code_bytes(v_type) +
                                       scale_bytes(v_type))


def section_offsets(n_kv_heads: int, page_tokens: int = PAGE_TOKENS, k_type: int = Q8_0, v_type: int = Q4_0):
    H, T = n_kv_heads, page_tokens
    k_codes = 0
    k_scales = H * T * code_bytes(k_type)
    v_codes = k_scales + H * T * scale_bytes(k_type)
    v_scales = v_codes + H * T * code_bytes(v_type)
    return k_codes, k_scales, v_codes, v_scales


_gather_cache = {}


def _code_offsets(role: str, t_: int, page_tokens: int, device):
    """Byte offset inside one head's code section of every element (token j,
    dim t), flat index j * 128 + t, and for 4-bit types whether it is the high
    nibble (placement only: the byte formulas of the page layout)."""
    key = (role, t_, page_tokens, str(device))
    if key in _gather_cache:
        return _gather_cache[key]
    T = page_tokens
    j = np.repeat(np.arange(T, dtype=np.int64), HEAD_DIM)
    t = np.tile(np.arange(HEAD_DIM, dtype=np.int64), T)
    hi = None
    if role == "K":
        lane = ((t % 32) // 8) * 16 + j % 16
        if t_ == Q8_0:
            off = (j // 16) * 2048 + (t // 64) * 1024 + lane * 16 + ((t // 32) % 2) * 8 + t % 8
        elif t_ == Q4_0:
            off = (j // 16) * 1024 + lane * 16 + (t // 32) * 4 + (t % 8) % 4
            hi = (t % 8) >= 4
        else:
            off = (j // 16) * 4096 + (t // 32) * 1024 + lane * 16 + (t % 8) * 2
    else:
        jj = j % 32
        g, slot = (jj % 16) // 4, (jj // 16) * 4 + jj % 4
        lane = g * 16 + t % 16
        if t_ == Q4_0:
            off = (j // 32) * 2048 + (t // 64) * 1024 + lane * 16 + ((t // 16) % 4) * 4 + jj % 4
            hi = jj >= 16
        elif t_ == Q8_0:
            off = (j // 32) * 4096 + (t // 32) * 1024 + lane * 16 + ((t // 16) % 2) * 8 + slot
        else:
            off = (j // 32) * 8192 + (t // 16) * 1024 + lane * 16 + slot * 2
    maps = (torch.from_numpy(off).to(device), None if hi is None else torch.from_numpy(hi).to(device))
    _gather_cache[key] = maps
    return maps


def _pack_codes(codes, role, t_, T):
    """codes [n_pages][H][T*128] (int8 codes, nibbles 0..15, or binary16 bits
    as int16) -> section bytes [n_pages][H][T * code_bytes]."""
    n_pages, H, _ = codes.shape
    off, hi = _code_offsets(role, t_, T, codes.device)
    nb = T * code_bytes(t_)
    out = torch.zeros((n_pages, H, nb), dtype=torch.int32, device=codes.device)
    c = codes.to(torch.int32)
    if t_ == Q8_0:
        out[:, :, off] = c & 0xFF
    elif t_ == Q4_0:
        lo_sel, hi_sel = ~hi, hi
        out[:, :, off[lo_sel]] |= c[:, :, lo_sel] & 0x0F
        out[:, :, off[hi_sel]] |= (c[:, :, hi_sel] & 0x0F) << 4
    else:
        out[:, :, off] = c & 0xFF
        out[:, :, off + 1] = (c >> 8) & 0xFF
    return out.to(torch.uint8)


def _vscale_map(page_tokens: int, device):
    """For each 2-byte V-scale slot of one head's section, the flat index
    (token * 4 + block) of the scale stored there."""
    key = ("vd", page_tokens, str(device))
    if key not in _gather_cache:
        slot = np.arange(page_tokens * 4, dtype=np.int64)
        tile, o = slot // 128, (slot % 128) * 2      # o: byte offset inside the 256-byte tile
        block = o // 64
        tok = 32 * tile + 16 * ((o % 16) // 8) + 4 * ((o % 64) // 16) + (o % 8) // 2
        _gather_cache[key] = torch.from_numpy(tok * 4 + block).to(device)
    return _gather_cache[key]


def pack_pages(kc, kd, vc, vd, page_tokens: int = PAGE_TOKENS, pad: str = "zero", pad_seed: int = 0,
               k_type: int = Q8_0, v_type: int = Q4_0):
    """Pack logical arrays into pages.

    kc [N][H][128]: int8 codes (Q8_0), uint8 nibbles 0..15 (Q4_0) or float16
    values (F16); kd float16 [N][H][4] (None for F16); vc, vd likewise for V.
    Returns uint8 [ceil(N/T)][page_bytes] on kc's device.  Token slots beyond
    N in the last page are filled with zeros (pad="zero") or with seeded
    random bytes, NaN-able scales included (pad="garbage"), which a correct
    reader never touches.
    """
    N, H, D = kc.shape
    assert D == HEAD_DIM and page_tokens % 32 == 0
    dev = kc.device
    T = page_tokens
    n_pages = -(-N // T)
    padN = n_pages * T

    def padded(a, kind):
        if padN == N:
            return a
        extra = list(a.shape)
        extra[0] = padN - N
        if pad == "garbage":
            g = torch.Generator(device="cpu")
            g.manual_seed(pad_seed)
            nbytes = int(np.prod(extra)) * a.element_size()
            raw = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8)
            fill = raw.view(a.dtype).reshape(extra).to(dev)
            if kind == "nib":
                fill = fill & 0x0F
        else:
            fill = torch.zeros(extra, dtype=a.dtype, device=dev)
        return torch.cat([a, fill], 0)

    def codes_of(c, t_):
        if t_ == F16:
            c = c.view(torch.int16)
        c = padded(c, "nib" if t_ == Q4_0 else "byte")
        return c.reshape(n_pages, T, H, D).permute(0, 2, 1, 3).reshape(n_pages, H, T * D)

    parts = [_pack_codes(codes_of(kc, k_type), "K", k_type, T).reshape(n_pages, -1)]
    if k_type != F16:
        kd_p = padded(kd, "half").reshape(n_pages, T, H, 4).permute(0, 2, 1, 3)
        parts.append(kd_p.contiguous().view(torch.uint8).reshape(n_pages, H * T * 8))
    parts.append(_pack_codes(codes_of(vc, v_type), "V", v_type, T).reshape(n_pages, -1))
    if v_type != F16:
        vd_p = padded(vd, "half").reshape(n_pages, T, H, 4).permute(0, 2, 1, 3)
        vd_src = _vscale_map(T, dev)
        vd_flat = vd_p.contiguous().reshape(n_pages, H, T * 4)   # (token, block) flat
        parts.append(vd_flat[:, :, vd_src].contiguous().view(torch.uint8).reshape(n_pages, H * T * 8))
    pages = torch.cat(parts, 1)
    assert pages.shape[1] == page_bytes(H, T, k_type, v_type)
    return pages.contiguous()


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------
@dataclass
class LayerKV:
    kc: torch.Tensor  # [N][H][128]: int8 codes (Q8_0), uint8 nibbles (Q4_0) or float16 values (F16)
    kd: torch.Tensor  # float16 [N][H][4], None for F16
    vc: torch.Tensor  # as kc, for V
    vd: torch.Tensor
    pages: torch.Tensor = field(default=None)  # uint8 [n_pages][page_bytes]
    k_type: int = Q8_0
    v_type: int = Q4_0


def quantize(x: torch.Tensor, t_: int):
    """fp32 [..., 128] -> (codes, scales) of element type t_ (F16: the values
    rounded to binary16, no scales)."""
    if t_ == Q8_0:
        return quantize_q8_0(x)
    if t_ == Q4_0:
        return quantize_q4_0(x)
    return x.to(torch.float16), None


def draw_layer(n_tokens, n_kv_heads, layer, wid, seed=BASE_SEED, device="cpu", pack=True, pad="zero",
               page_tokens=PAGE_TOKENS, k_type=Q8_0, v_type=Q4_0):
    """N(0,1) keys and values for one layer, quantised (and packed)."""
    gk = generator(seed, wid, layer, T_K, device)
    gv = generator(seed, wid, layer, T_V, device)
    K = torch.randn((n_tokens, n_kv_heads, HEAD_DIM), generator=gk, device=device, dtype=torch.float32)
    kc, kd = quantize(K, k_type)
    del K
    V = torch.randn((n_tokens, n_kv_heads, HEAD_DIM), generator=gv, device=device, dtype=torch.float32)
    vc, vd = quantize(V, v_type)
    del V
    out = LayerKV(kc, kd, vc, vd, k_type=k_type, v_type=v_type)
    if pack:
        out.pages = pack_pages(kc, kd, vc, vd, page_tokens, pad=pad,
                               pad_seed=derive_seed(seed, wid, layer, T_GARBAGE), k_type=k_type, v_type=v_type)
    return out


def draw_queries(rows, n_q_heads, layer, wid, seed=BASE_SEED, device="cpu"):
    """fp32 N(0,1) queries [rows][Hq][128]."""
    g = generator(seed, wid, layer, T_Q, device)
    return torch.randn((rows, n_q_heads, HEAD_DIM), generator=g, device=device, dtype=torch.float32)


def seeded_permutation(n, layer, wid, seed=BASE_SEED, tensor=T_PERM):
    rng = np.random.default_rng(derive_seed(seed, wid, layer, tensor))
    return rng.permutation(n).astype(np.uint32)


def resident_subset(n_pages, n_resident, layer, wid, seed=BASE_SEED):
    """Sorted logical pages that stay resident (a seeded random subset)."""
    rng = np.random.default_rng(derive_seed(seed, wid, layer, T_RESIDENT))
    return np.sort(rng.choice(n_pages, size=n_resident, replace=False)).astype(np.int64)


def scale_for(head_dim=HEAD_DIM) -> float:
    return 1.0 / math.sqrt(head_dim)
