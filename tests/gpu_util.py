"""Helpers for the GPU tests: build handles and place seeded pages.

Placement only (which page goes to which pool page or ring slot); every
attention step runs in the HIP library, every reference in the oracle.
"""
import sys

import numpy as np
import torch

import inputs
import long_context_attention_amd as kv
import oracle

TOL = 2e-3  # max-abs tolerance against the fp64 oracle (fp32 accumulation)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def handle(Hq, Hkv, n_pool, max_pages, max_rows, n_ring=0, split_pages=0, chunk_slots=0, n_layers=1,
           page_tokens=256, k_type=kv.TYPE_Q8_0, v_type=kv.TYPE_Q4_0, deterministic=0, compute_stream=None):
    p = kv.make_params(n_layers, Hq, Hkv, n_pool, max_pages, max_rows, n_ring_slots=n_ring,
                       split_pages=split_pages, chunk_slots=chunk_slots, page_tokens=page_tokens,
                       k_type=k_type, v_type=v_type, deterministic=deterministic)
    return kv.allocate(p, compute_stream=compute_stream)


def place(h, layer, kvl, table, history=None, page_tokens=256):
    """Copy the layer's pages to where `table` says (device copies into the
    caller-owned pool / ring) and set the layer."""
    pb = kv.page_bytes(h.params)
    pages = kvl.pages.to("cuda")
    n = pages.shape[0]
    for P in range(n):
        e = int(table[P])
        if e == kv.PT_HOST:
            continue
        if e & kv.PT_RING_FLAG:
            s = e & 0x7FFFFFFF
            h.ring[s * pb:(s + 1) * pb].copy_(pages[P])
        else:
            h.pool[e * pb:(e + 1) * pb].copy_(pages[P])
    torch.cuda.synchronize()
    h.set_layer(layer, np.asarray(table, dtype=np.uint32), kvl.kc.shape[0], history)


def oracle_out(kvl, q, Hq, Hkv, rows=None, page_tokens=256):
    n = kvl.pages.shape[0]
    out, _ = oracle.attend_paged(np.arange(n, dtype=np.uint32), kvl.kc.shape[0], page_tokens, Hq, Hkv,
                                 q.cpu().numpy(), inputs.scale_for(), pool=kvl.pages.cpu().numpy(), rows=rows,
                                 k_type=kvl.k_type, v_type=kvl.v_type)
    return out


def run(h, layer, q, W, kind):
    qd = q.to("cuda").contiguous()
    out = torch.full_like(qd, float("nan"))
    if kind == "decode":
        h.decode(layer, qd, out)
    elif kind == "verify":
        h.verify(layer, qd, W, out)
    else:
        h.prefill_chunk(layer, qd, W, out)
    h.synchronize()
    return out.cpu().double().numpy()
