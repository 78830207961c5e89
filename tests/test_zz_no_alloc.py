"""GPU: kvattn_verify_noalloc (split partials in the library's static device
scratch) against kvattn_verify (partials in the caller's workspace) through
the C ABI: two calls in a row, the second over a shorter history with fewer
rows, each bit for bit equal to kvattn_verify at a fixed chunk order and
within the oracle's tolerance; then the rejections (a plan whose partials
exceed the scratch, a streamed layer)."""
import numpy as np
import pytest
import torch

import inputs
import long_context_attention_amd as kv
from gpu_util import TOL, handle, oracle_out, place, say

pytestmark = pytest.mark.gpu


def test_verify_noalloc_matches_verify():
    Hq, Hkv = 40, 8
    shapes = [(40 * 256 - 9, 6), (9 * 256 + 17, 2)]   # second call: smaller history, fewer rows
    say(f"case no-alloc verify: calls {shapes}")
    layers = [inputs.draw_layer(N, Hkv, l, 95, pad="garbage") for l, (N, _) in enumerate(shapes)]
    n_max = max(x.pages.shape[0] for x in layers)
    h = handle(Hq, Hkv, 2 * n_max, n_max, 64, n_layers=2, deterministic=1)
    for l, x in enumerate(layers):
        n = x.pages.shape[0]
        place(h, l, x, (l * n_max + np.random.default_rng(l).permutation(n)).astype(np.uint32))
    for l, (N, W) in enumerate(shapes):
        q = inputs.draw_queries(W, Hq, l, 95).cuda()
        a = torch.full_like(q, float("nan"))
        b = torch.full_like(q, float("nan"))
        h.verify_noalloc(l, q, W, a)
        h.verify(l, q, W, b)
        h.synchronize()
        err = float(np.max(np.abs(a.cpu().double().numpy() - oracle_out(layers[l], q.cpu(), Hq, Hkv))))
        say(f"  call {l}: N={N} W={W}: bitwise equal to kvattn_verify: {torch.equal(a, b)}; vs oracle {err:.3e}")
        assert torch.equal(a, b)
        assert err <= TOL
    h.destroy()


def test_verify_noalloc_rejections():
    Hq, Hkv, N = 40, 8, 20 * 256
    say("case no-alloc rejections")
    x = inputs.draw_layer(N, Hkv, 0, 96)
    n = x.pages.shape[0]
    h = handle(Hq, Hkv, n, n, 64, n_ring=4, n_layers=2)
    place(h, 0, x, np.arange(n, dtype=np.uint32))
    q = inputs.draw_queries(64, Hq, 0, 96).cuda()
    out = torch.empty_like(q)
    # 64 rows x 40 heads x 320 rows per KV head: the wide plan's partials exceed 8 MiB
    with pytest.raises(kv.KVAttnError) as e:
        h.verify_noalloc(0, q, 64, out)
    assert e.value.code == kv.E_NOSPACE and "static scratch" in str(e.value)
    table = np.full(n, kv.PT_HOST, dtype=np.uint32)
    table[: n // 2] = np.arange(n // 2)
    h.set_layer(1, table, N, x.pages.contiguous().pin_memory())
    with pytest.raises(kv.KVAttnError) as e:
        h.verify_noalloc(1, q[:1].contiguous(), 1, out[:1])
    assert e.value.code == kv.E_UNSUPPORTED
    h.destroy()
