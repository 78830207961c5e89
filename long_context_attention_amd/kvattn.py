"""ctypes binding of the kvattn C-ABI (include/kvattn.h).

Argument marshalling only: every step of the attention path runs in the HIP
library ``libkvattn.so``.  PyTorch provides device memory, pinned host memory
and streams.  Loading fails loudly when the library has not been built;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvattn.so")

OK, E_ARG, E_UNSUPPORTED, E_RANGE, E_PLAN, E_NOSPACE, E_STATE, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "OK", -1: "E_ARG", -2: "E_UNSUPPORTED", -3: "E_RANGE", -4: "E_PLAN", -5: "E_NOSPACE",
                -6: "E_STATE", -7: "E_HIP"}
TYPE_F16, TYPE_Q4_0, TYPE_Q8_0 = 1, 2, 8
PT_RING_FLAG = 0x80000000
PT_HOST = 0xFFFFFFFF
HEAD_DIM = 128


def PT_RING(slot: int) -> int:
    return PT_RING_FLAG | int(slot)


class KVAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"kvattn {STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "struct_size", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "page_tokens", "k_type", "v_type",
        "n_pool_pages", "n_ring_slots", "max_pages_per_layer", "max_rows")] + [
        ("softmax_scale", ctypes.c_float), ("split_pages", ctypes.c_uint32), ("chunk_slots", ctypes.c_uint32),
        ("deterministic", ctypes.c_uint32)]


def make_params(n_layers, n_q_heads, n_kv_heads, n_pool_pages, max_pages_per_layer, max_rows, n_ring_slots=0,
                page_tokens=256, softmax_scale=0.0, split_pages=0, chunk_slots=0, head_dim=HEAD_DIM,
                k_type=TYPE_Q8_0, v_type=TYPE_Q4_0, deterministic=0) -> Params:
    p = Params()
    p.struct_size = ctypes.sizeof(Params)
    p.n_layers, p.n_q_heads, p.n_kv_heads, p.head_dim = n_layers, n_q_heads, n_kv_heads, head_dim
    p.page_tokens, p.k_type, p.v_type = page_tokens, k_type, v_type
    p.n_pool_pages, p.n_ring_slots, p.max_pages_per_layer, p.max_rows = n_pool_pages, n_ring_slots, \
        max_pages_per_layer, max_rows
    p.softmax_scale, p.split_pages, p.chunk_slots = softmax_scale, split_pages, chunk_slots
    p.deterministic = deterministic
    return p


POLICY_FITS, POLICY_HOLD, POLICY_CONTEXT, POLICY_GROW_RING, POLICY_SHRINK_RING = 0, 1, 2, 3, 4


class PolicyConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "n_layers", "page_tokens", "budget_pages", "min_ring_slots", "max_ring_slots", "ring_step", "grow_after",
        "shrink_after")] + [(n, ctypes.c_float) for n in ("miss_rate_high", "busy_high", "occupancy_low")]


class PolicyState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "ring_slots", "pages_per_layer", "pressure_streak", "saturated_streak", "idle_streak")]


class PolicyObservation(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ("n_tokens", "chunks", "ready_misses")] + [
        (n, ctypes.c_float) for n in ("ring_occupancy", "copy_busy")]


class PolicyDecision(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "reason", "changed", "ring_slots", "pages_per_layer", "resident_pages", "streamed_pages", "streamed_layers")]


def policy_config(n_layers, page_tokens, budget_pages, min_ring_slots=16, max_ring_slots=256, ring_step=16,
                  grow_after=2, shrink_after=4, miss_rate_high=0.25, busy_high=0.9, occupancy_low=0.5):
    return PolicyConfig(n_layers, page_tokens, budget_pages, min_ring_slots, max_ring_slots, ring_step, grow_after,
                        shrink_after, miss_rate_high, busy_high, occupancy_low)


_lib = None
EXPORTS = ["kvattn_supported", "kvattn_page_bytes", "kvattn_workspace_bytes", "kvattn_create",
           "kvattn_upload_pages", "kvattn_set_layer", "kvattn_decode", "kvattn_verify", "kvattn_verify_noalloc",
           "kvattn_prefill_chunk",
           "kvattn_append",
           "kvattn_synchronize", "kvattn_debug_read_page", "kvattn_debug_count_rescales", "kvattn_debug_check_ring", "kvattn_validate_page_table", "kvattn_sched_simulate",
           "kvattn_profile", "kvattn_profile_read", "kvattn_policy_step", "kvattn_observe", "kvattn_observe_read",
           "kvattn_set_ring_slots", "kvattn_destroy",
           "kvattn_last_error", "kvattn_global_error"]


def lib():
    """Load libkvattn.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m long_context_attention_amd.build "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, U, Z, I = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_int
    PP = ctypes.POINTER(Params)
    L.kvattn_supported.argtypes = [U, U, U]
    L.kvattn_supported.restype = I
    L.kvattn_page_bytes.argtypes = [PP]
    L.kvattn_page_bytes.restype = Z
    L.kvattn_workspace_bytes.argtypes = [PP]
    L.kvattn_workspace_bytes.restype = Z
    L.kvattn_create.argtypes = [PP, P, Z, P, Z, P, Z, P, P, ctypes.POINTER(P)]
    L.kvattn_create.restype = I
    L.kvattn_upload_pages.argtypes = [P, P, P, U]
    L.kvattn_upload_pages.restype = I
    L.kvattn_set_layer.argtypes = [P, U, P, U, P]
    L.kvattn_set_layer.restype = I
    L.kvattn_decode.argtypes = [P, U, P, P]
    L.kvattn_decode.restype = I
    L.kvattn_verify.argtypes = [P, U, P, U, P]
    L.kvattn_verify.restype = I
    L.kvattn_verify_noalloc.argtypes = [P, U, P, U, P]
    L.kvattn_verify_noalloc.restype = I
    L.kvattn_prefill_chunk.argtypes = [P, U, P, U, P]
    L.kvattn_prefill_chunk.restype = I
    L.kvattn_append.argtypes = [P, U, P, P, U, P, U, P]
    L.kvattn_append.restype = ctypes.c_int
    L.kvattn_synchronize.argtypes = [P]
    L.kvattn_synchronize.restype = I
    L.kvattn_debug_read_page.argtypes = [P, U, U, P]
    L.kvattn_debug_read_page.restype = I
    L.kvattn_debug_count_rescales.argtypes = [P, P]
    L.kvattn_debug_count_rescales.restype = I
    L.kvattn_debug_check_ring.argtypes = [P, P, U]
    L.kvattn_debug_check_ring.restype = I
    L.kvattn_validate_page_table.argtypes = [PP, P, U, I]
    L.kvattn_validate_page_table.restype = I
    L.kvattn_sched_simulate.argtypes = [U, U, U, P, P, U, P, U, ctypes.POINTER(U)]
    L.kvattn_sched_simulate.restype = I
    L.kvattn_profile.argtypes = [P, U]
    L.kvattn_profile.restype = I
    L.kvattn_profile_read.argtypes = [P, I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(U),
                                      ctypes.POINTER(ctypes.c_double), ctypes.POINTER(U)]
    L.kvattn_profile_read.restype = I
    L.kvattn_policy_step.argtypes = [ctypes.POINTER(PolicyConfig), ctypes.POINTER(PolicyState),
                                     ctypes.POINTER(PolicyObservation), ctypes.POINTER(PolicyState),
                                     ctypes.POINTER(PolicyDecision), P]
    L.kvattn_policy_step.restype = I
    L.kvattn_observe.argtypes = [P, U]
    L.kvattn_observe.restype = I
    L.kvattn_observe_read.argtypes = [P, I, ctypes.POINTER(PolicyObservation)]
    L.kvattn_observe_read.restype = I
    L.kvattn_set_ring_slots.argtypes = [P, U]
    L.kvattn_set_ring_slots.restype = I
    L.kvattn_destroy.argtypes = [P]
    L.kvattn_destroy.restype = I
    L.kvattn_last_error.argtypes = [P]
    L.kvattn_last_error.restype = ctypes.c_char_p
    L.kvattn_global_error.argtypes = []
    L.kvattn_global_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc, handle=None):
    if rc != OK:
        L = lib()
        msg = (L.kvattn_last_error(handle) if handle else L.kvattn_global_error()) or b""
        raise KVAttnError(rc, msg.decode(errors="replace"))


def _addr(t):
    """Device or host address of a tensor / numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


# ---------------------------------------------------------------- free functions
def policy_step(config: PolicyConfig, state: PolicyState, observation: PolicyObservation):
    """One step of the resident/ring policy: (next state, decision, resident
    pages per layer)."""
    nxt, dec = PolicyState(), PolicyDecision()
    resident = np.zeros(config.n_layers, dtype=np.uint32)
    _check(lib().kvattn_policy_step(ctypes.byref(config), ctypes.byref(state), ctypes.byref(observation),
                                    ctypes.byref(nxt), ctypes.byref(dec), resident.ctypes.data))
    return nxt, dec, resident


def supported(k_type=TYPE_Q8_0, v_type=TYPE_Q4_0, head_dim=HEAD_DIM) -> bool:
    return bool(lib().kvattn_supported(k_type, v_type, head_dim))


def page_bytes(params: Params) -> int:
    return int(lib().kvattn_page_bytes(ctypes.byref(params)))


def workspace_bytes(params: Params) -> int:
    return int(lib().kvattn_workspace_bytes(ctypes.byref(params)))


def validate_page_table(params: Params, page_table, n_tokens, has_history=False):
    """Status kvattn_set_layer would return for this table (host-only check)."""
    pt = np.ascontiguousarray(page_table, dtype=np.uint32)
    return int(lib().kvattn_validate_page_table(ctypes.byref(params), pt.ctypes.data, n_tokens, int(has_history)))


def global_error() -> str:
    return (lib().kvattn_global_error() or b"").decode(errors="replace")


def sched_simulate(n_layers, n_slots, chunk_slots, streamed_counts, call_layers, max_ops=1 << 20):
    counts = np.ascontiguousarray(streamed_counts, dtype=np.uint32)
    calls = np.ascontiguousarray(call_layers, dtype=np.uint32)
    ops = np.zeros((max_ops, 7), dtype=np.int64)
    n = ctypes.c_uint32(0)
    rc = lib().kvattn_sched_simulate(n_layers, n_slots, chunk_slots, counts.ctypes.data, calls.ctypes.data,
                                     len(calls), ops.ctypes.data, max_ops, ctypes.byref(n))
    if rc != OK:
        raise KVAttnError(rc, "kvattn_sched_simulate")
    return ops[: n.value].copy()


# ---------------------------------------------------------------- handle
class Handle:
    """A kvattn handle over caller-owned buffers (torch tensors kept alive here)."""

    def __init__(self, params: Params, pool, ring, workspace, compute_stream, copy_stream=None):
        self.params = params
        self._keep = [pool, ring, workspace]
        h = ctypes.c_void_p()
        rc = lib().kvattn_create(ctypes.byref(params), _addr(pool), 0 if pool is None else pool.numel(),
                                 _addr(ring), 0 if ring is None else ring.numel(), _addr(workspace),
                                 workspace.numel(), ctypes.c_void_p(compute_stream),
                                 ctypes.c_void_p(copy_stream if copy_stream is not None else compute_stream),
                                 ctypes.byref(h))
        _check(rc)
        self.h = h
        self._hist = {}
        self._tables = {}

    # -- marshalling wrappers (same names as the C entry points)
    def upload_pages(self, host_pages, dst):
        d = np.ascontiguousarray(dst, dtype=np.uint32)
        self._keep.append(host_pages)
        _check(lib().kvattn_upload_pages(self.h, _addr(host_pages), d.ctypes.data, len(d)), self.h)

    def set_layer(self, layer, page_table, n_tokens, history=None):
        pt = np.ascontiguousarray(page_table, dtype=np.uint32)
        self._hist[layer] = history
        _check(lib().kvattn_set_layer(self.h, layer, pt.ctypes.data, n_tokens, _addr(history)), self.h)
        self._tables[layer] = pt

    def layer_table(self, layer):
        """The page table last passed to set_layer for `layer` (host copy)."""
        return self._tables[layer]

    def decode(self, layer, q, out):
        _check(lib().kvattn_decode(self.h, layer, _addr(q), _addr(out)), self.h)

    def verify(self, layer, q, W, out):
        _check(lib().kvattn_verify(self.h, layer, _addr(q), W, _addr(out)), self.h)

    def verify_noalloc(self, layer, q, W, out):
        _check(lib().kvattn_verify_noalloc(self.h, layer, _addr(q), W, _addr(out)), self.h)

    def prefill_chunk(self, layer, q, R, out):
        _check(lib().kvattn_prefill_chunk(self.h, layer, _addr(q), R, _addr(out)), self.h)

    def append(self, layer, k, v, R, new_pages=None, publish=None):
        """Quantise R new rows (k, v: device fp32 [R][Hkv][128]) into the
        layer's pages; new_pages: pool ids for the pages the growth adds;
        publish: host buffer that receives the written pages (or None)."""
        n = 0 if new_pages is None else len(new_pages)
        np_ = np.ascontiguousarray(new_pages if new_pages is not None else [], dtype=np.uint32)
        if publish is not None:
            self._keep.append(publish)
        _check(lib().kvattn_append(self.h, layer, _addr(k), _addr(v), R, np_.ctypes.data if n else None, n,
                                   _addr(publish)), self.h)

    def synchronize(self):
        _check(lib().kvattn_synchronize(self.h), self.h)

    def debug_read_page(self, layer, logical_page):
        out = np.empty(page_bytes(self.params), dtype=np.uint8)
        _check(lib().kvattn_debug_read_page(self.h, layer, logical_page, out.ctypes.data), self.h)
        return out

    def count_rescales(self, counter):
        """Test aid: counter is a device uint32 tensor (zeroed by the caller)
        that later calls increment per softmax re-reference event; None stops."""
        _check(lib().kvattn_debug_count_rescales(self.h, None if counter is None else _addr(counter)), self.h)

    def check_ring(self, counters, skew=0):
        """Test aid: counters is a device tensor of two uint32 (zeroed by the
        caller): [0] ring-slot tag mismatches, [1] slot checks, counted around
        every streamed chunk computed from now on; None stops."""
        _check(lib().kvattn_debug_check_ring(self.h, None if counters is None else _addr(counters), skew), self.h)

    def profile(self, max_launches):
        _check(lib().kvattn_profile(self.h, max_launches), self.h)

    def profile_read(self, reset=True):
        """(split_ms_total, n_split, merge_ms_total, n_merge) since profile()."""
        a, b = ctypes.c_double(), ctypes.c_double()
        na, nb = ctypes.c_uint32(), ctypes.c_uint32()
        _check(lib().kvattn_profile_read(self.h, int(reset), ctypes.byref(a), ctypes.byref(na), ctypes.byref(b),
                                         ctypes.byref(nb)), self.h)
        return a.value, na.value, b.value, nb.value

    def observe(self, max_chunks):
        _check(lib().kvattn_observe(self.h, max_chunks), self.h)

    def observe_read(self, n_tokens=0, reset=True) -> PolicyObservation:
        o = PolicyObservation()
        o.n_tokens = n_tokens
        _check(lib().kvattn_observe_read(self.h, int(reset), ctypes.byref(o)), self.h)
        return o

    def set_ring_slots(self, n_slots):
        _check(lib().kvattn_set_ring_slots(self.h, n_slots), self.h)

    def destroy(self):
        if self.h:
            rc = lib().kvattn_destroy(self.h)
            self.h = None
            _check(rc)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()


def allocate(params: Params, device="cuda", compute_stream=None, copy_stream=None):
    """Allocate pool / ring / workspace with torch on `device` and create a
    handle.  Streams are torch.cuda.Stream objects (default: the current
    stream for compute, a new stream for copies)."""
    import torch
    pb = page_bytes(params)
    if pb == 0:
        raise KVAttnError(E_ARG, "invalid parameters")
    pool = torch.empty(max(1, params.n_pool_pages) * pb, dtype=torch.uint8, device=device)
    ring = torch.empty(params.n_ring_slots * pb, dtype=torch.uint8, device=device) if params.n_ring_slots else None
    ws = torch.empty(workspace_bytes(params), dtype=torch.uint8, device=device)
    cs = compute_stream or torch.cuda.current_stream(device)
    ks = copy_stream or torch.cuda.Stream(device)
    h = Handle(params, pool, ring, ws, cs.cuda_stream, ks.cuda_stream)
    h.pool, h.ring, h.workspace, h.compute_stream, h.copy_stream = pool, ring, ws, cs, ks
    return h


def default_scale():
    return 1.0 / math.sqrt(HEAD_DIM)
