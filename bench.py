#!/usr/bin/env python3
"""Benchmark of paged Q8_0-K / Q4_0-V attention on one MI355X.

A step is one pass of the hot path over one batch: every layer of the
workload attends once (64 layers).  Headline workload: all-resident TG1
decode, 40,960-token history (160 pages of 256 tokens) per layer, 40 query
heads over 8 KV heads, head_dim 128, 64 layers with their own seeded N(0,1)
data, pages scattered over the pool by a seeded permutation.  Inputs are
resident in HBM before timing starts.  The default run (`--workload all`)
then measures, in the same process and JSON line under "configs", the
163,840-token verify workload at widths 1-6, the 256-row prefill chunk over
a 122,880-token prefix, and the 262,144-token streamed workload (40 % of the
pages resident, the rest streamed from pinned host memory) at widths 1 and 4
against the host-link ceiling measured in the same run.

Prints one JSON line: throughput (tokens/s = query rows per pass x passes/s),
the roofline of the dominant kernel (the split-KV attention kernel with its
log-sum-exp merge: the quantised K+V bytes a layer must read / the mean
device time per layer, from HIP events on the compute stream around the
timed graph replays; the HBM bytes the counters saw per layer, when the
committed counter summary matches the kernel source), and the fp64 CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload all|decode-40k|verify-160k|stream-256k|prefill-120k]
                       [--width W] [--mode graph|eager] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn tokens/s and quantized-KV GB/s (% of HBM peak) at 40k-256k ctx, 1 GPU"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix, vendor figure
BYTES_PER_TOKEN_HEAD = 208    # Q8_0 K (4 x 34 B) + Q4_0 V (4 x 18 B) per token per KV head
# K/V element-type pairs: name -> (k_type, v_type, label, bytes per token per KV head)
KV_TYPES = {"q8_0-q4_0": (8, 2, "Q8_0 K / Q4_0 V", 208), "q8_0-q8_0": (8, 8, "Q8_0 K / Q8_0 V", 272),
            "q4_0-q4_0": (2, 2, "Q4_0 K / Q4_0 V", 144), "f16-f16": (1, 1, "F16 K / F16 V", 512)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    help="all (default): decode-40k as the headline, then verify-160k W=1-6, prefill-120k and "
                         "stream-256k W=1 and 4 in the same run; or one workload")
    ap.add_argument("--width", type=int, default=0, help="query rows for verify / streamed workloads")
    ap.add_argument("--mode", choices=["graph", "eager"], default=None,
                    help="graph: replay a captured HIP graph of the 64-layer pass (resident workloads); "
                         "eager: one C-ABI call per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (testing only)")
    ap.add_argument("--with-copy-kernel", action="store_true",
                    help="after timing, run a plain elementwise copy of 256 MiB (read 256 MiB, write 256 MiB) "
                         "three times: the reference dispatch for scaling HBM traffic counters")
    ap.add_argument("--writer", action="store_true",
                    help="also time the KV writer: one captured graph of one kvattn_append of the step's rows per "
                         "layer (decode / verify workloads)")
    ap.add_argument("--split-pages", type=int, default=0,
                    help="pages per split for calls of <= 32 rows per KV head (0: the library's choice)")
    ap.add_argument("--chunk-slots", type=int, default=0,
                    help="streamed workloads: ring slots per streamed chunk (0: the library's default, 16)")
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed chunk order inside splits (same bits every call) instead of waves claiming chunks")
    ap.add_argument("--adaptive", action="store_true",
                    help="streamed workloads: afterwards run the adaptive resident/ring policy in closed loop on the "
                         "same device-page budget and time its final split")
    ap.add_argument("--kv-types", choices=sorted(KV_TYPES), default="q8_0-q4_0",
                    help="K/V element-type pair of the cache (default: the workloads' Q8_0 K / Q4_0 V)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only measure the plain-read ceiling of the device for the workload's quantised-KV bytes "
                         "per layer (64 buffers, libkvattn_probe) and print it as JSON")
    ap.add_argument("--h2d-ceiling", action="store_true",
                    help="only measure the host-to-device ceiling (pinned copies) and print it as JSON")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter collections of a --with-copy-kernel run of --workload / "
                         "--width (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE) into "
                         "profiles/traffic_<workload>_w<rows>.txt, the per-layer HBM traffic the roofline reports")
    return ap.parse_args()


# --------------------------------------------------------------------------- setup
def build(w, width, n_layers, torch, kv, inputs, types=KV_TYPES["q8_0-q4_0"], split_pages=0, deterministic=False,
          chunk_slots=0):
    """Create the handle and place every layer's pages.  Returns (handle,
    queries, outputs, call kind, rows, host histories)."""
    dev = "cuda"
    n = w.n_pages
    streamed = w.resident_fraction < 1.0
    rows = width if width else w.widths[-1] if w.prefill_rows else (w.widths[0] if not streamed else 1)
    n_res = w.n_resident if streamed else n
    n_pool = n_layers * n_res
    compute = torch.cuda.Stream()
    copy = torch.cuda.Stream()
    params = kv.make_params(n_layers, w.n_q_heads, w.n_kv_heads, n_pool, n, max(rows, 1),
                            n_ring_slots=w.ring_slots, k_type=types[0], v_type=types[1], split_pages=split_pages,
                            deterministic=int(deterministic), chunk_slots=chunk_slots)
    h = kv.allocate(params, compute_stream=compute, copy_stream=copy)
    pb = kv.page_bytes(params)
    pool = h.pool.view(n_pool, pb)
    perm = np.random.default_rng(inputs.derive_seed(inputs.BASE_SEED, w.wid, 0, inputs.T_PERM)).permutation(n_pool)
    hist = []
    for l in range(n_layers):
        kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, l, w.wid, device=dev, k_type=types[0], v_type=types[1])
        table = np.empty(n, dtype=np.uint32)
        if streamed:
            res = inputs.resident_subset(n, n_res, l, w.wid)
            ids = perm[l * n_res:(l + 1) * n_res]
            table[:] = kv.PT_HOST
            table[res] = ids
            pool[torch.from_numpy(ids).to(dev)] = kvl.pages[torch.from_numpy(res).to(dev)]
            host = torch.empty((n, pb), dtype=torch.uint8, pin_memory=True)
            host.copy_(kvl.pages)
            hist.append(host)
            torch.cuda.synchronize()
            h.set_layer(l, table, w.n_tokens, host)
        else:
            ids = perm[l * n:(l + 1) * n]
            table[:] = ids
            pool[torch.from_numpy(ids.astype(np.int64)).to(dev)] = kvl.pages
            torch.cuda.synchronize()
            h.set_layer(l, table, w.n_tokens)
        del kvl
    qs = [inputs.draw_queries(rows, w.n_q_heads, l, w.wid, device=dev) for l in range(n_layers)]
    outs = [torch.empty_like(q) for q in qs]
    kind = "prefill" if w.prefill_rows else ("decode" if rows == 1 else "verify")
    torch.cuda.synchronize()
    return h, qs, outs, kind, rows, hist


def one_pass(h, qs, outs, kind, rows):
    for l in range(len(qs)):
        if kind == "decode":
            h.decode(l, qs[l], outs[l])
        elif kind == "verify":
            h.verify(l, qs[l], rows, outs[l])
        else:
            h.prefill_chunk(l, qs[l], rows, outs[l])


# --------------------------------------------------------------------------- traffic
def measured_traffic(workload, rows, field="traffic_bytes_per_layer"):
    """HBM bytes per layer call (split + merge kernels) from the committed
    FETCH_SIZE / WRITE_SIZE counter summary of this workload, if it was taken
    on the current kernel sources (the record names them and their hash;
    else None).  Streamed workloads: `field` picks the host-link bytes the
    ring copies read per layer call."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_w{rows}.txt")
    csrc = os.path.join(ROOT, "long_context_attention_amd", "csrc")
    try:
        with open(path) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for name in rec.get("kernel_sources", []):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
    except (OSError, ValueError, TypeError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get(field)


TRAFFIC_SOURCES = ["kernels_common.h", "split_kernel.hip", "wide_kernel.hip"]
STREAM_TRAFFIC_SOURCES = TRAFFIC_SOURCES + ["copy_kernels.hip"]


def traffic_record(fetch_csv, write_csv, workload, rows, cmd_fetch, cmd_write):
    """Per-dispatch means of FETCH_SIZE / WRITE_SIZE (KiB) for the attention
    kernel (split or wide) and the merge of each layer call, each scaled by
    the same counter's reading for the reference copy (torch.neg over 256 MiB:
    reads 256 MiB, writes 256 MiB) in the same run; the record names the kernel
    sources and their hash, and the roofline uses it only while they match."""
    import csv
    import hashlib

    def means(path, counter):
        acc = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"]
                kind = ("attention" if ("split_kernel" in k or "wide_kernel" in k) else
                        "merge" if "merge" in k else "copy_ref" if "neg_kernel" in k else
                        "ring_copy" if "ring_copy" in k else None)
                if kind:
                    acc.setdefault(kind, []).append(float(r["Counter_Value"]))
        return ({k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()},
                {k: sum(v) for k, v in acc.items()})

    f, nf, fsum = means(fetch_csv, "FETCH_SIZE")
    w, _, wsum = means(write_csv, "WRITE_SIZE")
    ref_kib = 256 * 1024
    fs, ws = ref_kib / f["copy_ref"], ref_kib / w["copy_ref"]
    import inputs
    wl = inputs.WORKLOADS[workload]
    streamed = wl.resident_fraction < 1.0
    sources = STREAM_TRAFFIC_SOURCES if streamed else TRAFFIC_SOURCES
    extra = {}
    if streamed:
        # several attention launches per layer call (resident pages, then one
        # per streamed chunk) and ring copies ahead of them: totals over the
        # run divided by the layer calls (one merge each)
        calls = nf["merge"]
        att = (fsum["attention"] * fs + wsum["attention"] * ws) * 1024 / calls
        mer = (fsum["merge"] * fs + wsum["merge"] * ws) * 1024 / calls
        rc_f = fsum.get("ring_copy", 0.0) * fs * 1024 / calls
        rc_w = wsum.get("ring_copy", 0.0) * ws * 1024 / calls
        h2d = (wl.n_pages - wl.n_resident) * 256 * wl.n_kv_heads * BYTES_PER_TOKEN_HEAD
        extra = {"layer_calls": calls, "ring_copy_fetch_bytes_per_layer": round(rc_f),
                 "ring_copy_write_bytes_per_layer": round(rc_w), "h2d_algorithmic_bytes_per_layer": h2d,
                 "note": "ring copies are counted per layer call of the run (the copies of one layer run "
                         "ahead of it); fetch = bytes read over the host link, write = bytes written into "
                         "the ring"}
    else:
        att = (f["attention"] * fs + w["attention"] * ws) * 1024
        mer = (f.get("merge", 0.0) * fs + w.get("merge", 0.0) * ws) * 1024
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_attention_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    rec = {"workload": workload, "rows": rows, "kernels": ["attention (split or wide kernel)", "merge"] +
           (["ring_copy"] if streamed else []),
            "kernel_sources": sources, "kernel_source_sha256": h.hexdigest(),
            "dispatches": nf,
            "fetch_size_kib": {k: round(v, 1) for k, v in f.items()},
            "write_size_kib": {k: round(v, 1) for k, v in w.items()},
            "scale": {"fetch": round(fs, 4), "write": round(ws, 4)},
            "traffic_bytes_per_layer": round(att + mer), "attention_bytes": round(att), "merge_bytes": round(mer),
            "algorithmic_bytes_per_layer": wl.n_tokens * wl.n_kv_heads * BYTES_PER_TOKEN_HEAD,
            "commands": {"fetch": cmd_fetch, "write": cmd_write},
            "method": "FETCH_SIZE and WRITE_SIZE in KiB per dispatch, averaged over the attention and merge "
                      "dispatches of the eager passes; each scaled by the reading of the same counter for "
                      "torch.neg over a 256 MiB float32 tensor (reads 256 MiB, writes 256 MiB) run three times in "
                      "the same process: fetch scale = 262144 / fetch_kib(copy), write scale = 262144 / "
                      "write_kib(copy).  The record holds for kernel sources whose concatenated sha256 matches."}
    rec.update(extra)
    return rec


# --------------------------------------------------------------------------- KV writer
def time_writer(h, w, rows, n_layers, steps, torch, inputs, stream, bytes_per_token_head=BYTES_PER_TOKEN_HEAD):
    """Each layer's history is shortened by two steps' rows, then one pass of
    kvattn_append (the step's rows, one call per layer) warms up and one is
    captured; replays of the captured pass rewrite the same positions, the
    same work as a real step's writer.  Returns microseconds per call."""
    g = torch.Generator(device="cuda").manual_seed(inputs.derive_seed(inputs.BASE_SEED, w.wid, 0, 99))
    ks = [torch.randn(rows, w.n_kv_heads, 128, device="cuda", generator=g) for _ in range(n_layers)]
    vs = [torch.randn(rows, w.n_kv_heads, 128, device="cuda", generator=g) for _ in range(n_layers)]
    for l in range(n_layers):
        table = np.asarray(h.layer_table(l), dtype=np.uint32)
        h.set_layer(l, table, w.n_tokens - 2 * rows)
    with torch.cuda.stream(stream):
        for l in range(n_layers):
            h.append(l, ks[l], vs[l], rows)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for l in range(n_layers):
            h.append(l, ks[l], vs[l], rows)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * n_layers)
    bytes_per_call = rows * w.n_kv_heads * bytes_per_token_head
    return {"us_per_call": round(us, 3), "rows_per_call": rows,
            "quantised_bytes_per_call": bytes_per_call,
            "timing": "HIP events around replays of a captured pass of one append per layer"}


# --------------------------------------------------------------------------- host link
def h2d_ceiling(torch, mb=436, reps=3):
    """Host-to-device copy rates: one large pinned copy (the ceiling) and
    page-sized pieces (425,984 B) into 64 rotating slots."""
    n = mb * 1024 * 1024
    page = 425984
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    host[::4096] = 1
    dev = torch.empty(n, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    with torch.cuda.stream(stream):
        for _ in range(reps):
            e0.record(stream)
            dev.copy_(host, non_blocking=True)
            e1.record(stream)
            e1.synchronize()
            best = max(best, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        pieces = n // page
        e0.record(stream)
        for i in range(pieces):
            dev[(i % 64) * page:(i % 64 + 1) * page].copy_(host[i * page:(i + 1) * page], non_blocking=True)
        e1.record(stream)
        e1.synchronize()
        piece_rate = pieces * page / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"contiguous_gbps": round(best, 2), "page_pieces_gbps": round(piece_rate, 2), "bytes": n}


def hbm_read_ceiling(bytes_per_launch, n_buffers=64, reps=5):
    """Plain-read ceiling for one launch reading `bytes_per_launch` (rounded
    up to 16 B) from one of n_buffers distinct device buffers in turn:
    microseconds per launch and GB/s for each load policy and grid size of
    kvattn_probe_read_ceiling (libkvattn_probe.so, a measurement helper
    beside the attention library)."""
    import ctypes
    from long_context_attention_amd import build as hipbuild
    if not os.path.exists(hipbuild.PROBE_LIB):
        raise RuntimeError(f"{hipbuild.PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(hipbuild.PROBE_LIB)
    lib.kvattn_probe_read_ceiling.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.kvattn_probe_read_ceiling.restype = ctypes.c_int
    nbytes = -(-int(bytes_per_launch) // 16) * 16
    us = (ctypes.c_double * 8)()
    best = ctypes.c_double(0.0)
    rc = lib.kvattn_probe_read_ceiling(nbytes, n_buffers, reps, us, ctypes.byref(best))
    if rc != 0:
        raise RuntimeError(f"kvattn_probe_read_ceiling returned {rc}")
    grids = [256, 512, 1024, 2048]
    table = {pol: {str(g): {"us": round(us[i * 4 + j], 3), "gbps": round(nbytes / us[i * 4 + j] / 1e3, 1)}
                   for j, g in enumerate(grids)} for i, pol in enumerate(["default", "nontemporal"])}
    return {"bytes_per_launch": nbytes, "buffers": n_buffers, "reps": reps, "best_gbps": round(best.value, 1),
            "best_frac_hbm_peak": round(best.value / HBM_PEAK_GBPS, 4), "by_policy_and_grid": table,
            "kernel": "workgroup-contiguous slices, 512 threads, eight 16-byte loads in flight per thread"}


# --------------------------------------------------------------------------- adaptive partition
def adaptive_run(h, w, hist, qs, outs, kind, rows, n_layers, steps, torch, kv, max_iters=8):
    """Closed loop of kvattn_policy_step on the streamed workload: the device
    budget is the fixed split's pool plus a minimal ring; each iteration runs
    one observed pass, steps the policy and applies a changed decision
    (resident pages re-placed from the pinned histories, ring resized).
    Returns the trajectory and the final split's pass time."""
    dev = "cuda"
    n = w.n_pages
    pb = kv.page_bytes(h.params)
    n_pool_alloc = n_layers * w.n_resident
    pool = h.pool.view(n_pool_alloc, pb)
    min_ring = 32
    c = kv.policy_config(n_layers, 256, n_pool_alloc + min_ring, min_ring_slots=min_ring,
                         max_ring_slots=w.ring_slots, ring_step=16, grow_after=1, shrink_after=2, busy_high=0.85)

    def apply(res, ring):
        h.set_ring_slots(ring)
        nxt = 0
        for l in range(n_layers):
            r = int(res[l])
            table = np.full(n, kv.PT_HOST, dtype=np.uint32)
            ids = np.arange(nxt, nxt + r, dtype=np.int64)
            table[n - r:] = ids
            if r:
                pool[torch.from_numpy(ids).to(dev)] = hist[l][n - r:].to(dev)
            torch.cuda.synchronize()
            h.set_layer(l, table, w.n_tokens, hist[l])
            nxt += r
        return nxt

    o = kv.PolicyObservation()
    o.n_tokens = w.n_tokens
    st, d, res = kv.policy_step(c, kv.PolicyState(), o)
    apply(res, d.ring_slots)
    traj = [{"reason": int(d.reason), "ring_slots": int(d.ring_slots), "streamed_layers": int(d.streamed_layers),
             "streamed_pages": int(d.streamed_pages)}]
    stream = h.compute_stream
    holds = 0
    for it in range(max_iters):
        with torch.cuda.stream(stream):
            one_pass(h, qs, outs, kind, rows)
        torch.cuda.synchronize()
        h.observe(1 << 14)
        with torch.cuda.stream(stream):
            one_pass(h, qs, outs, kind, rows)
        ob = h.observe_read(w.n_tokens)
        h.observe(0)
        st, d, res = kv.policy_step(c, st, ob)
        traj.append({"chunks": int(ob.chunks), "misses": int(ob.ready_misses),
                     "occupancy": round(float(ob.ring_occupancy), 3), "copy_busy": round(float(ob.copy_busy), 3),
                     "reason": int(d.reason), "ring_slots": int(d.ring_slots),
                     "streamed_layers": int(d.streamed_layers), "streamed_pages": int(d.streamed_pages)})
        log(f"bench: adaptive iteration {it}: {traj[-1]}")
        if d.changed:
            apply(res, d.ring_slots)
            holds = 0
        else:
            holds += 1
            if holds >= 2:
                break
    with torch.cuda.stream(stream):
        one_pass(h, qs, outs, kind, rows)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            one_pass(h, qs, outs, kind, rows)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"budget_pages": int(c.budget_pages), "trajectory": traj, "final_ring_slots": int(d.ring_slots),
            "final_streamed_layers": int(d.streamed_layers), "ms_per_step": round(ms, 3),
            "tokens_per_s": round(rows / (ms / 1e3), 3),
            "h2d_gbps": round(d.streamed_pages * pb / (ms / 1e3) / 1e9, 2)}


# --------------------------------------------------------------------------- machine
def _sysfs_clock(dev_dir, name):
    """Current level of a pp_dpm_* table ("<i>: <f>Mhz *" marks it), in MHz."""
    try:
        with open(os.path.join(dev_dir, name)) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return line.split(":", 1)[1].strip().rstrip("*").strip().lower().replace("mhz", "").strip()
    except OSError:
        pass
    return None


def gpu_info(torch):
    """Device name and CU count, plus the current shader and memory clocks read
    from the device's sysfs tables (pp_dpm_sclk / pp_dpm_mclk; absent when
    they are not readable).  No child process is started."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": props.multi_processor_count}
    dirs = []
    bus = getattr(props, "pci_bus_id", None)
    if bus is not None:
        dom, dev = getattr(props, "pci_domain_id", 0), getattr(props, "pci_device_id", 0)
        dirs.append(f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{dev:02x}.0")
    try:
        cards = sorted(d for d in os.listdir("/sys/class/drm") if d.startswith("card") and "-" not in d)
        found = [f"/sys/class/drm/{c}/device" for c in cards if os.path.exists(f"/sys/class/drm/{c}/device/pp_dpm_sclk")]
        if len(found) == 1:
            dirs.append(found[0])
    except OSError:
        pass
    for d in dirs:
        sclk, mclk = _sysfs_clock(d, "pp_dpm_sclk"), _sysfs_clock(d, "pp_dpm_mclk")
        if sclk or mclk:
            info.update({k: v for k, v in (("sclk_mhz", sclk), ("mclk_mhz", mclk)) if v})
            info["clock_source"] = os.path.join(d, "pp_dpm_*")
            break
    return info


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------------------- cpu baseline
def cpu_baseline(w, rows, kind, inputs, budget_s=10.0, types=KV_TYPES["q8_0-q4_0"], one_core=True):
    """The oracle (fp64 C, OpenMP over (row, head)) on a bounded sample of the
    same workload: whole layers (a seeded sample of rows for prefill) until
    about budget_s seconds of CPU work, scaled to tokens/s of the full
    64-layer pass."""
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    if kind == "prefill":
        # a sample of rows: first, last and 6 seeded others
        rng = np.random.default_rng(7)
        sample_rows = sorted({0, rows - 1, *rng.choice(rows, 6, replace=False).tolist()})
    else:
        sample_rows = list(range(rows))
    spent, layers = 0.0, 0
    while layers < w.n_layers and spent < budget_s:
        kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, layers, w.wid, device="cuda", k_type=types[0],
                                v_type=types[1])
        pages = kvl.pages.cpu().numpy()
        q = inputs.draw_queries(rows, w.n_q_heads, layers, w.wid, device="cuda").cpu().numpy()
        del kvl
        t0 = time.perf_counter()
        oracle.attend_paged(np.arange(pages.shape[0], dtype=np.uint32), w.n_tokens, 256, w.n_q_heads,
                            w.n_kv_heads, q, inputs.scale_for(), pool=pages, rows=sample_rows, n_threads=threads,
                            k_type=types[0], v_type=types[1])
        spent += time.perf_counter() - t0
        layers += 1
    # full pass = n_layers layers x rows rows; sample = `layers` layers x len(sample_rows) rows
    pass_s = spent * (w.n_layers / layers) * rows / len(sample_rows)
    out = {"value": rows / pass_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu": {"model": cpu_model(), "logical_cpus": os.cpu_count()},
           "sample": f"{layers} of {w.n_layers} layers of {w.name} ({w.n_tokens} keys, {w.n_q_heads} query heads, "
                     f"{len(sample_rows)} of {rows} rows), {spent:.1f} s measured, scaled to the full pass"}
    if not one_core:
        return out
    # one core: the first sampled row of one layer (the oracle is linear in rows and layers)
    kvl = inputs.draw_layer(w.n_tokens, w.n_kv_heads, 0, w.wid, device="cuda", k_type=types[0], v_type=types[1])
    pages = kvl.pages.cpu().numpy()
    q = inputs.draw_queries(rows, w.n_q_heads, 0, w.wid, device="cuda").cpu().numpy()
    del kvl
    t0 = time.perf_counter()
    oracle.attend_paged(np.arange(pages.shape[0], dtype=np.uint32), w.n_tokens, 256, w.n_q_heads, w.n_kv_heads, q,
                        inputs.scale_for(), pool=pages, rows=sample_rows[:1], n_threads=1, k_type=types[0],
                        v_type=types[1])
    one = time.perf_counter() - t0
    one_pass_s = one * w.n_layers * rows
    out["one_core"] = {"value": rows / one_pass_s, "unit": "tokens/s",
                       "sample": f"1 row of 1 layer, {one:.2f} s measured, scaled to the full pass"}
    return out


# --------------------------------------------------------------------------- timing
def time_workload(h, qs, outs, kind, rows, w, n_layers, mode, steps, warmup, torch, streamed):
    """Warm up, then time `steps` passes (HIP events on the compute stream
    around them), then the same steps again with an event between steps for
    the spread.  Returns (ms per pass, wall s, per-layer kernel ms, kernel
    timing description, per-launch split / merge figures, step spread)."""
    stream = h.compute_stream
    graph = None
    if mode == "graph":
        with torch.cuda.stream(stream):
            one_pass(h, qs, outs, kind, rows)  # warm the code paths before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            one_pass(h, qs, outs, kind, rows)
        torch.cuda.synchronize()

    def step():
        if graph is not None:
            graph.replay()
        else:
            one_pass(h, qs, outs, kind, rows)

    with torch.cuda.stream(stream):
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    chunks = -(-(w.n_pages - w.n_resident) // 16) if streamed else 0
    if graph is None:
        h.profile(max(1, steps) * n_layers * (2 * chunks + 40))
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        t_start = time.perf_counter()
        for _ in range(steps):
            step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    elapsed_ms = e0.elapsed_time(e1)
    per_launch = None
    if graph is None:
        timing = "per-launch HIP events on the compute stream during the timed steps"
        split_ms, n_split, merge_ms, n_merge = h.profile_read(reset=True)
        h.profile(0)
        layer_ms = split_ms + merge_ms
        if n_split:
            per_launch = {"split_mean": round(split_ms / n_split, 5), "split_launches": n_split,
                          "merge_mean": round(merge_ms / max(n_merge, 1), 5), "merge_launches": n_merge}
    else:
        # a resident layer is the attention kernel then its merge kernel, back
        # to back in the graph; HIP events around the timed replays give their
        # mean per layer (gaps included)
        timing = ("HIP events on the compute stream around the timed graph replays, per layer "
                  "(attention kernel + merge kernel)")
        layer_ms = elapsed_ms
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with torch.cuda.stream(stream):
        marks[0].record(stream)
        for i in range(steps):
            step()
            marks[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    spread = {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
              "p90": round(float(np.percentile(step_ms, 90)), 4),
              "how": "a second run of the same steps with an event between steps"}
    return elapsed_ms / steps, wall, layer_ms / (steps * n_layers), timing, per_launch, spread


def figures(w, rows, kind, n_layers, ms_per_step, layer_ms, types, streamed, ceiling=None):
    """Throughput and the roofline of the dominant kernel for one measured
    workload and width."""
    value = rows / (ms_per_step / 1e3)
    kv_bytes_layer = w.n_tokens * w.n_kv_heads * types[3]   # every key of the history, read once per layer
    flops_layer = 4.0 * w.n_q_heads * 128 * sum(w.n_tokens - rows + r + 1 for r in range(rows))
    kv_gbps = kv_bytes_layer * n_layers / (ms_per_step / 1e3) / 1e9
    out = {"value": round(value, 3), "unit": "tokens/s", "ms_per_step": round(ms_per_step, 4),
           "layers_per_s": round(n_layers / (ms_per_step / 1e3), 1), "kv_gbps": round(kv_gbps, 1),
           "kv_frac_hbm_peak": round(kv_gbps / HBM_PEAK_GBPS, 4),
           "algorithmic": {"kv_bytes_per_layer": kv_bytes_layer, "flops_per_layer": flops_layer}}
    default_types = types[0] == 8 and types[1] == 2
    if streamed:
        n_str = w.n_pages - w.n_resident
        h2d = n_str * 256 * w.n_kv_heads * types[3] * n_layers / (ms_per_step / 1e3) / 1e9
        out["h2d_gbps"] = round(h2d, 2)
        c = ceiling["contiguous_gbps"]
        # the pass is bound by the host link: streamed bytes against the measured ceiling
        # traffic: the bytes the ring copies read over the host link per pass,
        # from the committed counter record when it matches the sources
        rc = measured_traffic(w.name, rows, "ring_copy_fetch_bytes_per_layer") if default_types else None
        out["roofline"] = {"bound": "host-link", "achieved": out["h2d_gbps"], "peak": c, "unit": "GB/s",
                           "frac": round(out["h2d_gbps"] / c, 4),
                           "traffic": round(rc * n_layers) if rc is not None else None}
        att = measured_traffic(w.name, rows) if default_types else None
        if att is not None:
            out["hbm_traffic_bytes_per_layer"] = att
        return out
    achieved = kv_bytes_layer / (layer_ms / 1e3) / 1e9
    tflops = flops_layer / (layer_ms / 1e3) / 1e12
    traffic = measured_traffic(w.name, rows) if default_types else None
    if kind == "prefill":
        out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic}
        out["kv_gbps_kernels"] = round(achieved, 1)
    else:
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
        # the contraction runs on the matrix cores at every width: its rate
        out["mfma_tflops"] = round(tflops, 2)
        out["mfma_frac"] = round(tflops / MFMA_F16_PEAK_TFLOPS, 4)
    return out


def measure(w, widths, args, torch, kv, inputs, types, steps, warmup, cpu_budget, ceiling=None, extras=False):
    """Build one workload, then time it at each width (sharing the pages);
    returns {width: result}."""
    n_layers = args.layers or w.n_layers
    streamed = w.resident_fraction < 1.0
    mode = args.mode or ("eager" if streamed else "graph")
    if streamed and mode == "graph":
        raise SystemExit("streamed workloads run eagerly (the copy stream is driven by the host)")
    log(f"bench: workload {w.name}, {n_layers} layers, mode {mode}, widths {widths}: building inputs")
    t0 = time.perf_counter()
    h, qs, outs, kind, rows, hist = build(w, max(widths), n_layers, torch, kv, inputs, types, args.split_pages,
                                          args.deterministic, args.chunk_slots)
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    results = {}
    for W in widths:
        if W != rows:
            qs = [inputs.draw_queries(W, w.n_q_heads, l, w.wid, device="cuda") for l in range(n_layers)]
            outs = [torch.empty_like(q) for q in qs]
            rows = W
        k = "prefill" if kind == "prefill" else ("decode" if W == 1 else "verify")
        log(f"bench: {w.name} {k} rows={W}: warmup {warmup}, timing {steps} steps")
        ms, wall, layer_ms, timing, per_launch, spread = time_workload(h, qs, outs, k, W, w, n_layers, mode, steps,
                                                                       warmup, torch, streamed)
        r = figures(w, W, k, n_layers, ms, layer_ms, types, streamed, ceiling)
        r["config"] = {"workload": w.name, "layers": n_layers, "context": w.n_tokens, "page_tokens": 256,
                       "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": 128, "rows": W,
                       "kv_types": types[2], "mode": mode, "split_pages": args.split_pages or "auto",
                       "chunk_order": "static" if args.deterministic else
                       "claimed in splits of >= 96 chunks, else static",
                       "resident_fraction": w.resident_fraction, "ring_slots": w.ring_slots,
                       "chunk_slots": (args.chunk_slots or max(1, w.ring_slots * 3 // 8)) if streamed else None}
        r["steps"], r["warmup"], r["wall_s"], r["step_ms_spread"] = steps, warmup, round(wall, 3), spread
        if not streamed:
            r["kernel_ms"] = {"layer_mean": round(layer_ms, 5), "timing": timing}
            if per_launch:
                r["kernel_ms"].update(per_launch)
        if extras and args.adaptive and streamed:
            r["adaptive"] = adaptive_run(h, w, hist, qs, outs, k, W, n_layers, max(2, min(steps, 5)), torch, kv)
        if extras and args.writer and k != "prefill" and not streamed:
            r["writer"] = time_writer(h, w, W, n_layers, steps, torch, inputs, h.compute_stream, types[3])
        if cpu_budget > 0:
            log(f"bench: timing the oracle on a CPU sample ({w.name}, rows={W})")
            r["cpu_baseline"] = cpu_baseline(w, W, k, inputs, budget_s=cpu_budget, types=types, one_core=extras)
        results[W] = r
    h.destroy()
    del h, qs, outs, hist
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return results


# --------------------------------------------------------------------------- main
CONTRACT_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                 "vs_baseline", "dtype", "data", "config")


def main():
    args = parse()
    if args.traffic_record:
        wl = "decode-40k" if args.workload == "all" else args.workload
        import inputs
        w = inputs.WORKLOADS[wl]
        rows = args.width or (w.prefill_rows or w.widths[0])
        base = (f"python -u <repo>/bench.py --workload {wl} --width {rows} --mode eager --steps 2 --warmup 1 "
                "--no-cpu-baseline --with-copy-kernel" + (f" --layers {args.layers}" if args.layers else ""))
        cmd = "cd /tmp && timeout -s KILL 300 rocprofv3 --pmc {c} -f csv -d <out>/{d} -o {d} -- " + base
        rec = traffic_record(args.traffic_record[0], args.traffic_record[1], wl, rows,
                             cmd.format(c="FETCH_SIZE", d="fetch"), cmd.format(c="WRITE_SIZE", d="write"))
        path = os.path.join(ROOT, "profiles", f"traffic_{wl}_w{rows}.txt")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps({"traffic_record": path, "traffic_bytes_per_layer": rec["traffic_bytes_per_layer"],
                          "algorithmic_bytes_per_layer": rec["algorithmic_bytes_per_layer"]}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU mode (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import inputs
    import long_context_attention_amd as kv
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.h2d_ceiling:
        print(json.dumps({"h2d_ceiling": h2d_ceiling(torch)}), flush=True)
        return
    types = KV_TYPES[args.kv_types]
    every = args.workload == "all"
    w = inputs.WORKLOADS["decode-40k" if every else args.workload]
    if args.hbm_ceiling:
        layer_bytes = w.n_tokens * w.n_kv_heads * types[3]
        print(json.dumps({"workload": w.name, "hbm_read_ceiling": hbm_read_ceiling(layer_bytes)}), flush=True)
        return
    budget = 0.0 if args.no_cpu_baseline else 10.0
    streamed = w.resident_fraction < 1.0
    ceiling = h2d_ceiling(torch) if streamed else None
    width = args.width or (w.widths[-1] if w.prefill_rows else (w.widths[0] if not streamed else 1))
    head = measure(w, [width], args, torch, kv, inputs, types, args.steps, args.warmup, budget, ceiling,
                   extras=True)[width]
    result = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "f16", "data": "synthetic", "config": head["config"],
              "gpu": gpu_info(torch)}
    result.update({k: v for k, v in head.items() if k not in CONTRACT_KEYS})
    if ceiling is not None:
        result["h2d_ceiling"] = ceiling
    if every:
        # the other workloads of the same metric, each at its widths, in the
        # same run: their own throughput, roofline and oracle baseline
        # (smaller CPU samples)
        configs = {}
        cb = 0.0 if args.no_cpu_baseline else 3.0
        for W, r in measure(inputs.WORKLOADS["verify-160k"], [1, 2, 3, 4, 5, 6], args, torch, kv, inputs, types,
                            args.steps, args.warmup, cb).items():
            configs[f"verify-160k W={W}"] = r
        pf = inputs.WORKLOADS["prefill-120k"]
        for W, r in measure(pf, [pf.prefill_rows], args, torch, kv, inputs, types, args.steps, args.warmup,
                            cb).items():
            configs[f"prefill-120k R={W}"] = r
        sw = inputs.WORKLOADS["stream-256k"]
        ceil = h2d_ceiling(torch)
        result["h2d_ceiling"] = ceil
        s_steps = max(1, min(args.steps, 3))
        for W, r in measure(sw, [1, 4], args, torch, kv, inputs, types, s_steps, 1, cb, ceil).items():
            configs[f"stream-256k W={W}"] = r
        result["configs"] = configs
    if args.with_copy_kernel:
        a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        result["copy_kernel_bytes"] = {"read": a.numel() * 4, "write": b.numel() * 4}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
