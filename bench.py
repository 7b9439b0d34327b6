#!/usr/bin/env python3
"""Benchmark of quantized-KV attention (K Q8_0, V Q4_0, 256-token pages) on one
MI355X.

Default workload: a 16-layer stack of full-attention layers, 24 query heads /
4 KV heads x head_dim 256, 262,144 cached tokens per layer (436,207,616 bytes
of quantized KV per layer, 6.98 GB for the stack).  One step = for every
layer, the decode step kvq_append_attn: the new token's K/V row (position
262,143) is quantized into the cache and one query attends over all 262,144
tokens (split over pages, merged by online log-sum-exp) -- two kernels per
layer; --unfused runs kvq_append and then the attention call instead.  Each
layer has its own pool, so consecutive layers never share cache lines and
every step streams the whole 6.98 GB from HBM.

Prints one JSON line: effective KV GB/s (algorithmic bytes / time), us per
layer, the roofline of the decode kernel measured with HIP events on the
launch stream, and the CPU oracle timed on a bounded sample of the same
workload.  Inputs are seeded synthetic N(0,1) fp32 drawn on the device.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def kv_bytes_per_token_layer(n_kv: int, D: int, codec: int = 0) -> int:
    """Algorithmic bytes one token of one layer occupies: per 32-value block a
    34-byte Q8_0 K block and an 18-byte Q4_0 V block; with the INT2 codec per
    128-value block 36 bytes (32 of codes, fp16 scale and zero) for K and V."""
    if codec == 1:
        return n_kv * (D // 128) * 2 * 36
    return n_kv * (D // 32) * (34 + 18)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the launch stream
    around the attention kernel; torch's Event objects cannot be handed over,
    since torch creates their handle only on its own first record)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreate(self.ct.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(self.ct.c_void_p(ev))


def device_normal(shape, seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def outlier_channels(w, layer, device):
    """The outlier channels of a workload that has them (1% of the flattened
    (head, dim) channels of K, V and q, scaled x20 for every token): the same
    seeded choice the oracle-side generators make (synth.outlier_channels), as
    device index tensors; (None, None, None) otherwise."""
    if not w.outliers:
        return None, None, None
    import torch
    import synth
    pick = lambda t, n: torch.from_numpy(synth.outlier_channels((0, w.wid, layer, t), n)).to(device)
    return (pick(synth.K, w.n_kv * w.head_dim), pick(synth.V, w.n_kv * w.head_dim),
            pick(synth.Q, w.n_heads * w.head_dim))


def with_outliers(x, channels, factor=20.0):
    """x [..., H, D] with the given channels of its flattened (H, D) axis
    scaled by factor, in place (no-op without channels)."""
    if channels is not None:
        flat = x.view(x.shape[:-2] + (x.shape[-2] * x.shape[-1],))
        flat[..., channels] *= factor
    return x


class Layer:
    def __init__(self, w, layer, device, shuffle_pages=False, fill_chunk=16384):
        import torch
        import attention_quantized_kv_amd as kvq
        self.kvq = kvq
        self.w = w
        self.L = kvq.Layout(w.n_kv, w.head_dim, w.page_size, w.n_pages, w.codec)
        self.pool = torch.empty(kvq.kvq_pool_bytes(self.L), dtype=torch.uint8, device=device)
        if shuffle_pages:
            perm = torch.randperm(w.n_pages, generator=torch.Generator().manual_seed(1000 + layer))
        else:          # one sequence filled in order: logical page i is physical page i
            perm = torch.arange(w.n_pages)
        self.pt = perm.to(torch.int32).to(device)
        base = (w.wid * 1000 + layer) * 1_000_003
        ch_k, ch_v, ch_q = outlier_channels(w, layer, device)
        for r in range(0, w.cached, fill_chunk):
            n = min(fill_chunk, w.cached - r)
            k = with_outliers(device_normal((n, w.n_kv, w.head_dim), base + 2 * r + 1, device), ch_k)
            v = with_outliers(device_normal((n, w.n_kv, w.head_dim), base + 2 * r + 2, device), ch_v)
            kvq.kvq_append(self.L, self.pool, self.pt, r, k, v)
        self.k_new = with_outliers(device_normal((w.n_new, w.n_kv, w.head_dim), base + 7, device), ch_k)
        self.v_new = with_outliers(device_normal((w.n_new, w.n_kv, w.head_dim), base + 8, device), ch_v)
        self.q = with_outliers(device_normal((w.n_q, w.n_heads, w.head_dim), base + 9, device), ch_q)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.n_q, w.n_heads), dtype=torch.float32, device=device)

    def append(self):
        self.kvq.kvq_append(self.L, self.pool, self.pt, self.w.cached, self.k_new, self.v_new)

    cps = 0

    def decode_step(self, ws, kernel, events=None):
        """kvq_append_attn: append the new rows and attend in one call; `events`
        (begin, end) are recorded around the split pass over the cached keys."""
        self.kvq.kvq_append_attn(self.L, self.pool, self.pt, self.w.cached, self.k_new, self.v_new, self.q,
                                 self.w.scale, self.out, self.lse, ws, kernel=kernel, chunks_per_split=self.cps,
                                 events=events)

    def attend(self, ws, kernel, events=None):
        """kvq_attn_ex with the automatic plan (kernel 0: the same choice as
        kvq_decode_attn / kvq_prefill_attn) or a forced kernel; `events`
        (begin, end) are recorded by the library around the attention kernel
        itself, excluding the split merge."""
        self.kvq.kvq_attn_ex(self.L, self.pool, self.pt, self.w.ctx, self.q, self.w.scale, self.out, self.lse,
                             ws, kernel=kernel, chunks_per_split=self.cps, events=events)


class BatchLayer:
    """One layer of the batched-decode workload: n_seqs sequences of ctx tokens
    in one pool, page p of sequence b at physical page p * n_seqs + b (the
    requests' pages interleaved, as in a serving pool)."""

    def __init__(self, w, layer, device, fill_chunk=16384):
        import torch
        import attention_quantized_kv_amd as kvq
        self.kvq = kvq
        self.w = w
        pages = w.n_pages
        self.L = kvq.Layout(w.n_kv, w.head_dim, w.page_size, pages * w.n_seqs, w.codec)
        self.pool = torch.empty(kvq.kvq_pool_bytes(self.L), dtype=torch.uint8, device=device)
        pt = torch.arange(pages)[None, :] * w.n_seqs + torch.arange(w.n_seqs)[:, None]
        self.pt = pt.to(torch.int32).to(device).contiguous()
        base = (w.wid * 1000 + layer) * 1_000_003
        for b in range(w.n_seqs):
            for r in range(0, w.ctx, fill_chunk):
                n = min(fill_chunk, w.ctx - r)
                k = device_normal((n, w.n_kv, w.head_dim), base + 4 * (b * w.ctx + r) + 1, device)
                v = device_normal((n, w.n_kv, w.head_dim), base + 4 * (b * w.ctx + r) + 2, device)
                kvq.kvq_append(self.L, self.pool, self.pt[b], r, k, v)
        self.q = device_normal((w.n_seqs, w.n_q, w.n_heads, w.head_dim), base + 9, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.n_seqs, w.n_q, w.n_heads), dtype=torch.float32, device=device)
        self.ctx_lens = [w.ctx] * w.n_seqs

    def attend(self, ws, kernel, events=None):
        """kvq_decode_attn_batch over every sequence; `events` (begin, end) are
        recorded around the streaming kernel."""
        self.kvq.kvq_decode_attn_batch(self.L, self.pool, self.pt, self.ctx_lens, self.q, self.w.scale,
                                       self.out, self.lse, ws, events=events)


KERNEL_SOURCES = {"attn_mfma_stream": "attn_mfma_stream.hip", "attn_mfma_tiled": "attn_mfma_tiled.hip",
                  "attn_valu": "attn_valu.hip", "attn_int2": "attn_int2.hip"}


def kernel_name(w, kernel: int) -> str:
    """Name of the attention kernel the plan picks (mirrors the library's
    automatic choice: streaming MFMA for decode / verify with at most 64 query
    rows per KV head, the LDS-tiled MFMA kernel otherwise; over the 2-bit
    cache its streaming kernel up to 16 rows, else the LDS-tiled one)."""
    rows = w.n_q * (w.n_heads // w.n_kv)
    if w.codec == 1:
        return "attn_int2" if (kernel in (0, 4) and w.n_q <= 8 and rows <= 16) else "attn_mfma_tiled"
    if kernel == 0:
        kernel = 2 if (w.n_q <= 8 and rows <= 64) else 3
    return {1: "attn_valu", 2: "attn_mfma_stream", 3: "attn_mfma_tiled"}[kernel]


def kernel_source_files(kname: str):
    """The kernel's .hip file and every local header it includes, directly or
    through another one (`#include "..."` lines), in first-include order."""
    import re
    csrc = os.path.join(ROOT, "attention_quantized_kv_amd", "csrc")
    files, todo = [], [os.path.join(csrc, KERNEL_SOURCES[kname])]
    while todo:
        path = os.path.normpath(todo.pop(0))
        if path in files:
            continue
        files.append(path)
        if os.path.exists(path):
            for m in re.finditer(r'^\s*#\s*include\s+"([^"]+)"', open(path).read(), re.M):
                todo.append(os.path.join(os.path.dirname(path), m.group(1)))
    return files


def source_digest(kname: str):
    """sha256 over the kernel's source files (kernel_source_files, in that
    order); None if one is missing."""
    import hashlib
    h = hashlib.sha256()
    for path in kernel_source_files(kname):
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kname: str):
    """HBM bytes per launch of `kname` on `workload` from the committed
    rocprofv3 counter summary (profiles/hbm_traffic.txt: FETCH_SIZE and
    WRITE_SIZE scaled by the factors a plain copy of known size gives), or
    None when there is no entry or the kernel sources have changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest = source_digest(kname)
    if digest is None:
        return None
    for line in open(path):
        f = line.split()
        if len(f) >= 8 and not line.startswith("#") and f[0] == workload and f[1] == kname:
            if f[2] != digest:
                return None
            return float(f[7])
    return None


def attention_flops(w) -> float:
    """Algorithmic flops of one layer's attention: 2 flops per multiply-add,
    q.k and p.v over every visible key of every query row."""
    pairs = sum(w.ctx - w.n_q + 1 + i for i in range(w.n_q))
    return 4.0 * pairs * w.n_heads * w.head_dim


def cpu_baseline(w, min_seconds: float, max_reps: int = 8):
    """The oracle, as it stands, on one layer of the same workload (host numpy
    inputs), repeated until min_seconds of CPU work."""
    import oracle
    import synth
    k, v = synth.layer_kv(w, 0)
    cache = (oracle.Int2Cache if w.codec == 1 else oracle.QuantCache).from_float(k, v)
    del k, v
    q = synth.layer_q(w, 0)
    if w.n_q <= 8:
        rows = [(i, h) for i in range(w.n_q) for h in range(w.n_heads)]
        desc = f"one {w.ctx}-token layer, all {len(rows)} query rows"
        if w.n_seqs > 1:
            desc = f"one of the {w.n_seqs} sequences of a layer ({w.ctx} tokens), all {len(rows)} query rows"
        bytes_per_rep = w.ctx * kv_bytes_per_token_layer(w.n_kv, w.head_dim, w.codec)
    else:
        rng = __import__("numpy").random.default_rng(0)
        sel = sorted({0, 255, 256, w.n_q - 1, *rng.integers(0, w.n_q, 12).tolist()})
        rows = [(i, h) for i in sel for h in range(w.n_heads)]
        desc = f"{len(sel)} of {w.n_q} query rows x {w.n_heads} heads at full context"
        bytes_per_rep = None
    reps, t_total, threads = 0, 0.0, oracle.max_threads()
    while reps < max_reps and (t_total < min_seconds or reps == 0):
        t0 = time.perf_counter()
        oracle.attention(q, cache, w.scale, rows=rows)
        t_total += time.perf_counter() - t0
        reps += 1
    if bytes_per_rep is not None:
        value = reps * bytes_per_rep / t_total / 1e9
        unit = "GB/s"
    else:
        flops = 4.0 * sum(w.ctx - w.n_q + 1 + i for i, _ in rows) * w.head_dim
        value = reps * flops / t_total / 1e12
        unit = "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{desc}, {reps} repetition(s), {t_total:.1f} s",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (\"unknown\" without it)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_ceiling(device, nbytes=436207616, reps=8):
    """Plain-read bandwidth of this GPU for the decode kernels' access pattern
    (libkvq_probe.so: whole 1 KiB wave requests, 8 waves per workgroup, one
    workgroup per CU), best of 4 and 8 pieces in flight per wave, with and
    without the non-temporal hint, in GB/s;
    the ceiling a streaming kernel can reach here, next to the nominal 8 TB/s.
    None when the probe library is missing."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "attention_quantized_kv_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.kvq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kvq_probe_read.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(device).multi_processor_count
    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    src.fill_(3)
    out = torch.empty(cus * 512, dtype=torch.int32, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for unroll, nt in ((4, 0), (8, 0), (4, 1), (8, 1)):
        call = lambda: lib.kvq_probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                          cus, 8, unroll, nt, stream)
        for _ in range(2):
            if call() != 0:
                raise RuntimeError("kvq_probe_read failed")
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            call()
        stop.record()
        torch.cuda.synchronize()
        best[(unroll, nt)] = nbytes * reps / (start.elapsed_time(stop) / 1e3) / 1e9
    del src, out
    u = max(best, key=best.get)
    return {"GBps": round(best[u], 1), "pieces_in_flight_per_wave": u[0], "nontemporal": bool(u[1]),
            "all": {f"{k[0]}{'nt' if k[1] else ''}": round(v, 1) for k, v in best.items()},
            "probe": f"16 B/lane loads of 1 KiB wave pieces over {nbytes} B, {cus} workgroups x 8 waves, "
                     "plain or non-temporal"}


def bench_stream(args, w, n_layers):
    """Host-resident KV streaming: every layer's cache sits in pinned host
    memory; per step each layer's pages are staged (kvq_stage_pages) into one
    of two device buffers on a copy stream while the previous layer's
    attention runs on the compute stream, ordered by events."""
    import torch
    import attention_quantized_kv_amd as kvq
    dev = torch.device("cuda", 0)
    L = kvq.Layout(w.n_kv, w.head_dim, w.page_size, w.n_pages)
    nbytes = kvq.kvq_pool_bytes(L)
    fill = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    pt_dev = torch.arange(w.n_pages, dtype=torch.int32, device=dev)
    hosts, qs = [], []
    t0 = time.time()
    for layer in range(n_layers):
        base = (w.wid * 1000 + layer) * 1_000_003
        for r in range(0, w.ctx, 16384):
            n = min(16384, w.ctx - r)
            k = device_normal((n, w.n_kv, w.head_dim), base + 2 * r + 1, dev)
            v = device_normal((n, w.n_kv, w.head_dim), base + 2 * r + 2, dev)
            kvq.kvq_append(L, fill, pt_dev, r, k, v)
        h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(fill)
        hosts.append(h)
        qs.append(device_normal((w.n_q, w.n_heads, w.head_dim), base + 9, dev))
    del fill
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: {n_layers} host-resident layers filled in {time.time() - t0:.1f} s",
          file=sys.stderr, flush=True)
    host_table = list(range(w.n_pages))          # the layer's pages, in order: one copy per layer
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.empty((w.n_q, w.n_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.n_q, w.n_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(max(kvq.kvq_workspace_bytes(L, w.n_heads, w.ctx, w.n_q), 256), dtype=torch.uint8, device=dev)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    copied = [torch.cuda.Event(), torch.cuda.Event()]
    used = [torch.cuda.Event(), torch.cuda.Event()]

    def step(ev=None, s=0):
        for e in used:
            e.record(compute)
        with torch.cuda.stream(copy):
            kvq.kvq_stage_pages(L, hosts[0], host_table, L, bufs[0], stream=copy)
            copied[0].record(copy)
        for i in range(n_layers):
            b = i % 2
            if i + 1 < n_layers:
                nb = (i + 1) % 2
                with torch.cuda.stream(copy):
                    copy.wait_event(used[nb])
                    kvq.kvq_stage_pages(L, hosts[i + 1], host_table, L, bufs[nb], stream=copy)
                    copied[nb].record(copy)
            compute.wait_event(copied[b])
            e = ev if (ev is not None and i == s % n_layers) else None
            kvq.kvq_attn_ex(L, bufs[b], pt_dev, w.ctx, qs[i], w.scale, out, lse, ws, events=e)
            used[b].record(compute)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hip_ev = HipEvents()
    evs = [[hip_ev.create() for _ in range(2)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        step(evs[s], s)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    attn_us = 1000.0 * sum(hip_ev.elapsed_ms(e[0], e[1]) for e in evs) / len(evs)
    for e in evs:
        hip_ev.destroy(e[0])
        hip_ev.destroy(e[1])
    # the link's rate for plain pinned copies of the same host buffers, as
    # many as the timed steps make (every layer's, in order, once per step),
    # for reference
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        for h in hosts:
            bufs[0].copy_(h, non_blocking=True)
    stop.record()
    torch.cuda.synchronize()
    copy_gbs = args.steps * len(hosts) * nbytes / (start.elapsed_time(stop) / 1e3) / 1e9
    bytes_layer = w.ctx * kv_bytes_per_token_layer(w.n_kv, w.head_dim, w.codec)
    us_per_layer = 1000.0 * total_ms / args.steps / n_layers
    value = bytes_layer / (us_per_layer / 1e6) / 1e9
    rec = {
        "data": "synthetic", "dtype": "f16 MFMA / f32",
        "config": {"workload": w.name, "layers": n_layers, "n_heads": w.n_heads, "n_kv_heads": w.n_kv,
                   "head_dim": w.head_dim, "ctx": w.ctx, "n_q": w.n_q, "page_size": w.page_size,
                   "kv_format": "K Q8_0 + V Q4_0", "kernel": "auto",
                   "step": "per layer: kvq_stage_pages host -> device (copy stream) overlapped with the "
                           "previous layer's kvq_attn_ex (two device buffers, events)",
                   "kv_home": "pinned host memory"},
        "metric": "host-resident KV streaming decode: KV GB/s over the host link, attention overlapped",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "roofline": {"bound": "hbm", "achieved": round(bytes_layer / (attn_us / 1e6) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(bytes_layer / (attn_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_mfma_stream", "bytes_per_launch": bytes_layer,
                     "avg_launch_us": round(attn_us, 3)},
        "us_per_layer": round(us_per_layer, 3),
        "link": {"streamed_GBps": round(value, 2), "plain_pinned_copy_GBps": round(copy_gbs, 2),
                 "frac_of_plain_copy": round(value / copy_gbs, 4)},
        "kv_bytes_per_layer": bytes_layer,
    }
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode262k",
                    choices=["tiny", "decode65k", "decode262k", "verify131k", "prefill262k", "batch16x16k",
                             "stream262k", "int2decode262k", "int2batch16x16k", "int2prefill262k"])
    ap.add_argument("--layers", type=int, default=None, help="layers in the stack (default: the workload's)")
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA streaming, 3 MFMA tiled")
    ap.add_argument("--cps", type=int, default=0, help="chunks_per_split of kvq_attn_opts: 32-token chunks per wave of a split for the "
                    "streaming kernels, per split for the others (0: the library's choice)")
    ap.add_argument("--unfused", action="store_true",
                    help="decode / verify: kvq_append, then the attention call (three kernels per layer)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shuffle-pages", action="store_true",
                    help="random page table (pages scattered over the pool) instead of in-order pages")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (every layer) in a HIP graph and time its replays; the attention "
                         "kernel is then timed by library events in a separate eager pass")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="only copy a buffer of this many GiB --steps times (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path; "
              "the single-GPU value is the measurement.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_quantized_kv_amd as kvq

    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": args.steps,
                          "GB_per_s_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    n_layers = args.layers or w.layers
    if w.host_resident:
        rec = bench_stream(args, w, n_layers)
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
            rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        print(json.dumps(rec), flush=True)
        return
    prefill = w.n_q > kvq.KVQ_MAX_NQ_DECODE
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    t0 = time.time()
    batched = w.n_seqs > 1
    if batched:
        layers = [BatchLayer(w, i, dev) for i in range(n_layers)]
    else:
        layers = [Layer(w, i, dev, shuffle_pages=args.shuffle_pages) for i in range(n_layers)]
    Layer.cps = args.cps
    # decode and verify run the fused step kvq_append_attn (over both codecs)
    fused = not prefill and not args.unfused and not batched
    if batched:
        ws_n = kvq.kvq_decode_attn_batch_workspace_bytes(layers[0].L, layers[0].ctx_lens, w.n_heads, w.n_q)
    elif fused:
        ws_n = kvq.kvq_append_attn_workspace_bytes(layers[0].L, w.n_heads, w.cached, w.n_q, args.kernel, args.cps)
    else:
        ws_n = kvq.kvq_workspace_bytes_ex(layers[0].L, w.n_heads, w.ctx, w.n_q, args.kernel, args.cps)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: {n_layers} layers filled in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    # The attention kernel is timed by events the library records around it,
    # on one layer per step (rotating through the layers): a pair of event
    # records between kernels costs about 5 us of queue time, which on every
    # layer would inflate the step time being measured.
    def step(ev=None, s=0):
        for i, lay in enumerate(layers):
            e = ev if (ev is not None and i == s % n_layers) else None
            if batched:
                lay.attend(ws, args.kernel, e)
            elif fused:
                lay.decode_step(ws, args.kernel, e)
            else:
                lay.append()
                lay.attend(ws, args.kernel, e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip_ev = HipEvents()
    evs = [[hip_ev.create() for _ in range(2)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(evs[s], s)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    if args.graph:
        # the step's launches recorded once, replayed as one graph per step
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        eager_ms = total_ms
        total_ms = start.elapsed_time(stop)
    attn_ms = [hip_ev.elapsed_ms(e[0], e[1]) for e in evs]
    for e in evs:
        hip_ev.destroy(e[0])
        hip_ev.destroy(e[1])
    avg_attn_us = 1000.0 * sum(attn_ms) / len(attn_ms)       # the attention kernel alone
    kname = kernel_name(w, args.kernel)
    traffic = measured_traffic(w.name, kname)

    ms_per_step = total_ms / args.steps
    bytes_layer = w.n_seqs * w.ctx * kv_bytes_per_token_layer(w.n_kv, w.head_dim, w.codec)
    # bytes the timed kernel reads: the fused step's split pass reads the cached keys only
    bytes_kernel = w.n_seqs * (w.cached if fused else w.ctx) * kv_bytes_per_token_layer(w.n_kv, w.head_dim, w.codec)
    us_per_layer = 1000.0 * ms_per_step / n_layers
    flops_layer = attention_flops(w)
    rec = {
        "data": "synthetic",
        "dtype": "f16 MFMA / f32" if args.kernel in (0, 2, 3) else "f32",
        "config": {"workload": w.name, "layers": n_layers, **({"n_seqs": w.n_seqs} if batched else {}), "n_heads": w.n_heads, "n_kv_heads": w.n_kv,
                   "head_dim": w.head_dim, "ctx": w.ctx, "n_q": w.n_q, "page_size": w.page_size,
                   "kv_format": ("K INT2 + V INT2 (128-value blocks, fp16 scale and zero)" if w.codec == 1
                                 else "K Q8_0 + V Q4_0"), "kernel": args.kernel or "auto",
                   "chunks_per_split": args.cps or "auto",
                   "step": ("kvq_append_attn (append + attention, 2 kernels)" if fused else
                            f"kvq_decode_attn_batch over {w.n_seqs} sequences (2 kernels; cache filled beforehand)"
                            if batched else "kvq_append, then attention" if not prefill else "attention"),
                   "page_table": ("interleaved: page p of sequence b at p * n_seqs + b" if batched else
                                  "shuffled" if args.shuffle_pages else "in order"),
                   "launch": "hipGraph replay of the step" if args.graph else "eager"},
    }
    if not prefill:
        value = n_layers * bytes_layer * args.steps / (total_ms / 1e3) / 1e9
        achieved = bytes_kernel / (avg_attn_us / 1e6) / 1e9
        rec.update({
            "metric": ("quantized-KV batched decode attention: effective KV GB/s (% HBM peak)" if batched else
                       "quantized-KV decode attention: effective KV GB/s (% HBM peak), us/layer @262k"),
            "value": round(value, 2), "unit": "GB/s",
        })
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": kname, "bytes_per_launch": bytes_kernel,
                "avg_launch_us": round(avg_attn_us, 3)}
        extra = {"us_per_layer": round(us_per_layer, 3), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                 "ctx_tokens_per_s": round(w.ctx / (us_per_layer / 1e6), 1),
                 "kv_bytes_per_layer": bytes_layer}
    else:
        value = flops_layer * n_layers * args.steps / (total_ms / 1e3) / 1e12
        achieved = flops_layer / (avg_attn_us / 1e6) / 1e12
        rec.update({"metric": "quantized-KV chunked prefill attention: TFLOP/s (MFMA utilisation)",
                    "value": round(value, 2), "unit": "TFLOP/s"})
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": kname, "flops_per_launch": flops_layer,
                "avg_launch_us": round(avg_attn_us, 3)}
        extra = {"us_per_layer": round(us_per_layer, 3), "flops_per_layer": flops_layer}

    rec.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None})
    if not prefill:
        ceil = read_ceiling(dev)
        if ceil is not None:
            rec["read_ceiling"] = ceil
            rec["pct_read_ceiling"] = round(100 * value / ceil["GBps"], 2)
            roof["frac_of_read_ceiling"] = round(achieved / ceil["GBps"], 4)
    rec["roofline"] = roof
    rec.update(extra)
    if args.graph:
        rec["eager_us_per_layer"] = round(1000.0 * eager_ms / args.steps / n_layers, 3)
    del layers
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, max_reps=8 * w.n_seqs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
