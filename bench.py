"""Benchmark of the TurboQuant decode hot path on one MI355X.

One step = one pass of the whole path over one batch of the workload: the
step's new token of every sequence is compressed into the cache (K and V, every
KV head of every layer) and decode attention runs for every query head of
every layer over the whole cache.

Headline workload (config.workload, the largest single-GPU configuration):
  w3  dense 28-layer shape in the asymmetric mode, 4 KV heads, 28 query heads
      (GQA 7), head_dim 128, batch 1, 32,768 cached tokens; layers 0, 1, 26,
      27 keep K and V in fp16, layers 2..25 keep K in fp16 and V at 4 bits
      (MSE-only).  A step is one tq_decode_step call per storage format (the
      4 fp16 layers, the 24 fp16-K / 4-bit-V layers): 1.29 GB of cache read.
Reported beside it in the same line, each with its own roofline:
  w4  one layer, 8 KV heads, 64 query heads, 262,144 tokens, K 3 bits (2
      Lloyd-Max + 1 QJL), V 2 bits; with multi-query scores of 64 query rows
      per KV head over the same cache (tq_score_multi against tq_score);
  w5  16 sequences of ragged length (4,096..32,768), 8 KV heads, 64 query
      heads, K 4 bits, V 4 bits; with the bulk compression of a 32,768-token
      bf16 prefill of all 8 heads (Mtokens/s per KV head), alone and on a
      second stream beside the decode steps;
  w2  28 layers, 4 KV heads, 28 query heads, 8,192 tokens, K 4 bits, V 4 bits;
  w1  one head, 1,024 tokens, K 3 bits, V 2 bits (latency-bound).
Inputs are the seeded synthetic workloads of workloads/ (Gaussian K/V with
per-channel log-normal scales and outlier channels, bf16), resident in HBM
before timing.  Timed loops rotate among enough cache copies to exceed twice
the 256 MB Infinity Cache, so decode reads come from HBM.

Prints one JSON line: metric / value (the headline step's algorithmic GB/s),
the dominant kernel's roofline, the other workloads, and the float64 CPU
oracle timed on a bounded sample of the headline workload.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0
MALL_BYTES = 256 << 20
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_quantization_norm_amd", "csrc", f)
                  for f in ("tq_kernels.hip", "tq_host.cpp", "tq_internal.h")]
D = 128


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed,
    so that an edit to comments alone leaves the digest unchanged (string
    and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """sha256 of the kernel and host sources' code (comments and layout
    excluded): the key under which committed counter summaries are valid."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def traffic_key(short, k_bits, v_bits):
    """Name of a decode kernel's committed HBM traffic summary."""
    return f"decode_{short}_k{k_bits}v{v_bits}"


def measured_traffic(name):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary profiles/<name>_hbm_traffic.txt (FETCH_SIZE and WRITE_SIZE, each
    scaled by what the counter reads for a plain copy of known size), or None
    when the summary is missing or was taken on other kernel sources."""
    try:
        txt = open(os.path.join(ROOT, "profiles", name + "_hbm_traffic.txt")).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in txt.splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256:")))
    if fields.get("kernel_source_sha256", "").strip() != kernel_source_digest():
        return None
    return int(fields["traffic_bytes_per_launch"].strip())


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--only", default="w3,w4,w5,w2,w1",
                   help="workloads to run, comma separated (the first listed of w3 w4 w5 w2 w1 is the headline)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-stream-probe", action="store_true")
    p.add_argument("--copy-probe", action="store_true", help="also run a plain 1 GiB copy (PMC scaling)")
    return p.parse_args()


def rec_bytes(k_bits, v_bits):
    k = 2 * D if k_bits == 0 else D * (k_bits - 1) // 8 + D // 8 + 8
    v = 2 * D if v_bits == 0 else D * v_bits // 8 + 4
    return k, v


class Part:
    """One storage format of a workload: the layers that share it, their cache
    (and copies), tables, queries and the step's new tokens."""

    def __init__(self, tq, torch, w, layers, k_bits, v_bits, starts, lens, cap, dev, new_slots):
        self.tq, self.torch = tq, torch
        self.layers = layers
        self.L = len(layers)
        self.k_bits, self.v_bits = k_bits, v_bits
        self.fmt = tq.make_format(D, k_bits, v_bits)
        self.tables = tq.Tables.create(self.fmt, layers, dev)
        self.cache = tq.Cache.allocate(self.fmt, self.L, w.n_kv_heads, cap, dev)
        import workloads as wl
        dt = torch.bfloat16
        B, H = len(lens), w.n_kv_heads
        self.k_new = torch.empty((self.L, B, H, D), dtype=dt, device=dev)
        self.v_new = torch.empty_like(self.k_new)
        for i, layer in enumerate(layers):
            k, v = wl.gen_kv(w, layer)           # [sum(lens)][H][D], sequences in order
            kt = torch.from_numpy(k).to(dev, dt)
            vt = torch.from_numpy(v).to(dev, dt)
            pos = 0
            for b, n in enumerate(lens):
                # the cache holds tokens 0 .. n-2; token n-1 is the step's new token
                if n > 1:
                    self.tq.tq_compress_kv(self.fmt, self.tables, self.cache, kt[pos:pos + n - 1][None].contiguous(),
                                           vt[pos:pos + n - 1][None].contiguous(), layer0=i, slot0=int(starts[b]))
                self.k_new[i, b] = kt[pos + n - 1]
                self.v_new[i, b] = vt[pos + n - 1]
                pos += n
            del kt, vt
        torch.cuda.synchronize()
        self.q = torch.from_numpy(np.stack([wl.gen_q(w, layer) for layer in layers])).to(dev).contiguous()
        self.out = torch.empty((self.L, B, w.n_q_heads, D), device=dev)
        self.seq_start = torch.from_numpy(np.asarray(starts, np.int64)).to(dev)
        self.seq_len = torch.from_numpy(np.asarray(lens, np.int32)).to(dev)
        self.new_slots = torch.from_numpy(np.asarray(new_slots, np.int64)).to(dev)
        self.B, self.Hq, self.T = B, w.n_q_heads, int(max(lens))
        self.ws = tq.workspace_for(self.fmt, self.cache, B, self.Hq, self.T, dev)
        kr, vr = rec_bytes(k_bits, v_bits)
        self.record_bytes = self.L * H * int(sum(lens)) * (kr + vr)
        self.copies = [self.cache]

    def make_copies(self, n):
        tq = self.tq
        self.copies = [self.cache] + [tq.Cache(self.fmt, self.L, self.cache.n_kv_heads, self.cache.capacity,
                                               {k: (None if t is None else t.clone())
                                                for k, t in self.cache.planes.items()}) for _ in range(n - 1)]

    def step(self, i, stream):
        """Append the step's new tokens and decode (one tq_decode_step call)."""
        c = self.copies[i % len(self.copies)]
        B = self.B
        if B == 1:
            self.tq.tq_decode_step(self.fmt, self.tables, c, self.k_new, self.v_new, self.q, self.seq_start,
                                   self.seq_len, self.T, self.out, self.ws, slot0=int(self.new_slot0), stream=stream)
        else:
            self.tq.tq_decode_step(self.fmt, self.tables, c, self.k_new, self.v_new, self.q, self.seq_start,
                                   self.seq_len, self.T, self.out, self.ws, slots=self.new_slots, stream=stream)

    def prepare(self, stream):
        self.tq.tq_decode_prepare(self.fmt, self.tables, self.cache, self.q, self.T, self.ws, stream=stream)

    def attend(self, i, stream):
        c = self.copies[i % len(self.copies)]
        self.tq.tq_decode_attend(self.fmt, self.tables, c, self.B, self.Hq, self.seq_start, self.seq_len, self.T,
                                 self.out, self.ws, stream=stream)

    def kernel_bytes(self):
        """Algorithmic bytes one decode_kernel launch (tq_decode_attend) reads
        and writes: the records, the prepared queries, Pi once per layer (the
        output rotation of values kept as codes) and the outputs."""
        q = self.L * self.B * self.Hq * 2 * D * 4
        pi = self.L * D * D * 4 if self.v_bits > 0 else 0
        out = self.L * self.B * self.Hq * D * 4
        return self.record_bytes + q + pi + out


def build_parts(tq, torch, w, dev):
    """The storage formats of workload w, each with its layers."""
    import workloads as wl
    lens = list(w.seq_lens)
    # every sequence starts on a 32-slot boundary, with room for its last token
    starts, pos = [], 0
    for n in lens:
        starts.append(pos)
        pos += (n + 31) // 32 * 32
    cap = max(pos, 32)
    new_slots = [s + n - 1 for s, n in zip(starts, lens)]
    groups = {}
    for layer, mode in enumerate(w.modes()):
        if mode == wl.MODE_TQ:
            key = (w.k_bits, w.v_bits)
        elif mode == wl.MODE_KF16:
            key = (0, w.v_bits)
        else:
            key = (0, 0)
        groups.setdefault(key, []).append(layer)
    parts = []
    # the fp16 / fp16 part last: two parts whose second is fp16 / fp16 share one
    # decode launch (tq_decode_step_parts)
    for (kb, vb), layers in sorted(groups.items(), key=lambda kv: kv[0] == (0, 0)):
        p = Part(tq, torch, w, layers, kb, vb, starts, lens, cap, dev, new_slots)
        p.new_slot0 = new_slots[0]
        parts.append(p)
    return parts


def step_parts(tq, parts, i, stream):
    """One decode step over every part: one tq_decode_step call for a single
    format, else one tq_decode_step_parts call over all of them."""
    if len(parts) == 1:
        parts[0].step(i, stream)
        return
    p0 = parts[0]
    sp = [tq.StepPart(p.fmt, p.tables, p.copies[i % len(p.copies)], p.k_new, p.v_new, p.q, p.out, p.ws)
          for p in parts]
    if p0.B == 1:
        tq.tq_decode_step_parts(sp, p0.seq_start, p0.seq_len, p0.T, slot0=int(p0.new_slot0), stream=stream)
    else:
        tq.tq_decode_step_parts(sp, p0.seq_start, p0.seq_len, p0.T, slots=p0.new_slots, stream=stream)


def attend_parts(tq, parts, i, stream):
    """The decode launch of step_parts alone, on prepared queries."""
    p0 = parts[0]
    sp = [tq.StepPart(p.fmt, p.tables, p.copies[i % len(p.copies)], None, None, p.q, p.out, p.ws) for p in parts]
    tq.tq_decode_attend_parts(sp, p0.seq_start, p0.seq_len, p0.T, stream=stream)


def timed(torch, stream, fn, warmup, steps):
    """Mean ms per call of fn(i) over `steps` calls after `warmup` calls, with
    two HIP events on `stream` around the timed calls; about 0.1 s of the same
    calls comes first, untimed, besides the warm-up calls.  Python's garbage
    collector stays off meanwhile: a collection that frees device memory
    synchronizes the device and would stall the launches being timed."""
    import gc
    gc.collect()
    gc.disable()
    try:
        # spin-up: about 0.1 s of the same work first (after seconds of host-side
        # setup the GPU's clocks take longer to rise than a few launches last)
        t_end = time.perf_counter() + 0.1
        j = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn(j)
                j += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / steps


def run_workload(tq, torch, w, short, args, stream, dev):
    import gc
    gc.collect()                 # the previous workload's buffers, freed before anything is timed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    t0 = time.time()
    parts = build_parts(tq, torch, w, dev)
    total_cache = sum(p.cache.nbytes() for p in parts)
    n_copies = max(2, math.ceil(2 * MALL_BYTES / total_cache) + 1)
    for p in parts:
        p.make_copies(n_copies)
    log(f"{w.name}: {len(parts)} format(s), cache {total_cache / 1e6:.1f} MB x {n_copies} copies, "
        f"setup {time.time() - t0:.1f}s")
    H, Hq, B = w.n_kv_heads, w.n_q_heads, w.batch
    # one step over every part (one tq_decode_step_parts call for several formats)
    step_ms = timed(torch, stream, lambda i: step_parts(tq, parts, i, stream), args.warmup, args.steps)
    records = sum(p.record_bytes for p in parts)
    new_tok = w.n_layers * B * H * 2 * D * 2 + sum(p.L * B * H * sum(rec_bytes(p.k_bits, p.v_bits)) for p in parts)
    qo = 2 * w.n_layers * B * Hq * D * 4
    tables = sum(p.L * D * D * 4 * ((p.k_bits > 0) * 2 + (p.v_bits > 0)) for p in parts)   # Pi, S, S Pi^T read
    step_bytes = records + new_tok + qo + tables
    res = {"workload": w.name, "layers": w.n_layers, "kv_heads": H, "q_heads": Hq, "batch": B,
           "cached_tokens": int(sum(w.seq_lens)), "formats": [f"K{p.k_bits}/V{p.v_bits} x {p.L} layers"
                                                               for p in parts],
           "step_us": round(step_ms * 1e3, 2), "step_bytes": step_bytes,
           "step_GBs": round(step_bytes / (step_ms * 1e-3) / 1e9, 1), "cache_copies": n_copies}
    # the dominant kernel: each part's decode_kernel alone (tq_decode_attend on
    # prepared queries), launched back to back over the copies, events around
    # the batch on the stream it runs on
    kern = []
    for p in parts:
        p.prepare(stream)
        us = timed(torch, stream, lambda i, p=p: p.attend(i, stream), args.warmup, args.steps) * 1e3
        kb = p.kernel_bytes()
        mk = max(p.k_bits - 1, 0)
        kern.append({"kernel": f"decode_kernel<{mk}, {p.v_bits}, false>", "layers": p.L,
                     "us_per_launch": round(us, 2), "bytes_per_launch": kb,
                     "GBs": round(kb / (us * 1e-6) / 1e9, 1),
                     "frac_of_hbm_peak": round(kb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "workgroups": tq.tq_decode_split(p.fmt, p.L, B, H, Hq, p.T)["n_workgroups"],
                     "traffic": measured_traffic(traffic_key(short, p.k_bits, p.v_bits))})
    if len(parts) == 2 and (parts[1].k_bits, parts[1].v_bits) == (0, 0):
        # the step's decode: both parts in one launch of decode_pair_kernel
        us = timed(torch, stream, lambda i: attend_parts(tq, parts, i, stream), args.warmup, args.steps) * 1e3
        kb = sum(p.kernel_bytes() for p in parts)
        mk = max(parts[0].k_bits - 1, 0)
        kern.append({"kernel": f"decode_pair_kernel<{mk}, {parts[0].v_bits}>", "layers": sum(p.L for p in parts),
                     "us_per_launch": round(us, 2), "bytes_per_launch": kb,
                     "GBs": round(kb / (us * 1e-6) / 1e9, 1),
                     "frac_of_hbm_peak": round(kb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "workgroups": 256,
                     "traffic": measured_traffic(f"decode_pair_{short}")})
    res["decode_kernels"] = kern
    dom = max(kern, key=lambda k: k["bytes_per_launch"])
    res["roofline"] = {"bound": "hbm", "achieved": dom["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": dom["frac_of_hbm_peak"], "traffic": dom["traffic"], "kernel": dom["kernel"]}
    return res, parts


def multi_query_scores(tq, torch, p, args, stream, dev, rows=64):
    """Scores of `rows` query rows per KV head (say 8 heads x 8 query tokens of
    a prefill chunk) over a workload part's cache: tq_score_multi reads and
    decodes each KV head's key codes once per 64 rows, tq_score's decode
    kernel once per 8 rows.  Both include the query preparation."""
    H = p.cache.n_kv_heads
    Hq = H * rows
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    q = torch.randn((p.L, p.B, Hq, D), generator=g, device=dev)
    ws = tq.workspace_for(p.fmt, p.cache, p.B, Hq, p.T, dev)
    lg = torch.empty((p.L, p.B, Hq, p.T), device=dev)
    n = len(p.copies)
    res = {"what": f"{rows} query rows per KV head scored against the cache ({Hq} rows in all)"}
    for name, fn in (("multi", tq.tq_score_multi), ("decode_kernel_8_rows_per_pass", tq.tq_score)):
        us = timed(torch, stream, lambda i, fn=fn: fn(p.fmt, p.tables, p.copies[i % n], q, p.seq_start, p.seq_len,
                                                      p.T, lg, ws, stream=stream), args.warmup, args.steps) * 1e3
        res[name + "_us"] = round(us, 2)
    kr, _ = rec_bytes(p.k_bits, p.v_bits)
    tokens = int(p.seq_len.sum().item())
    key_bytes = p.L * H * tokens * kr
    logit_bytes = p.L * Hq * tokens * 4
    res["key_record_bytes_read_once"] = key_bytes
    res["key_record_bytes_read_8_rows_per_pass"] = key_bytes * ((rows + 7) // 8)
    res["logit_bytes_written"] = logit_bytes
    res["multi_GBs_algorithmic"] = round((key_bytes + logit_bytes) / (res["multi_us"] * 1e-6) / 1e9, 1)
    res["speedup"] = round(res["decode_kernel_8_rows_per_pass_us"] / res["multi_us"], 3)
    del lg, ws, q
    return res


def bulk_compress(tq, torch, w, args, stream, dev, decode_parts=None):
    """Bulk compression of the workload's prefill (all KV heads of one layer):
    alone, and on a second stream while decode steps run."""
    import workloads as wl
    k, v = wl.gen_prefill(w, 0)
    P, H = k.shape[0], w.n_kv_heads
    fmt = tq.make_format(D, w.k_bits, w.v_bits)
    tables = tq.Tables.create(fmt, [0], dev)
    K = torch.from_numpy(k).to(dev, torch.bfloat16)[None].contiguous()
    V = torch.from_numpy(v).to(dev, torch.bfloat16)[None].contiguous()
    target = tq.Cache.allocate(fmt, 1, H, (P + 31) // 32 * 32, dev)
    ms = timed(torch, stream, lambda i: tq.tq_compress_kv(fmt, tables, target, K, V, slot0=0, stream=stream),
               max(2, args.warmup), max(5, args.steps))
    flops = 6 * D * D * P * H          # Pi x (K), Pi x (V), (S Pi^T) r: 2 d^2 each per token-head
    rd, wr = 2 * P * H * D * 2, P * H * sum(rec_bytes(w.k_bits, w.v_bits))
    res = {"what": f"bulk compress of a {P}-token bf16 prefill x {H} KV heads, one call",
           "ms": round(ms, 4), "mtokens_per_s_per_kv_head": round(P / (ms * 1e-3) / 1e6, 2),
           "mtoken_heads_per_s": round(P * H / (ms * 1e-3) / 1e6, 2),
           "algorithmic_gflop": round(flops / 1e9, 2),
           "mfma_tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_of_f16_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFS, 4),
           "hbm_GBs": round((rd + wr) / (ms * 1e-3) / 1e9, 1)}
    if decode_parts:
        side = torch.cuda.Stream()
        p = decode_parts[0]
        step_ms = timed(torch, stream, lambda i: p.step(i, stream), args.warmup, args.steps)
        n_steps = max(1, int(round(ms / step_ms)))
        vals = []
        for rep in range(4):   # the first is a warm-up
            torch.cuda.synchronize()
            start, a1, b0, b1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            start.record(stream)
            side.wait_event(start)
            b0.record(side)
            tq.tq_compress_kv(fmt, tables, target, K, V, slot0=0, stream=side)
            b1.record(side)
            for i in range(n_steps):
                p.step(i, stream)
            a1.record(stream)
            torch.cuda.synchronize()
            if rep:
                vals.append((start.elapsed_time(a1), b0.elapsed_time(b1),
                             max(start.elapsed_time(a1), start.elapsed_time(b1))))
        vals.sort(key=lambda x: x[2])
        a, b, wall = vals[len(vals) // 2]
        res["with_decode_on_main_stream"] = {
            "decode_steps": n_steps, "step_us_alone": round(step_ms * 1e3, 2),
            "step_us_overlapped": round(a / n_steps * 1e3, 2), "compress_ms_overlapped": round(b, 4),
            "wall_ms": round(wall, 4), "serial_ms": round(n_steps * step_ms + ms, 4)}
    del K, V, target
    return res


def stream_read(tq, torch, stream, dev):
    """A plain streaming read (tq_stream_read_probe over 2 GiB, two buffers in
    turn, past the Infinity Cache): the best of a few workgroup counts."""
    bufs = [torch.ones(1 << 29, device=dev) for _ in range(2)]
    best = 0.0
    for nwg in (1024, 2048, 4096, 8192):
        part = torch.zeros(nwg, device=dev)
        ms = timed(torch, stream, lambda i: tq.tq_stream_read_probe(bufs[i % 2], part, nwg, stream=stream), 4, 10)
        best = max(best, (1 << 31) / (ms * 1e-3) / 1e9)
    del bufs
    return round(best, 1)


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model


def cpu_baseline(w, budget_s):
    """The float64 oracle decoding a bounded sample of the headline workload:
    whole layers (all KV and query heads, every cached token; the packed layers
    oracle-compressed first, untimed), in layer order, until about budget_s
    seconds of decode work; then the slowest of those layers again with the
    BLAS pool held to one thread (its rate beside the same layer's on all
    threads)."""
    import workloads as wl
    from oracle import attention, codebook, quant, rotation
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    lens = list(w.seq_lens)
    starts, pos = [], 0
    for n in lens:
        starts.append(pos)
        pos += (n + 31) // 32 * 32
    cap = max(pos, 32)

    def layer_fmt(layer):
        mode = w.modes()[layer]
        if mode == wl.MODE_TQ:
            return quant.Format(D, w.k_bits, w.v_bits)
        return quant.Format(D, 0, w.v_bits if mode == wl.MODE_KF16 else 0)

    def one_layer(layer):
        fmt = layer_fmt(layer)
        pi, s = rotation.layer_rotations(D, layer)
        cbk = codebook.table_codebook(D, fmt.k_mse_bits) if fmt.k_bits else None
        cbv = codebook.table_codebook(D, fmt.v_bits) if fmt.v_bits else None
        k, v = wl.gen_kv(w, layer)
        cache = quant.empty_cache(fmt, w.n_kv_heads, cap)
        slots = np.concatenate([np.arange(st, st + n) for st, n in zip(starts, lens)])
        quant.compress_into(cache, k.astype(np.float64), v.astype(np.float64), slots, pi, s, cbk, cbv)
        q = wl.gen_q(w, layer)
        t0 = time.perf_counter()
        attention.decode_attention(cache, q, starts, lens, pi, s, cbk, cbv)
        dt = time.perf_counter() - t0
        kr, vr = rec_bytes(fmt.k_bits, fmt.v_bits)
        return dt, w.n_kv_heads * sum(lens) * (kr + vr) + 2 * w.batch * w.n_q_heads * D * 4

    dec_s, nbytes, done, per = 0.0, 0, [], {}
    for layer in range(w.n_layers):
        dt, b = one_layer(layer)
        dec_s += dt
        nbytes += b
        done.append(layer)
        per[layer] = (dt, b)
        log(f"cpu oracle layer {layer}: {dt:.2f}s (total {dec_s:.1f}s)")
        if dec_s >= budget_s:
            break
    slow = max(per, key=lambda x: per[x][0])
    with threadpool_limits(limits=1):
        dt1, b1 = one_layer(slow)
    return {"value": round(nbytes / dec_s / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} of {w.n_layers} layers of {w.name} (layers {done[0]}..{done[-1]}, every KV and "
                      f"query head, every cached token), decode only ({dec_s:.1f}s on {threads} threads)",
            "one_thread_GBs": round(b1 / dt1 / 1e9, 4),
            "one_thread_sample": f"layer {slow} alone with one BLAS thread ({dt1:.1f}s)",
            "same_layer_all_threads_GBs": round(per[slow][1] / per[slow][0] / 1e9, 4),
            "cpu_model": cpu_info(), "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; more than one GPU is not part of this benchmark",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import kv_cache_quantization_norm_amd as tq
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    order = [x.strip() for x in args.only.split(",") if x.strip()]
    results = {}
    for short in order:
        w = wl.BY_SHORT[short]
        res, parts = run_workload(tq, torch, w, short, args, stream, dev)
        if short == "w5":
            res["bulk_compress"] = bulk_compress(tq, torch, w, args, stream, dev, parts)
        if short == "w4":
            res["multi_query_scores"] = multi_query_scores(tq, torch, parts[0], args, stream, dev)
        results[short] = res
        log(json.dumps(res))
        del parts
        torch.cuda.empty_cache()
    head = order[0]
    hr = results[head]
    # the dominant kernel of the headline step: the part with the most bytes
    dom = max(hr["decode_kernels"], key=lambda k: k["bytes_per_launch"])
    read_gbs = None if args.no_stream_probe else stream_read(tq, torch, stream, dev)
    result = {
        "metric": "decode-attention GB/s & % HBM roofline; compress Mtokens/s per KV head",
        "value": hr["step_GBs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hr["step_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (fp16 MFMA operands with high/remainder splits, f32 accumulation)",
        "data": "synthetic",
        "config": {"workload": wl.BY_SHORT[head].name, "layers": hr["layers"], "kv_heads": hr["kv_heads"],
                   "q_heads": hr["q_heads"], "head_dim": D, "batch": hr["batch"],
                   "cached_tokens": hr["cached_tokens"], "formats": hr["formats"], "kv_dtype": "bf16",
                   "step": "append-compress the new token of every sequence x every layer + decode attention "
                           "x every layer (one tq_decode_step per storage format)"},
        "roofline": {"bound": "hbm", "achieved": dom["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom["frac_of_hbm_peak"], "traffic": dom["traffic"],
                     "kernel": dom["kernel"], "bytes_per_launch": dom["bytes_per_launch"],
                     "us_per_launch": dom["us_per_launch"], "measured_stream_read_GBs": read_gbs,
                     "frac_of_measured_read": round(dom["GBs"] / read_gbs, 4) if read_gbs else None},
        "workloads": results,
    }
    if args.copy_probe:
        n = 1 << 28
        a = torch.empty(n, device=dev)
        b = torch.empty(n, device=dev)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = 2 * n * 4
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl.BY_SHORT[head], args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
