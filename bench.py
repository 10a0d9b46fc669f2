"""Benchmark of the TurboQuant decode hot path on one MI355X.

One step = one pass of the whole path over the dense 28-layer workload
(28 layers, 4 KV heads, 28 query heads (GQA 7), head_dim 128, batch 1,
8192 cached tokens, K 4 bits = 3 Lloyd-Max + 1 QJL, V 4 bits MSE-only):
  1. compress the step's new token (K and V, all 4 KV heads of all 28 layers)
     into slot 8191 of the packed cache;
  2. decode attention for all 28 query heads of all 28 layers over the 8192
     packed tokens.
One tq_decode_step call: the query preparation, then one decode launch whose
first 28 workgroups compress the new token while the others attend (a wave
waits for its layer's append only before the chunk that holds slot 8191), the
pieces of each problem merged inside the kernel by its last workgroup.
The same step as tq_append_prepare + tq_decode_attend and as tq_compress_kv +
tq_decode_attention is timed beside it.
Inputs are seeded synthetic bf16 K/V (per-channel log-normal scales, two
outlier channels per head) already resident in HBM.  The timed loop rotates
among enough cache copies to exceed twice the 256 MB Infinity Cache, so
decode reads come from HBM.

Prints one JSON line: metric / value (algorithmic GB/s of the step), the
decode kernel's roofline, bulk-compression throughput, and the float64 CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_w2_dense28L_hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_quantization_norm_amd", "csrc", f)
                  for f in ("tq_kernels.hip", "tq_host.cpp", "tq_internal.h")]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode_kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size), or None when the summary was taken on
    other kernel sources than the ones in this tree."""
    try:
        txt = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in txt.splitlines() if line.startswith(("traffic_bytes_per_launch:",
                                                                                         "kernel_source_sha256:")))
    if fields.get("kernel_source_sha256", "").strip() != kernel_source_digest():
        return None
    return int(fields["traffic_bytes_per_launch"].strip())
MALL_BYTES = 256 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--workload", default="w2")
    p.add_argument("--copies", type=int, default=0, help="cache copies (0 = enough to exceed 2x the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--copy-probe", action="store_true", help="also run a plain copy of known size (PMC scaling)")
    p.add_argument("--per-layer", action="store_true",
                   help="also time 28 one-layer decode calls per step (adds one-layer decode launches to a profile)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the path is measured on one GPU's share)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import kv_cache_quantization_norm_amd as tq
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = wl.BY_SHORT[args.workload]
    assert len(w.seq_lens) == 1 and not w.layer_modes, "the timed step covers single-sequence symmetric workloads"
    L, H, HQ, T, D = w.n_layers, w.n_kv_heads, w.n_q_heads, w.seq_lens[0], w.head_dim
    fmt = tq.make_format(D, w.k_bits, w.v_bits)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    stream = torch.cuda.current_stream()

    # ---------------- setup: tables, inputs, bulk compression of the cache
    t0 = time.time()
    tables = tq.Tables.create(fmt, list(range(L)), dev)
    K = torch.empty((L, T, H, D), dtype=dt, device=dev)
    V = torch.empty_like(K)
    for layer in range(L):
        k, v = wl.gen_kv(w, layer)
        K[layer].copy_(torch.from_numpy(k).to(dt))
        V[layer].copy_(torch.from_numpy(v).to(dt))
    Q = torch.from_numpy(np.stack([wl.gen_q(w, layer) for layer in range(L)])).to(dev).contiguous()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    cap = (T + 31) // 32 * 32
    base = tq.Cache.allocate(fmt, L, H, cap, dev)
    # Bulk compression of the whole 28-layer prefill, timed.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tq.tq_compress_kv(fmt, tables, base, K, V, slot0=0)  # warm
    torch.cuda.synchronize()
    reps = 5
    ev0.record(stream)
    for _ in range(reps):
        tq.tq_compress_kv(fmt, tables, base, K, V, slot0=0)
    ev1.record(stream)
    torch.cuda.synchronize()
    bulk_ms = ev0.elapsed_time(ev1) / reps
    cache_bytes = base.nbytes()
    n_copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / cache_bytes) + 1)
    caches = [base] + [tq.Cache(fmt, L, H, cap, {k: (None if t is None else t.clone()) for k, t in base.planes.items()})
                       for _ in range(n_copies - 1)]
    log(f"cache {cache_bytes / 1e6:.1f} MB x {n_copies} copies; bulk compress {bulk_ms:.3f} ms")

    # the step's new token: token T-1 of every layer
    k_new = K[:, T - 1:T].contiguous()
    v_new = V[:, T - 1:T].contiguous()
    seq_start = torch.zeros(1, dtype=torch.int64, device=dev)
    seq_len = torch.full((1,), T, dtype=torch.int32, device=dev)
    ws = tq.workspace_for(fmt, base, 1, HQ, T, dev)
    out = torch.empty((L, 1, HQ, D), device=dev)

    def step(c):
        tq.tq_decode_step(fmt, tables, c, k_new, v_new, Q, seq_start, seq_len, T, out, ws, slot0=T - 1,
                          stream=stream)

    def step_prepare_attend(c):
        tq.tq_append_prepare(fmt, tables, c, k_new, v_new, Q, T, ws, slot0=T - 1, stream=stream)
        tq.tq_decode_attend(fmt, tables, c, 1, HQ, seq_start, seq_len, T, out, ws, stream=stream)

    def step_two_calls(c):
        tq.tq_compress_kv(fmt, tables, c, k_new, v_new, slot0=T - 1, stream=stream)
        tq.tq_decode_attention(fmt, tables, c, Q, seq_start, seq_len, T, out, ws, stream=stream)

    def decode_only(c):
        tq.tq_decode_attention(fmt, tables, c, Q, seq_start, seq_len, T, out, ws, stream=stream)

    # ---------------- timed steps
    for i in range(args.warmup):
        step(caches[i % n_copies])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(caches[i % n_copies])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = e0.elapsed_time(e1) / args.steps

    # the same step as tq_compress_kv + tq_decode_attention (three launches)
    # and as tq_append_prepare + tq_decode_attend (two launches)
    def time_steps(fn):
        for i in range(args.warmup):
            fn(caches[i % n_copies])
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(caches[i % n_copies])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    step_two_calls_ms = time_steps(step_two_calls)
    step_prepare_attend_ms = time_steps(step_prepare_attend)

    # decode call alone (query prep + decode kernel), same rotation
    for i in range(args.warmup):
        decode_only(caches[i % n_copies])
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        decode_only(caches[i % n_copies])
    e1.record(stream)
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1) / args.steps

    # the dominant kernel alone: the staged entry points, with events around
    # the tq_decode_attend launch (decode_kernel) only, on the stream it runs on
    def staged(c, ev=None):
        tq.tq_decode_prepare(fmt, tables, c, Q, T, ws, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        tq.tq_decode_attend(fmt, tables, c, 1, HQ, seq_start, seq_len, T, out, ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        staged(caches[i % n_copies])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        staged(caches[i % n_copies], evs[i])
    torch.cuda.synchronize()
    kern_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    # the same launches back to back (the queries prepared once; every launch
    # reads another cache copy), two events around the batch: the mean launch
    # time without an event pair per launch
    tq.tq_decode_prepare(fmt, tables, base, Q, T, ws, stream=stream)
    for i in range(args.warmup):
        tq.tq_decode_attend(fmt, tables, caches[i % n_copies], 1, HQ, seq_start, seq_len, T, out, ws, stream=stream)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(args.steps):
        tq.tq_decode_attend(fmt, tables, caches[i % n_copies], 1, HQ, seq_start, seq_len, T, out, ws, stream=stream)
    b1.record(stream)
    torch.cuda.synchronize()
    kern_batch_us = b0.elapsed_time(b1) * 1e3 / args.steps

    # ---------------- background recompression.  The MLX write-up recompresses
    # its packed store in the background while decoding; here the bulk
    # compression of the whole prefill runs into another cache on a second
    # stream (default priority) while decode steps run on the main one.
    # Unbounded, the compression takes every CU; bounded to the CUs that the
    # decode kernel leaves free (tq_compress_kv_bounded), it runs beside it.
    side = torch.cuda.Stream()
    target = tq.Cache.allocate(fmt, L, H, cap, dev)
    # CUs the step's decode launch leaves free: its decode workgroups and its
    # append workgroups (one per layer and 8 (token, head) items)
    free_cus = max(1, 256 - tq.tq_decode_split(fmt, L, 1, H, HQ, T)["n_workgroups"] - L * -(-H // 8))

    def overlapped(max_wgs, n_steps):
        ov = []
        for rep in range(4):   # the first is a warm-up
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            a1, b0, b1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            start.record(stream)
            side.wait_event(start)
            b0.record(side)
            tq.tq_compress_kv_bounded(fmt, tables, target, K, V, max_wgs, slot0=0, stream=side)
            b1.record(side)
            for i in range(n_steps):
                step(caches[i % n_copies])
            a1.record(stream)
            torch.cuda.synchronize()
            if rep:
                ov.append((start.elapsed_time(a1), b0.elapsed_time(b1),
                           max(start.elapsed_time(a1), start.elapsed_time(b1))))
        ov.sort(key=lambda x: x[2])
        return ov[len(ov) // 2]

    def bounded_alone(max_wgs):
        tq.tq_compress_kv_bounded(fmt, tables, target, K, V, max_wgs, slot0=0, stream=stream)
        torch.cuda.synchronize()
        t0_, t1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0_.record(stream)
        tq.tq_compress_kv_bounded(fmt, tables, target, K, V, max_wgs, slot0=0, stream=stream)
        t1_.record(stream)
        torch.cuda.synchronize()
        return t0_.elapsed_time(t1_)

    n_ov = max(1, int(round(bulk_ms / step_ms)))
    ov_steps_ms, ov_compress_ms, ov_wall_ms = overlapped(0, n_ov)
    bnd_alone_ms = bounded_alone(free_cus)
    n_bnd = max(1, int(round(bnd_alone_ms / step_ms)))
    bnd_steps_ms, bnd_compress_ms, bnd_wall_ms = overlapped(free_cus, n_bnd)
    del target

    # ---------------- decode over the packed cache plus an fp16 tail of 255
    # recent tokens (the largest tail under a 256-token compression trigger)
    TT = 255
    fmt16 = tq.make_format(D, 0, 0)
    tail = tq.Cache.allocate(fmt16, L, H, 256, dev)
    tq.tq_compress_kv(fmt16, tables, tail, K[:, :TT].contiguous(), V[:, :TT].contiguous(), slot0=0)
    tst = torch.zeros(1, dtype=torch.int64, device=dev)
    tln = torch.full((1,), TT, dtype=torch.int32, device=dev)
    tws = tq.tail_workspace_for(fmt, base, 1, HQ, T, TT, dev)
    for i in range(args.warmup):
        tq.tq_decode_attention_tail(fmt, tables, caches[i % n_copies], tail, Q, seq_start, seq_len, T, tst, tln, TT,
                                    out, tws, stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        tq.tq_decode_attention_tail(fmt, tables, caches[i % n_copies], tail, Q, seq_start, seq_len, T, tst, tln, TT,
                                    out, tws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    tail_ms = e0.elapsed_time(e1) / args.steps
    del tail, tws

    # ---------------- a plain streaming read for reference (tq_stream_read_probe
    # over 2 GiB, two buffers in turn, past the Infinity Cache): the best of a
    # few workgroup counts
    bufs = [torch.ones(1 << 29, device=dev) for _ in range(2)]
    read_gbs = 0.0
    for nwg in (1024, 2048, 4096):
        part = torch.zeros(nwg, device=dev)
        for i in range(4):
            tq.tq_stream_read_probe(bufs[i % 2], part, nwg, stream=stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(10):
            tq.tq_stream_read_probe(bufs[i % 2], part, nwg, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        read_gbs = max(read_gbs, (1 << 31) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9)
    del bufs

    per_layer_ms = None
    if args.per_layer:
        per_layer_ms = time_per_layer(tq, fmt, tables, base, Q, seq_start, seq_len, T, stream, dev)

    # ---------------- algorithmic bytes
    k_rec = D * (w.k_bits - 1) // 8 + D // 8 + 8
    v_rec = D * w.v_bits // 8 + 4
    records = L * H * T * (k_rec + v_rec)
    tables_bytes = L * 3 * D * D * 4            # Pi, S and S Pi^T, read once per step
    qo = 2 * L * HQ * D * 4
    new_tok = L * H * 2 * D * (2 if dt != torch.float32 else 4) + L * H * (k_rec + v_rec)
    step_bytes = records + qo + tables_bytes + new_tok
    decode_bytes = records + qo + L * 2 * D * D * 4   # Pi and S
    # decode_kernel with the in-kernel merge: packed records, the prepared
    # queries (Pi q, S q), Pi for the output rotation (once per layer) and the
    # outputs
    kernel_bytes = records + L * HQ * 2 * D * 4 + L * D * D * 4 + L * HQ * D * 4
    pieces = decode_pieces(L * H * -(-(HQ // H) // 8), T)
    split_overhead = pieces * (HQ // H) * (D + 2) * 4  # fp32 partials written (and read back by the merge)
    step_gbs = step_bytes / (step_ms * 1e-3) / 1e9
    decode_gbs = decode_bytes / (decode_ms * 1e-3) / 1e9
    kern_mean = kern_batch_us
    kern_gbs = kernel_bytes / (kern_mean * 1e-6) / 1e9
    bulk_tokens = L * T
    result = {
        "metric": "decode-attention GB/s & % HBM roofline; compress Mtokens/s per KV head",
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (MFMA f16 hi+lo operands, f32 accumulation)",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "kv_heads": H, "q_heads": HQ, "head_dim": D,
                   "batch": 1, "cached_tokens": T, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "kv_dtype": w.dtype, "layers_per_call": L, "cache_copies": n_copies,
                   "step": "append-compress 1 token x 28 layers + decode attention x 28 layers"},
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": f"decode_kernel<{max(w.k_bits - 1, 0)},{w.v_bits},false>",
                     "bytes_per_launch": kernel_bytes, "us_per_launch": round(kern_mean, 2),
                     "us_per_launch_event_pair": {"mean": round(float(kern_us.mean()), 2),
                                                  "median": round(float(np.median(kern_us)), 2),
                                                  "p10": round(float(np.percentile(kern_us, 10)), 2),
                                                  "p90": round(float(np.percentile(kern_us, 90)), 2)},
                     "split_partials_bytes": split_overhead,
                     "measured_stream_read_GBs": round(read_gbs, 1),
                     "frac_of_measured_read": round(kern_gbs / read_gbs, 4)},
        "decode_call": {"us": round(decode_ms * 1e3, 2), "GBs": round(decode_gbs, 1),
                        "bytes": decode_bytes, "kernels": "qprep_kernel + decode_kernel (pieces merged in-kernel)"},
        "decode_step_bytes": step_bytes,
        "step_launches": "qprep_kernel + decode_kernel (append workgroups, decode, pieces merged in-kernel)",
        "step_two_calls_us": round(step_two_calls_ms * 1e3, 2),
        "step_append_prepare_attend_us": round(step_prepare_attend_ms * 1e3, 2),
        "compress": {"what": f"bulk prefill {T} tokens x {L} layers x {H} KV heads, one call",
                     "ms": round(bulk_ms, 4),
                     "mtokens_per_s_per_kv_head": round(bulk_tokens / (bulk_ms * 1e-3) / 1e6, 2),
                     "mtoken_heads_per_s": round(bulk_tokens * H / (bulk_ms * 1e-3) / 1e6, 2)},
        "decode_with_tail": {"tail_tokens": TT, "packed_tokens": T, "us": round(tail_ms * 1e3, 2),
                             "decode_call_us": round(decode_ms * 1e3, 2),
                             "kernels": "qprep_kernel (rotated and plain) + decode_kernel (fp16 tail) + decode_kernel (packed, merges both piece sets)"},
        "background_recompress": {
            "what": f"bulk compress of the {L} x {T}-token prefill on a second stream while decode steps run",
            "decode_steps": n_ov, "step_us_alone": round(step_ms * 1e3, 2),
            "step_us_overlapped": round(ov_steps_ms / n_ov * 1e3, 2),
            "compress_ms_alone": round(bulk_ms, 4), "compress_ms_overlapped": round(ov_compress_ms, 4),
            "wall_ms": round(ov_wall_ms, 4), "serial_ms": round(n_ov * step_ms + bulk_ms, 4),
            "bounded": {"compress_workgroups": free_cus, "decode_steps": n_bnd,
                        "step_us_overlapped": round(bnd_steps_ms / n_bnd * 1e3, 2),
                        "compress_ms_alone": round(bnd_alone_ms, 4), "compress_ms_overlapped": round(bnd_compress_ms, 4),
                        "wall_ms": round(bnd_wall_ms, 4), "serial_ms": round(n_bnd * step_ms + bnd_alone_ms, 4)}},
        "wall_s_timed": round(wall, 4),
    }
    if per_layer_ms is not None:
        result["per_layer_calls"] = {"us_per_step": round(per_layer_ms * 1e3, 2),
                                     "GBs": round(decode_bytes / (per_layer_ms * 1e-3) / 1e9, 1)}

    if args.copy_probe:
        n = 1 << 28  # 1 GiB of float32 read + 1 GiB written
        a = torch.empty(n, device=dev)
        b = torch.empty(n, device=dev)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = 2 * n * 4

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, result)
    print(json.dumps(result), flush=True)


def decode_pieces(problems, t, chunk=32, waves=8, max_workgroups=256, crossing_chunks=16):
    """Number of (problem, workgroup) pieces of a decode call, each leaving one
    partial per query head, following the library's work split: equal runs of
    chunks over the problem-major chunk sequence, or, when that is nearly as
    short, k = max_workgroups // problems aligned runs per problem."""
    cpp = -(-max(t, 1) // chunk)
    total = problems * cpp
    wgs = min(max_workgroups, -(-total // waves))
    cpw = -(-total // wgs)
    k = min(max_workgroups // problems, cpp // waves)
    if k >= 1 and cpp % cpw != 0 and -(-cpp // k) <= cpw + crossing_chunks:
        cpw = -(-cpp // k)
        cpp = k * cpw
    return sum((p * cpp + cpp - 1) // cpw - (p * cpp) // cpw + 1 for p in range(problems))


def time_per_layer(tq, fmt, tables, base, Q, seq_start, seq_len, T, stream, dev):
    """28 one-layer decode calls per step, as a model would issue them."""
    import torch
    L, H, cap = base.n_layers, base.n_kv_heads, base.capacity
    HQ, D = Q.shape[2], Q.shape[3]
    per_layer = [tq.Cache(fmt, 1, H, cap, {k: (None if t is None else t.view(L, -1)[l])
                                           for k, t in base.planes.items()}) for l in range(L)]
    layer_tables = []
    for l in range(L):
        lt = tq.Tables(fmt, tables.pi[l:l + 1], tables.s[l:l + 1], tables.pi_s[l:l + 1], tables.k_centroids,
                       tables.k_boundaries, tables.v_centroids, tables.v_boundaries, {})
        layer_tables.append(lt)
    ws1 = tq.workspace_for(fmt, per_layer[0], 1, HQ, T, dev)
    q_l = [Q[l:l + 1].contiguous() for l in range(L)]
    out_l = torch.empty((1, 1, HQ, D), device=dev)
    for _ in range(3):
        for l in range(L):
            tq.tq_decode_attention(fmt, layer_tables[l], per_layer[l], q_l[l], seq_start, seq_len, T, out_l, ws1,
                                   stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    nrep = 10
    for _ in range(nrep):
        for l in range(L):
            tq.tq_decode_attention(fmt, layer_tables[l], per_layer[l], q_l[l], seq_start, seq_len, T, out_l, ws1,
                                   stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / nrep


def cpu_baseline(w, budget_s, gpu_result):
    """The float64 oracle decoding a bounded sample of the same workload:
    whole layers (all KV and query heads, all 8192 tokens), oracle-compressed
    first (untimed), until about budget_s seconds of decode work."""
    import workloads as wl
    from oracle import attention, codebook, quant, rotation
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    fmt = quant.Format(w.head_dim, w.k_bits, w.v_bits)
    cbk = codebook.table_codebook(w.head_dim, fmt.k_mse_bits)
    cbv = codebook.table_codebook(w.head_dim, fmt.v_bits)
    T = w.seq_lens[0]
    cap = (T + 31) // 32 * 32
    k_rec = fmt.k_record_bytes()
    v_rec = fmt.v_record_bytes()
    dec_s = comp_s = 0.0
    layers = 0
    tok_heads = 0
    for layer in range(w.n_layers):
        pi, s = rotation.layer_rotations(w.head_dim, layer)
        k, v = wl.gen_kv(w, layer)
        cache = quant.empty_cache(fmt, w.n_kv_heads, cap)
        t0 = time.perf_counter()
        quant.compress_into(cache, k.astype(np.float64), v.astype(np.float64), np.arange(T), pi, s, cbk, cbv)
        comp_s += time.perf_counter() - t0
        q = wl.gen_q(w, layer)
        t0 = time.perf_counter()
        attention.decode_attention(cache, q, [0], [T], pi, s, cbk, cbv)
        dec_s += time.perf_counter() - t0
        layers += 1
        tok_heads += T * w.n_kv_heads
        log(f"cpu oracle layer {layer}: decode {dec_s:.1f}s compress {comp_s:.1f}s")
        if dec_s >= budget_s:
            break
    bytes_ = layers * w.n_kv_heads * T * (k_rec + v_rec) + 2 * layers * w.n_q_heads * w.head_dim * 4 \
        + layers * 2 * w.head_dim * w.head_dim * 4
    return {"value": round(bytes_ / dec_s / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{layers} of {w.n_layers} layers, full 8192-token cache, all heads (decode only, "
                      f"{dec_s:.1f}s); oracle compression of the same sample {comp_s:.1f}s = "
                      f"{tok_heads / comp_s / 1e6:.4f} Mtoken-heads/s",
            "compress_mtoken_heads_per_s": round(tok_heads / comp_s / 1e6, 5)}


if __name__ == "__main__":
    main()
