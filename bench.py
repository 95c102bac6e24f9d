"""Decode-step benchmark of the CommVQ hot path on one MI355X.

Workload: LLaMA-3.1-8B attention-layer shape (32 query heads, 8 KV heads,
head_dim 128) at 128K context, 1-bit CommVQ (g = 8, Nc' = 256, R = 1). The cache
is prefilled to 131008 tokens; each step appends one newly encoded token (keys and
values, all KV heads) and runs one decode-attention call over the packed codes,
so the context walks 131009 ... 131072 over 64 decode positions. Steps rotate
over several layer slices whose caches together exceed the 256 MB Infinity
Cache, so every step reads its codes from HBM.

Prints one JSON line. `value` is cached tokens attended per second,
sum_b L_b / step time. `roofline` reports the decode kernel's packed-code HBM
bytes per launch over its average duration (HIP events around each launch on
the stream it runs on). `cpu_baseline` times the CPU oracle on a bounded sample.
"""

from __future__ import annotations

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

METRIC = "decode-attn cached tokens/s (GQA 32q/8kv, 128K ctx) + % HBM peak on packed codes"
HBM_PEAK_GBS = 8000.0
WORKLOAD = "llama8b_ctx128k_1bit_64steps"
PREFILL = 131008
N_POSITIONS = 64

# HBM bytes per commvq_decode_step call (decode kernel + chunk-merge kernel) from
# rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
# reads on a plain streaming kernel of known size; the commands and figures are
# in the decode_fast summary under profiles/), valid for the kernel sources whose
# SHA-256 is given: any change to them voids it.
KERNEL_SOURCES = ['decode_fast.hip', 'decode_merge.hip', 'decode.hip', 'decode_common.hpp', 'encode_common.hpp', 'commvq_internal.hpp']
TRAFFIC = {"sha256": "7f16368fa5e13dfd296fc496bf2824f9d995dac40efa8f88e5265e6e3fc2e51e",
           "read_bytes": 35943454, "write_bytes": 555520}


def measured_traffic():
    """Counter-measured HBM bytes per launch, or None once the kernel's sources
    differ from the ones the counters were taken on."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_attention_commvq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != TRAFFIC["sha256"]:
        return None
    return TRAFFIC["read_bytes"] + TRAFFIC["write_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=16, help="layer slices rotated over (caches > MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="decode workload to time (default: the 128K 1-bit decode-step workload)")
    ap.add_argument("--encode", action="store_true",
                    help="time the prefill encoder instead (131072 tokens x 8 KV heads of K and V, 2-bit)")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps issued from the host one call at a time (default: the timed steps are "
                         "captured once in a HIP graph and its replay is timed; per-step eager event times are "
                         "reported either way)")
    ap.add_argument("--naive", action="store_true",
                    help="time the comparison path (dequantise the codes to fp16, then dense attention) against "
                         "commvq_decode_attention on the same 128K 1-bit caches, instead of the headline step")
    ap.add_argument("--bitv", action="store_true",
                    help="time decode attention with binary value codes (1024 bits per token) at 128K against the "
                         "same generic kernel with residual-codebook values, and the fast path")
    ap.add_argument("--em", action="store_true",
                    help="time one EM iteration of codebook fitting (commvq_em_step) on the prefill workload's keys")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain streaming kernel (fp32 negate) over this many MiB, 5 times, and exit; "
                         "its FETCH_SIZE/WRITE_SIZE counters calibrate the decode kernel's")
    return ap.parse_args()


def copy_calibration(mib: int):
    """A plain streaming kernel of known size: reads and writes `mib` MiB once
    per launch, so hardware byte counters taken over it give the factor between
    counted and actual HBM bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "fp32 negate", "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4, "launches": 5}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s: float):
    """Time the fp64 oracle (unpack -> dequantise -> RoPE -> dense softmax) on
    (KV head, decode position) units of the workload at full context: one unit
    is one KV head with its 4 query heads at L = 131009 + t. Units are run until
    the budget is spent (at least one step's 8 heads), then the mean unit time
    is scaled to one 8-head step. BLAS may use every host core this process is
    allowed (at most 16); the rest of NumPy runs on one thread."""
    from threadpoolctl import threadpool_limits

    from long_context_attention_commvq_amd import synth
    from oracle import commvq_oracle as O

    w = synth.WORKLOADS[WORKLOAD]
    G = w.head_dim // w.group_size
    kcb = synth.codebook(w.seed + 1, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    vcb = synth.codebook(w.seed + 2, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    rep = w.n_q_heads // w.n_kv_heads
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    units, t_total, toks = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        while units < N_POSITIONS * w.n_kv_heads and (units < w.n_kv_heads or t_total < budget_s):
            t = units // w.n_kv_heads
            L = PREFILL + t + 1
            kc = synth.random_codes(w.seed + 100 + units, (L, 1, w.n_rounds, G), w.n_entries)
            vc = synth.random_codes(w.seed + 200 + units, (L, 1, w.n_rounds, G), w.n_entries)
            kp = O.pack_codes(kc, w.n_entries).transpose(1, 0, 2)[None]
            vp = O.pack_codes(vc, w.n_entries).transpose(1, 0, 2)[None]
            q = synth.queries(w.seed + 300 + units, 1, rep, w.head_dim)
            t0 = time.perf_counter()
            O.decode_attention_from_packed(q, np.array([L - 1]), kp, vp, np.array([L]), kcb, vcb, w.theta_base)
            t_total += time.perf_counter() - t0
            units += 1
            toks += L
    t_step = t_total / units * w.n_kv_heads
    L_mean = toks / units
    return {"value": L_mean / t_step, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{units} (KV head, step) units of the {WORKLOAD} workload, mean L={L_mean:.0f}, "
                      f"fp64 NumPy, BLAS threads={cores}; {t_total:.1f} s measured, "
                      f"mean unit time scaled x{w.n_kv_heads} to one 8-head step"}


def decode_cpu_baseline(budget_s: float, w, lens, value_bits: int = 0):
    """Time the fp64 oracle on (sequence, KV head) units of a decode workload w:
    unit u is sequence u % B's query heads of one KV head over its L_b cached
    positions (seeded random records), run for at least one unit and until the
    budget is spent. One call covers every KV head, so the rate is the units'
    positions over their time divided by Hkv. value_bits > 0 times the binary
    value oracle instead (value codes of value_bits bits per token; one KV
    head's D columns of the rows)."""
    from threadpoolctl import threadpool_limits

    from long_context_attention_commvq_amd import synth
    from oracle import commvq_oracle as O

    G = w.head_dim // w.group_size
    kcb = synth.codebook(w.seed + 1, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    vcb = synth.codebook(w.seed + 2, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    rep = w.n_q_heads // w.n_kv_heads
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    units, t_total, toks = 0, 0.0, 0
    with threadpool_limits(limits=cores):
        while units < len(lens) * w.n_kv_heads and (units == 0 or t_total < budget_s):
            L = int(lens[units % len(lens)])
            kc = synth.random_codes(w.seed + 500 + units, (L, 1, w.n_rounds, G), w.n_entries)
            kp = O.pack_codes(kc, w.n_entries).transpose(1, 0, 2)[None]
            q = synth.queries(w.seed + 700 + units, 1, rep, w.head_dim)
            if value_bits:
                r = synth.rng(w.seed + 600 + units)
                vb = r.integers(0, 256, size=(1, L, value_bits // 8)).astype(np.uint8)
                rows = (r.standard_normal((value_bits, w.head_dim)) / math.sqrt(value_bits / 2)).astype(np.float16)
                t0 = time.perf_counter()
                O.decode_attention_bit_values(q, np.array([L - 1]), kp, vb, np.array([L]), kcb, rows, w.theta_base)
            else:
                vc = synth.random_codes(w.seed + 600 + units, (L, 1, w.n_rounds, G), w.n_entries)
                vp = O.pack_codes(vc, w.n_entries).transpose(1, 0, 2)[None]
                t0 = time.perf_counter()
                O.decode_attention_from_packed(q, np.array([L - 1]), kp, vp, np.array([L]), kcb, vcb, w.theta_base)
            t_total += time.perf_counter() - t0
            units += 1
            toks += L
    kind = f"binary value codes ({value_bits} bits per token)" if value_bits else "residual value codebook"
    return {"value": toks / t_total / w.n_kv_heads, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{units} (sequence, KV head) units of the {w.name} shape ({kind}), {toks} cached positions, "
                      f"fp64 NumPy, BLAS threads={cores}; {t_total:.1f} s measured, scaled to all "
                      f"{w.n_kv_heads} KV heads of one call"}


def encode_cpu_baseline(budget_s: float, w):
    """Time the fp64 oracle encoder (squared distances to every entry, argmin,
    residual update, round by round) on slices of 1024 tokens x all KV heads of
    the workload's heavy-tailed keys, until the budget is spent."""
    from threadpoolctl import threadpool_limits

    from long_context_attention_commvq_amd import synth
    from oracle import commvq_oracle as O

    cb = synth.codebook(w.seed + 1, w.n_kv_heads, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    n, slices, t_total = 1024, 0, 0.0
    with threadpool_limits(limits=cores):
        while slices == 0 or t_total < budget_s:
            x = synth.kv(w.seed + 800 + slices, n, w.n_kv_heads, w.head_dim, heavy_tail=True)
            t0 = time.perf_counter()
            O.encode(x, cb)
            t_total += time.perf_counter() - t0
            slices += 1
    th = slices * n * w.n_kv_heads
    return {"value": th / t_total, "unit": "token-heads/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{slices} slices of {n} tokens x {w.n_kv_heads} KV heads ({th} token-heads), fp64 NumPy, "
                      f"BLAS threads={cores}; {t_total:.1f} s measured"}


VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9  # CUs x vector lanes per clock per CU x clock


def bench_encode(args):
    """Prefill encoder on the 128K heavy-tailed workload: one step = commvq_encode
    of K then V (131072 tokens x 8 KV heads each), inputs resident in HBM."""
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wname = "llama8b_encode128k_b4_2bit"
    w = synth.WORKLOADS[wname]
    N, H, D = w.context, w.n_kv_heads, w.head_dim
    G = D // w.group_size
    kq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    vq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    print(f"[bench] encode: generating {N} x {H} x {D} K and V", file=sys.stderr, flush=True)
    kx = torch.from_numpy(synth.kv(w.seed + 10, N, H, D, heavy_tail=True)).to(dev)
    vx = torch.from_numpy(synth.kv(w.seed + 11, N, H, D, heavy_tail=True)).to(dev)
    bpt = kq.bytes_per_token
    kc = torch.empty((N, H, bpt), dtype=torch.uint8, device=dev)
    vc = torch.empty((N, H, bpt), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream

    def step():
        _lib.commvq_encode(kq.desc, kx.data_ptr(), N, H * D, kc.data_ptr(), H * bpt, bpt, stream=sid)
        _lib.commvq_encode(vq.desc, vx.data_ptr(), N, H * D, vc.data_ptr(), H * bpt, bpt, stream=sid)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    launch_s = ms_step * 1e-3 / 2  # two equal launches per step (K, V)
    token_heads = N * H
    candidates = token_heads * G * w.n_rounds * w.n_entries  # per launch
    ops = candidates  # the argmin consumes every candidate score in at least one vector operation
    rec = {
        "metric": "prefill encode token-heads/s (K and V, 131072 tokens x 8 KV heads, 2-bit)",
        "value": 2 * token_heads / (ms_step * 1e-3),
        "unit": "token-heads/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 products, fp32 sums", "data": "synthetic",
        "config": {"workload": wname, "tokens": N, "n_kv_heads": H, "head_dim": D, "group_size": w.group_size,
                   "n_entries": w.n_entries, "n_rounds": w.n_rounds, "heavy_tail": True,
                   "step": "commvq_encode of K then V"},
        "roofline": {"bound": "alu", "achieved": ops / launch_s / 1e12, "peak": VALU_PEAK_LANE_OPS / 1e12,
                     "unit": "T lane-ops/s", "frac": ops / launch_s / VALU_PEAK_LANE_OPS,
                     "hbm_GBps": (N * H * D * 2 + N * H * bpt) / launch_s / 1e9,
                     "avg_launch_us": launch_s * 1e6,
                     "work": "1 vector op per (token, head, group, round, entry) candidate score"},
        "cpu_baseline": None if args.no_cpu else encode_cpu_baseline(args.cpu_seconds, w),
    }
    print(json.dumps(rec), flush=True)


def bench_decode_workload(args):
    """One commvq_decode_attention call per step over a whole decode workload
    (every sequence and head), caches of seeded random records rotated over
    layer slices whose total exceeds the Infinity Cache."""
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    B, Hq, H, D, Lmax = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
    kq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    vq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    bpt = kq.bytes_per_token
    lens = (synth.ragged_lengths(w.seed + 5, B, *w.ragged) if w.ragged else np.full(B, Lmax)).astype(np.int32)
    layer_bytes = 2 * B * H * Lmax * bpt
    NL = max(1, min(args.layers, -(-(512 << 20) // layer_bytes)))
    print(f"[bench] {args.workload}: {NL} layer slices of {layer_bytes / 2**20:.0f} MiB", file=sys.stderr, flush=True)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 40)
    caches = [(torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g),
               torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g)) for _ in range(NL)]
    q = torch.from_numpy(synth.queries(w.seed + 42, B, Hq, D)).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    qpos = lens_d - 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, dev)
    rope = _lib.make_rope(w.theta_base)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    sm = 1.0 / math.sqrt(D)

    def call(i):
        kc, vc = caches[i % NL]
        _lib.commvq_decode_attention(kq.desc, vq.desc, rope, q.data_ptr(), qpos.data_ptr(), kc.data_ptr(),
                                     vc.data_ptr(), lens_d.data_ptr(), B, Hq, Lmax, Lmax, sm, out.data_ptr(),
                                     ws.buf.data_ptr(), ws.nbytes, 0, sid)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        call(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    toks = int(lens.sum())
    code_bytes = toks * H * 2 * bpt
    achieved = code_bytes / (ms * 1e-3) / 1e9
    # beside it: dense fp16 attention over keys and values of the same shape
    # (commvq_dense_decode_attention, one fp16 buffer pair per layer slice)
    dense = None
    if D == 128:
        f16_bytes = B * H * Lmax * D * 2
        NLd = max(1, min(args.layers, -(-(512 << 20) // (2 * f16_bytes))))
        kv16 = [(torch.randn((B, H, Lmax, D), dtype=torch.float16, device=dev, generator=g),
                 torch.randn((B, H, Lmax, D), dtype=torch.float16, device=dev, generator=g)) for _ in range(NLd)]
        dws = api.DenseWorkspace(B, Hq, H, D, Lmax, dev)

        def dcall(i):
            k16, v16 = kv16[i % NLd]
            _lib.commvq_dense_decode_attention(rope, q.data_ptr(), qpos.data_ptr(), k16.data_ptr(), v16.data_ptr(),
                                               lens_d.data_ptr(), B, Hq, H, D, Lmax, Lmax, sm, out.data_ptr(),
                                               dws.buf.data_ptr(), dws.nbytes, sid)
        for i in range(args.warmup):
            dcall(i)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            dcall(args.warmup + i)
        stop.record(stream)
        torch.cuda.synchronize()
        dms = start.elapsed_time(stop) / args.steps
        dense = {"ms_per_step": dms, "commvq_over_dense": ms / dms, "layer_slices": NLd,
                 "call": "commvq_dense_decode_attention over fp16 keys and values of the same shape"}
    rec = {
        "metric": METRIC, "value": toks / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "n_q_heads": Hq, "n_kv_heads": H, "head_dim": D,
                   "context": Lmax, "sum_len": toks, "group_size": w.group_size, "n_entries": w.n_entries,
                   "n_rounds": w.n_rounds, "layer_slices": NL,
                   "step": "commvq_decode_attention over every sequence and head"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": code_bytes,
                     "avg_launch_us": ms * 1e3,
                     "kernel": "commvq_decode_attention call: decode kernel, then chunk-merge kernel"},
        "cpu_baseline": None if args.no_cpu else decode_cpu_baseline(args.cpu_seconds, w, lens),
        "dense_fp16_same_shape": dense,
    }
    print(json.dumps(rec), flush=True)


def bench_naive(args):
    """Decode latency of the table/histogram path against the comparison path on
    the same packed caches: 128K positions x 8 KV heads x 32 query heads, 1-bit,
    caches of seeded random records rotated over layer slices beyond the
    Infinity Cache. The comparison path per step: commvq_dequantize_kv into one
    fp16 key/value buffer pair (512 MiB, reused by every slice), then
    commvq_dense_decode_attention. Each variant and each of the comparison
    path's two calls is timed on its own, HIP events on the launch stream."""
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[WORKLOAD]
    B, Hq, H, D, Lmax = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
    kq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    vq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    bpt = kq.bytes_per_token
    NL = max(1, args.layers)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 80)
    caches = [(torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g),
               torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g)) for _ in range(NL)]
    k16 = torch.empty((B, H, Lmax, D), dtype=torch.float16, device=dev)
    v16 = torch.empty_like(k16)
    q = torch.from_numpy(synth.queries(w.seed + 81, B, Hq, D)).to(dev)
    lens = torch.full((B,), Lmax, dtype=torch.int32, device=dev)
    qpos = lens - 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, dev)
    dws = api.DenseWorkspace(B, Hq, H, D, Lmax, dev)
    rope = _lib.make_rope(w.theta_base)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    sm = 1.0 / math.sqrt(D)

    def table(i):
        kc, vc = caches[i % NL]
        _lib.commvq_decode_attention(kq.desc, vq.desc, rope, q.data_ptr(), qpos.data_ptr(), kc.data_ptr(),
                                     vc.data_ptr(), lens.data_ptr(), B, Hq, Lmax, Lmax, sm, out.data_ptr(),
                                     ws.buf.data_ptr(), ws.nbytes, 0, sid)

    def dequant(i):
        kc, vc = caches[i % NL]
        _lib.commvq_dequantize_kv(kq.desc, vq.desc, rope, kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), B, Lmax,
                                  Lmax, k16.data_ptr(), v16.data_ptr(), sid)

    def dense(i):
        _lib.commvq_dense_decode_attention(rope, q.data_ptr(), qpos.data_ptr(), k16.data_ptr(), v16.data_ptr(),
                                           lens.data_ptr(), B, Hq, H, D, Lmax, Lmax, sm, out.data_ptr(),
                                           dws.buf.data_ptr(), dws.nbytes, sid)

    def naive(i):
        dequant(i)
        dense(i)

    def timed(fn, label):
        print(f"[bench] {label}: warmup {args.warmup}, timing {args.steps}", file=sys.stderr, flush=True)
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            fn(args.warmup + i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps * 1e3  # us per call

    t_table = timed(table, "commvq_decode_attention")
    t_naive = timed(naive, "dequantise + dense attention")
    t_deq = timed(dequant, "commvq_dequantize_kv alone")
    t_dense = timed(dense, "commvq_dense_decode_attention alone")
    toks = B * Lmax
    code_bytes = toks * H * 2 * bpt
    f16_bytes = toks * H * 2 * D * 2  # keys and values
    deq_gbs = (code_bytes + f16_bytes) / (t_deq * 1e-6) / 1e9
    dense_gbs = f16_bytes / (t_dense * 1e-6) / 1e9
    rec = {
        "metric": "decode-attn latency per call, CommVQ table/histogram path vs dequantise-to-fp16 + dense attention "
                  "on the same codes (GQA 32q/8kv, 128K ctx, 1-bit)",
        "value": t_naive / t_table, "unit": "x (comparison-path time / CommVQ time)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD + "_full_context", "batch": B, "n_q_heads": Hq, "n_kv_heads": H,
                   "head_dim": D, "context": Lmax, "layer_slices": NL},
        "commvq_us": t_table, "comparison_us": t_naive,
        "comparison_calls": {
            "commvq_dequantize_kv_us": t_deq, "dequantize_GBps": deq_gbs,
            "dequantize_bytes": code_bytes + f16_bytes,
            "commvq_dense_decode_attention_us": t_dense, "dense_GBps": dense_gbs, "dense_bytes": f16_bytes,
            "hbm_peak_GBps": HBM_PEAK_GBS},
        "pages": "6x-9.6x lower decode latency than a naive implementation of the same quantization "
                 "(GPU and kernel configuration not stated)",
        # the comparison path's dominant kernel: the dequantisation (codes in, fp16 keys and values out)
        "roofline": {"bound": "hbm", "achieved": deq_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": deq_gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": code_bytes + f16_bytes,
                     "avg_launch_us": t_deq, "kernel": "dequant_kv_kernel (commvq_dequantize_kv)"},
        "cpu_baseline": None if args.no_cpu else decode_cpu_baseline(args.cpu_seconds, w, np.full(B, Lmax)),
    }
    print(json.dumps(rec), flush=True)


def bench_bitv(args):
    """Decode attention at 128K (B 1, 32 query / 8 KV heads, 1-bit keys g 8,
    Nc' 256, R 1) with the paper's binary value codes, 1024 bits per token over
    the 1024 value scalars (1 bit per scalar): commvq_decode_attention_bitv on
    its fast path and on the generic kernel (COMMVQ_DECODE_EXACT), beside
    commvq_decode_attention on the same keys with residual-codebook values
    through the generic and the fast kernel. Caches of seeded random records
    rotated over layer slices beyond the Infinity Cache; HIP events on the
    launch stream."""
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[WORKLOAD]
    B, Hq, H, D, Lmax = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
    nb = 1024
    kq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    vq = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)).to(dev),
                       w.group_size)
    rows = (torch.randn((nb, H * D), device=dev) / math.sqrt(nb / 2)).to(torch.float16)
    vcb = _lib.make_bit_codebook(rows, nb, H * D)
    bpt = kq.bytes_per_token
    NL = max(1, min(args.layers, 8))
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 90)
    slices = [(torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g),
               torch.randint(0, 256, (B, H, Lmax, bpt), dtype=torch.uint8, device=dev, generator=g),
               torch.randint(0, 256, (B, nb // 128, Lmax, 16), dtype=torch.uint8, device=dev, generator=g))
              for _ in range(NL)]  # (value codes in the library's range-major storage)
    q = torch.from_numpy(synth.queries(w.seed + 91, B, Hq, D)).to(dev)
    lens = torch.full((B,), Lmax, dtype=torch.int32, device=dev)
    qpos = lens - 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, dev)
    rope = _lib.make_rope(w.theta_base)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    sm = 1.0 / math.sqrt(D)

    wsb = api.BitvWorkspace(kq, nb, H * D, B, Hq, Lmax, dev)

    def bitv(flags):
        def call(i):
            kc, _, vb = slices[i % NL]
            _lib.commvq_decode_attention_bitv(kq.desc, vcb, rope, q.data_ptr(), qpos.data_ptr(), kc.data_ptr(),
                                              vb.data_ptr(), lens.data_ptr(), B, Hq, Lmax, Lmax, sm, out.data_ptr(),
                                              wsb.buf.data_ptr(), wsb.nbytes, flags, sid)
        return call

    def residual(flags):
        def call(i):
            kc, vc, _ = slices[i % NL]
            _lib.commvq_decode_attention(kq.desc, vq.desc, rope, q.data_ptr(), qpos.data_ptr(), kc.data_ptr(),
                                         vc.data_ptr(), lens.data_ptr(), B, Hq, Lmax, Lmax, sm, out.data_ptr(),
                                         ws.buf.data_ptr(), ws.nbytes, flags, sid)
        return call

    def timed(fn, label):
        print(f"[bench] {label}", file=sys.stderr, flush=True)
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            fn(args.warmup + i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps * 1e3

    t_bitv = timed(bitv(0), "binary value codes (fast kernel scores, matrix-core value sums)")
    t_bitv_gen = timed(bitv(_lib.COMMVQ_DECODE_EXACT), "binary value codes (generic kernel)")
    t_gen = timed(residual(_lib.COMMVQ_DECODE_EXACT), "residual value codebook (generic kernel)")
    t_fast = timed(residual(0), "residual value codebook (fast kernel)")
    toks = B * Lmax
    bitv_bytes = toks * (H * bpt + nb // 8)  # key records of every KV head + one value code per token
    rec = {
        "metric": "decode-attn cached tokens/s with the paper's binary value codes (GQA 32q/8kv, 128K ctx, 1 bit per "
                  "value scalar)",
        "value": toks / (t_bitv * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_bitv * 1e-3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "llama8b_ctx128k_1bit_binary_values", "batch": B, "n_q_heads": Hq, "n_kv_heads": H,
                   "head_dim": D, "context": Lmax, "value_bits": nb, "layer_slices": NL},
        "calls_us": {"commvq_decode_attention_bitv": t_bitv, "commvq_decode_attention_bitv_exact_generic": t_bitv_gen,
                     "commvq_decode_attention_exact_generic": t_gen,
                     "commvq_decode_attention_fast": t_fast},
        "roofline": {"bound": "hbm", "achieved": bitv_bytes / (t_bitv * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": bitv_bytes / (t_bitv * 1e-6) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": bitv_bytes, "avg_launch_us": t_bitv,
                     "kernel": "commvq_decode_attention_bitv call: fast decode kernel (scores, softmax, weights), "
                               "bitv_values_kernel, bitv_merge_kernel"},
        "cpu_baseline": None if args.no_cpu else decode_cpu_baseline(args.cpu_seconds, w, np.full(B, Lmax),
                                                                     value_bits=nb),
    }
    print(json.dumps(rec), flush=True)


def bench_em(args):
    """One EM iteration of codebook fitting on the prefill workload's key tensor
    (131072 tokens x 8 KV heads, heavy-tailed channels, g = 8, Nc' = 256, a
    two-round codebook): round 0 at temperature 0 (nearest entry) and 1, and
    round 1 at temperature 0 (which first reduces every vector by its round-0
    choice). Each is timed over the steps with HIP events on the launch stream."""
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS["llama8b_encode128k_b4_2bit"]
    N, H, D, g, Nc = w.context, w.n_kv_heads, w.head_dim, w.group_size, w.n_entries
    G = D // g
    x = torch.from_numpy(synth.kv(w.seed + 10, N, H, D, heavy_tail=True)).to(dev)
    q = api.Quantizer(torch.from_numpy(synth.codebook(w.seed + 1, H, D, g, Nc, 2)).to(dev), g)
    work = torch.empty(int(_lib.commvq_em_work_bytes(q.desc)), dtype=torch.uint8, device=dev)
    new = torch.empty_like(q.entries)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    out = {}
    for label, r, T in [("round0_hard", 0, 0.0), ("round0_soft_T1", 0, 1.0), ("round1_hard", 1, 0.0)]:
        def step():
            _lib.commvq_em_step(q.desc, x.data_ptr(), N, H * D, r, T, 0.0, new.data_ptr(), None, work.data_ptr(),
                                work.numel(), sid)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        # vector-ALU work per (vector, group, entry): at temperature 0 the step runs the matrix-core encoder
        # (distances on MFMA; one vector op per candidate score, every round of the codebook searched) and
        # adds each vector to its entry's sums; at temperature > 0 the fitting kernel spends g subtractions, g FMAs
        # and a compare-select per candidate of each round searched, and one exponential and g + 1 FMAs per entry
        # of the fitted round
        per_entry = q.n_rounds if T == 0 else (r + 1) * (2 * g + 1) + (1 + g + 1)
        ops = N * H * G * Nc * per_entry
        out[label] = {"ms": ms, "vectors_per_s": N * H * G / (ms * 1e-3),
                      "achieved_T_lane_ops": ops / (ms * 1e-3) / 1e12,
                      "frac_valu": ops / (ms * 1e-3) / VALU_PEAK_LANE_OPS}
        print(f"[bench] em {label}: {ms:.2f} ms", file=sys.stderr, flush=True)
    main_rec = out["round0_hard"]
    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle sample (em_step)", file=sys.stderr, flush=True)
        cpu = em_cpu_baseline(args.cpu_seconds, x.cpu().numpy(), q.entries.cpu().numpy())
    rec = {
        "metric": "codebook-fitting EM iteration, (vector, group) pairs per second (131072 tokens x 8 KV heads x 16 groups)",
        "value": main_rec["vectors_per_s"], "unit": "vector-groups/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_rec["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "llama8b_encode128k_b4_2bit keys", "tokens": N, "n_kv_heads": H, "head_dim": D,
                   "group_size": g, "n_entries": Nc, "step": "commvq_em_step, round 0, temperature 0"},
        "roofline": {"bound": "alu", "achieved": main_rec["achieved_T_lane_ops"], "peak": VALU_PEAK_LANE_OPS / 1e12,
                     "unit": "T lane-ops/s", "frac": main_rec["frac_valu"],
                     "work": "1 vector op per (vector, group, entry, codebook round) candidate score of the "
                             "matrix-core encoder that makes the nearest-entry choices"},
        "variants": out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def em_cpu_baseline(budget_s: float, x, cb):
    """Time the fp64 oracle's em_step (round 0, temperature 0) on (KV head,
    group) slices of the same key tensor, each over all its vectors, until the
    budget is spent; scale the mean slice time to all slices."""
    from threadpoolctl import threadpool_limits

    from oracle import commvq_oracle as O

    N, H, D = x.shape
    _, G, R, Nc, g = cb.shape
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    done, t_total = 0, 0.0
    with threadpool_limits(limits=cores):
        while done < H * G and (done < 2 or t_total < budget_s):
            h, j = divmod(done, G)
            xs = x[:, h:h + 1, j * g:(j + 1) * g]
            cs = cb[h:h + 1, j:j + 1]
            t0 = time.perf_counter()
            O.em_step(xs, cs, 0, 0.0)
            t_total += time.perf_counter() - t0
            done += 1
    t_all = t_total / done * H * G
    return {"value": N * H * G / t_all, "unit": "vector-groups/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{done} of {H * G} (KV head, group) slices, {N} vectors each, em_step round 0 at "
                      f"temperature 0, fp64 NumPy, BLAS threads={cores}; {t_total:.1f} s measured, scaled to all slices"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the decode path would "
              "shard by KV head or by context chunk, and no multi-GPU launcher is provided", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.encode:
        bench_encode(args)
        return
    if args.naive:
        bench_naive(args)
        return
    if args.em:
        bench_em(args)
        return
    if args.bitv:
        bench_bitv(args)
        return
    if args.workload != WORKLOAD:
        bench_decode_workload(args)
        return
    import torch

    from long_context_attention_commvq_amd import _lib, api, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[WORKLOAD]
    B, Hq, H, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    Lmax = w.context
    kcb = synth.codebook(w.seed + 1, H, D, w.group_size, w.n_entries, w.n_rounds)
    vcb = synth.codebook(w.seed + 2, H, D, w.group_size, w.n_entries, w.n_rounds)
    kq = api.Quantizer(torch.from_numpy(kcb).to(dev), w.group_size)
    vq = api.Quantizer(torch.from_numpy(vcb).to(dev), w.group_size)
    bpt_k, bpt_v = kq.bytes_per_token, vq.bytes_per_token

    # prefill one cache with the GPU encoder, then copy it to every layer slice
    print(f"[bench] prefill {PREFILL} tokens x {H} KV heads", file=sys.stderr, flush=True)
    kcache0 = torch.zeros((B, H, Lmax, bpt_k), dtype=torch.uint8, device=dev)
    vcache0 = torch.zeros((B, H, Lmax, bpt_v), dtype=torch.uint8, device=dev)
    step = 16384
    for t0 in range(0, PREFILL, step):
        n = min(step, PREFILL - t0)
        kx = torch.from_numpy(synth.kv(w.seed + 10 + t0, n, H, D)).to(dev)
        vx = torch.from_numpy(synth.kv(w.seed + 20 + t0, n, H, D)).to(dev)
        api.encode_into_cache(kq, kx, kcache0, 0, t0)
        api.encode_into_cache(vq, vx, vcache0, 0, t0)
    NL = max(1, args.layers)
    kcaches = [kcache0] + [kcache0.clone() for _ in range(NL - 1)]
    vcaches = [vcache0] + [vcache0.clone() for _ in range(NL - 1)]
    torch.cuda.synchronize()

    # per-step inputs: new K/V token, query, device-side positions and lengths
    n_total = args.warmup + args.steps
    knew = torch.from_numpy(synth.kv(w.seed + 30, n_total, H, D)).to(dev).reshape(n_total, 1, H, D)
    vnew = torch.from_numpy(synth.kv(w.seed + 31, n_total, H, D)).to(dev).reshape(n_total, 1, H, D)
    qs = torch.from_numpy(synth.queries(w.seed + 32, n_total, Hq, D)).to(dev).reshape(n_total, 1, Hq, D)
    positions = torch.arange(PREFILL, PREFILL + N_POSITIONS, dtype=torch.int32, device=dev).reshape(-1, 1)
    lens = positions + 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, dev)

    def layer_and_pos(i):
        return i % NL, (i // NL) % N_POSITIONS

    # Each step is one commvq_decode_step call (append the new token's K and V codes
    # at position t, then attend over [0, t]). Its arguments are marshalled once,
    # before timing, so the timed loop issues launches back to back.
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    rope = _lib.make_rope(w.theta_base)
    sm_scale = 1.0 / math.sqrt(D)
    n_total = args.warmup + args.steps
    calls = []
    for i in range(n_total):
        li, t = layer_and_pos(i)
        calls.append((knew[i].data_ptr(), vnew[i].data_ptr(), positions[t].data_ptr(), qs[i].data_ptr(),
                      positions[t].data_ptr(), kcaches[li].data_ptr(), vcaches[li].data_ptr(), lens[t].data_ptr()))

    def run_step(i, stream_id=sid, call_list=None):
        kn, vn, pos, q, qp, kc, vc, ln = (calls if call_list is None else call_list)[i]
        _lib.commvq_decode_step(kq.desc, vq.desc, rope, kn, vn, pos, q, qp, kc, vc, ln, B, Hq, Lmax, Lmax, sm_scale,
                                out, ws.buf, ws.nbytes, 0, stream_id)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    # (1) per-step device times: every step bracketed by HIP events on its stream,
    # all steps queued behind a spin kernel so that no host-issue gap falls inside
    # an interval; median and p10/p90 over the K steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.0e6 + 6.0e4 * args.steps))  # ~1-2 ms of GPU time while the host queues the steps
    evs[0].record(stream)
    for k in range(args.steps):
        run_step(args.warmup + k)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    per_step_us = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(args.steps)])
    eager_ms_step = evs[0].elapsed_time(evs[-1]) / args.steps

    # (2) the timed region: the K steps recorded once in a HIP graph (the library
    # allocates nothing and records no memset, so a decode loop can be captured)
    # and replayed as one launch, bracketed by events and synchronisations
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for k in range(args.steps):
                run_step(args.warmup + k, cap)
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps" + (" (one graph replay)" if graph else " (eager)"), file=sys.stderr,
          flush=True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for k in range(args.steps):
            run_step(args.warmup + k)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # (3) beside it, not as the value: the same steps on layer slice 0 alone, whose
    # codes stay resident in the Infinity Cache (the warm figure)
    warm_us = None
    if graph is not None and NL > 1:
        calls_w = [(c[0], c[1], c[2], c[3], c[4], kcaches[0].data_ptr(), vcaches[0].data_ptr(), c[7]) for c in calls]
        graph_w = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_w):
            cap = torch.cuda.current_stream().cuda_stream
            for k in range(args.steps):
                run_step(args.warmup + k, cap, calls_w)
        torch.cuda.synchronize()
        graph_w.replay()  # (untimed: brings the slice into the caches)
        torch.cuda.synchronize()
        ws0, ws1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ws0.record(stream)
        graph_w.replay()
        ws1.record(stream)
        torch.cuda.synchronize()
        warm_us = ws0.elapsed_time(ws1) / args.steps * 1e3
    # one step is one commvq_decode_step call on `stream`; the roofline is taken
    # over the whole call (the rocprofv3 trace gives its kernels' split)
    dec_avg_ms = ms_step
    # cached tokens per step and packed-code bytes per decode launch
    toks, code_bytes = 0, 0
    for k in range(args.steps):
        _, t = layer_and_pos(args.warmup + k)
        L = PREFILL + t + 1
        toks += B * L
        code_bytes += B * L * H * (bpt_k + bpt_v)
    toks_per_step = toks / args.steps
    bytes_per_launch = code_bytes / args.steps
    achieved = bytes_per_launch / (dec_avg_ms * 1e-3) / 1e9
    print(f"[bench] step {ms_step * 1e3:.2f} us ({'graph replay' if graph else 'eager'}); per-step events: median "
          f"{np.median(per_step_us):.2f} us, p10 {np.percentile(per_step_us, 10):.2f}, p90 "
          f"{np.percentile(per_step_us, 90):.2f}; eager queued {eager_ms_step * 1e3:.2f} us/step; host "
          f"{t_wall / args.steps * 1e6:.1f} us/step" + (f"; warm (one slice) {warm_us:.2f} us/step" if warm_us else ""),
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": toks_per_step / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": B, "n_q_heads": Hq, "n_kv_heads": H, "head_dim": D,
                   "context": Lmax, "prefill": PREFILL, "group_size": w.group_size, "n_entries": w.n_entries,
                   "n_rounds": w.n_rounds, "bits_per_scalar": w.n_rounds * math.log2(w.n_entries) / w.group_size,
                   "layer_slices": NL, "step": "commvq_decode_step: encode+append K and V of 1 token (8 KV heads), then attention"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(), "traffic_unit": "bytes per launch",
                     "kernel": "commvq_decode_step call: fused append + attention kernel, then chunk-merge kernel", "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": dec_avg_ms * 1e3},
        "step_us": {"timed": "graph replay" if graph is not None else "eager", "mean": ms_step * 1e3,
                    "median": float(np.median(per_step_us)), "p10": float(np.percentile(per_step_us, 10)),
                    "p90": float(np.percentile(per_step_us, 90)), "eager_queued_mean": eager_ms_step * 1e3,
                    "per_step_source": "HIP events around each eager call, all calls queued behind a spin kernel",
                    "cache": f"cold: {NL} layer slices rotated ({NL * 2 * B * H * Lmax * bpt_k / 2**20:.0f} MiB of "
                             f"codes, beyond the 256 MB Infinity Cache)" if NL > 1 else "warm: one layer slice",
                    "warm_mean": warm_us,
                    "warm_cache": "the same steps on one layer slice (codes resident in the Infinity Cache); not the value"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
