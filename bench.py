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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=16, help="layer slices rotated over (caches > MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


def cpu_baseline(budget_s: float):
    """Time the fp64 oracle (unpack -> dequantise -> RoPE -> dense softmax) on
    one KV head (its 4 query heads) of a step at full context, repeated over
    heads until the budget is spent, scaled to the 8-head step."""
    from threadpoolctl import threadpool_limits

    from long_context_attention_commvq_amd import synth
    from oracle import commvq_oracle as O

    w = synth.WORKLOADS[WORKLOAD]
    L = PREFILL + 1
    G = w.head_dim // w.group_size
    kcb = synth.codebook(w.seed + 1, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    vcb = synth.codebook(w.seed + 2, 1, w.head_dim, w.group_size, w.n_entries, w.n_rounds)
    rep = w.n_q_heads // w.n_kv_heads
    units, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while units < w.n_kv_heads and (units == 0 or t_total < budget_s):
            kc = synth.random_codes(w.seed + 100 + units, (L, 1, w.n_rounds, G), w.n_entries)
            vc = synth.random_codes(w.seed + 200 + units, (L, 1, w.n_rounds, G), w.n_entries)
            kp = O.pack_codes(kc, w.n_entries).transpose(1, 0, 2)[None]
            vp = O.pack_codes(vc, w.n_entries).transpose(1, 0, 2)[None]
            q = synth.queries(w.seed + 300 + units, 1, rep, w.head_dim)
            t0 = time.perf_counter()
            O.decode_attention_from_packed(q, np.array([L - 1]), kp, vp, np.array([L]), kcb, vcb, w.theta_base)
            t_total += time.perf_counter() - t0
            units += 1
    t_step = t_total / units * w.n_kv_heads
    return {"value": L / t_step, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} of 8 KV heads (4 query heads each) at L={L}, fp64 NumPy, 1 thread; "
                      f"{t_total:.1f} s measured, scaled x{w.n_kv_heads / units:.1f} to one 8-head step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              "(the path shards by KV head or context chunk, see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_attention_commvq_amd import api, synth

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
    knew = torch.from_numpy(synth.kv(w.seed + 30, n_total, H, D)).to(dev).reshape(n_total, 1, 1, H, D)
    vnew = torch.from_numpy(synth.kv(w.seed + 31, n_total, H, D)).to(dev).reshape(n_total, 1, 1, H, D)
    qs = torch.from_numpy(synth.queries(w.seed + 32, n_total, Hq, D)).to(dev).reshape(n_total, 1, Hq, D)
    positions = torch.arange(PREFILL, PREFILL + N_POSITIONS, dtype=torch.int32, device=dev).reshape(-1, 1)
    lens = positions + 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = api.DecodeWorkspace(kq, vq, B, Hq, Lmax, dev)

    def layer_and_pos(i):
        return i % NL, (i // NL) % N_POSITIONS

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def run_step(i, timed_idx=None):
        li, t = layer_and_pos(i)
        if timed_idx is not None:
            ev[timed_idx][0].record(stream)
        # append the new token's K and V codes at position t, then attend over [0, t]
        api.decode_step(kq, vq, knew[i][0], vnew[i][0], positions[t], qs[i], positions[t], kcaches[li], vcaches[li],
                        lens[t], Lmax, w.theta_base, out=out, workspace=ws)
        if timed_idx is not None:
            ev[timed_idx][1].record(stream)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        run_step(args.warmup + k, timed_idx=k)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    dec_avg_ms = float(np.mean(dec_ms))
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
    print(f"[bench] step {ms_step * 1e3:.1f} us, decode kernel {dec_avg_ms * 1e3:.1f} us "
          f"(median {np.median(dec_ms) * 1e3:.1f}), wall {t_wall / args.steps * 1e6:.1f} us/step",
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode step (fused append + attention)", "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": dec_avg_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
