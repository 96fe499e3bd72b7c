"""Benchmark of one decode step of the quantized KV-cache hot path on one MI355X.

A step is the whole path for one batch: append one new key/value token per
sequence into the full-precision ring, flush (quantize + pack any block that
leaves the window), and decode attention of one query token per sequence over
the packed cache plus the ring. Inputs are seeded synthetic tensors shaped like
the workload and already resident in HBM when timing starts. To measure HBM
rather than the 256 MB Infinity Cache, the step rotates over enough copies of
the cache that their total exceeds 3x that size.

Prints one JSON line on stdout; human-readable detail goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-KV decode attention: effective HBM GB/s & % of peak; µs/step"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def quantized_prefix(S, R, G):
    return G * (max(S - R, 0) // G)


def decode_bytes(w, lengths, record_bytes):
    """Algorithmic HBM bytes of one decode-attention launch: packed codes and fp16
    scale/zero of every quantized token, the full-precision ring tokens, q and out."""
    per_tok = record_bytes / w.k_group
    total = 0.0
    for S in lengths:
        Q = quantized_prefix(S, w.residual, w.k_group)
        total += w.num_kv_heads * (Q * per_tok + (S - Q) * w.head_dim * 2 * 2)
    total += w.batch * w.num_q_heads * w.head_dim * (2 + 4)
    return total


def cpu_baseline(w, inp, lengths, budget_s=15.0):
    """Time the oracle's decode attention on a bounded sample of (sequence, kv head)
    pairs of the same workload; returns GB/s of the same algorithmic bytes."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kivi
    spec = kivi.CacheSpec(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                          w.k_group, w.v_group, w.residual, w.residual + w.k_group, w.dtype)
    q = inp.q.float().cpu().numpy()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    done, nbytes, t_used = 0, 0.0, 0.0
    per_tok = kivi.record_bytes(spec) / w.k_group
    with threadpool_limits(limits=1):
        for b, h in pairs:
            k = {(b, h): inp.k[b, h].float().cpu().numpy()}
            v = {(b, h): inp.v[b, h].float().cpu().numpy()}

            class _P:
                def __init__(s, d):
                    s.d = d

                def __getitem__(s, key):
                    return s.d[(key[0], key[1])]
            t0 = time.perf_counter()
            kivi.decode_attention(spec, q, _P(k), _P(v), lengths, pairs=[(b, h)])
            t_used += time.perf_counter() - t0
            S = lengths[b]
            Q = quantized_prefix(S, w.residual, w.k_group)
            nbytes += Q * per_tok + (S - Q) * w.head_dim * 4 + w.num_q_heads // w.num_kv_heads * w.head_dim * 6
            done += 1
            if t_used > budget_s:
                break
    return {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"numpy fp64 oracle decode attention (quantize+dequantize+attend) on {done} of "
                      f"{len(pairs)} (sequence, kv head) pairs of one {w.name} step, {t_used:.1f} s, "
                      f"BLAS limited to 1 thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2-7b-layer")
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto, > 3x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_kv_cache_append_amd import binding
    from quantized_kv_cache_append_amd import workloads as W
    from quantized_kv_cache_append_amd.cache import cache_for_workload

    if not binding.library_path_exists():
        import __graft_entry__
        __graft_entry__.build()
    binding.load()

    w = W.WORKLOADS[args.workload]
    if w.layers != 1:
        raise SystemExit("multi-layer workloads are run per layer: pick a single-layer workload")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lengths0 = W.sequence_lengths(w)
    total_steps = args.warmup + args.steps
    log(f"[bench] workload {w.name}: {w.description}")

    inp = W.make_layer(w, device=dev, lengths=lengths0)
    chunk = 512
    probe = cache_for_workload(w, lengths0, chunk, extra_tokens=0, device=dev)
    rec = probe.record_bytes
    per_copy = probe.blocks.numel() + 2 * probe.k_ring.numel() * 2
    del probe
    copies = args.copies or max(1, math.ceil(3 * MALL_BYTES / per_copy))
    steps_per_copy = math.ceil(total_steps / copies) + 1
    caches = []
    t_fill = 0.0
    for i in range(copies):
        c = cache_for_workload(w, lengths0, chunk, extra_tokens=steps_per_copy, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c.prefill(inp.k, inp.v, lengths0, chunk)
        torch.cuda.synchronize()
        t_fill += time.perf_counter() - t0
        caches.append(c)
    log(f"[bench] {copies} cache copies of {per_copy / 1e6:.1f} MB, prefill {t_fill / copies * 1e3:.1f} ms/copy")

    # decode-step inputs, drawn before timing
    pool = 16
    toks = [W.new_tokens(w, inp, 1, device=dev, step=s) for s in range(pool)]
    outs = [torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev) for _ in caches]
    max_len = max(lengths0) + steps_per_copy
    ws_bytes = max(c.workspace_bytes(max_len) for c in caches)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    lens = [list(lengths0) for _ in caches]

    def step(i, ev=None):
        ci = i % copies
        c = caches[ci]
        kn, vn, q = toks[i % pool]
        c.append_flush(kn, vn)
        lens[ci] = [s + 1 for s in lens[ci]]
        if ev is not None:
            ev[0].record()
        c.decode(q, out=outs[ci], max_seq_tokens=max_len, workspace=ws)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_bytes = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for j in range(args.steps):
        i = args.warmup + j
        step(i, evs[j])
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    # bytes of each timed decode launch, from the lengths it saw
    lens_replay = [list(lengths0) for _ in caches]
    for i in range(total_steps):
        ci = i % copies
        lens_replay[ci] = [s + 1 for s in lens_replay[ci]]
        if i >= args.warmup:
            step_bytes.append(decode_bytes(w, lens_replay[ci], rec))
    err = max(c.read_device_error() for c in caches)
    if err:
        raise SystemExit(f"device error word {err} after the timed steps")

    ms_step = ms_total / args.steps
    avg_bytes = sum(step_bytes) / len(step_bytes)
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    value = avg_bytes / (ms_step * 1e-3) / 1e9
    achieved = avg_bytes / (dec_avg_ms * 1e-3) / 1e9
    log(f"[bench] {ms_step * 1e3:.1f} us/step, decode launch {dec_avg_ms * 1e3:.1f} us, "
        f"{avg_bytes / 1e6:.1f} MB/step -> step {value:.0f} GB/s, decode {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s)")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": max(lengths0),
                   "input_dtype": w.dtype, "k_bits": w.k_bits, "v_bits": w.v_bits, "k_group": w.k_group,
                   "v_group": w.v_group, "residual": w.residual, "paged": w.paged,
                   "cache_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "kernel": "kvq_decode_attention (split decode + combine)",
                     "us_per_launch": round(dec_avg_ms * 1e3, 2),
                     "bytes_per_launch": int(avg_bytes)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, [s + 0 for s in lengths0])
        log(f"[bench] oracle on the host: {result['cpu_baseline']['value']:.3f} GB/s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
