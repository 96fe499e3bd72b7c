"""Benchmark of the quantized KV-cache decode step on one MI355X.

A step is the whole hot path for one batch: append one new key/value token per
sequence into the full-precision ring and flush (quantize + pack) any block
that leaves the window -- one fused launch -- then decode attention of one
query token per sequence over the packed cache plus the ring: the partial
states of every work unit (the dominant kernel) and their merge. Inputs are
seeded synthetic tensors shaped like the workload and already resident in HBM
when timing starts. To measure HBM rather than the 256 MB Infinity Cache, the
steps rotate over enough copies of the cache that their total exceeds 3x that
size.

Prints one JSON line on stdout; human-readable detail goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sink P]

The default workload is the largest configuration that fits one GPU: the
70B-shaped model at 131,072 tokens, a full 80-layer decode step (GQA 64/8,
d = 128, batch 4, bf16 inputs, INT2 keys and values, G = G_V = 64, R = 128).

With --query-tokens T a step appends T tokens per sequence and runs the
attention of all T of them, causal within the block (kvq_decode_attention_multi:
block-wise prefill or checking T drafted tokens).

With --fp8-blocks W the W most recent quantized blocks of every (sequence, kv
head) are also kept as FP8 records and decode reads them there (FP8 tier).

With --rotate 1|2|3 the key rows, the value rows or both are rotated by a
Walsh-Hadamard transform before they are quantized (and read back through its
inverse by decode).

With --sink P the first P tokens of every sequence stay in full precision
beside the quantized blocks and the ring (attention sink); the decode-partials
time then covers the sink kernel's launch as well.

A multi-layer workload (the 80-layer 70B-shaped one) keeps one cache per layer
resident (27 GB for 80 layers, so no copies are rotated) and times the full
decode step: for each layer in turn, append+flush, decode partials and combine,
all on one stream; `roofline` is then the per-layer decode-partials launch.

The timed steps are launched one by one on one stream (--graph 1 replays them
as HIP graphs instead, a whole step per graph: no faster here, since the
launches already queue back to back); the per-launch kernel timings are taken
on further steps with events around the decode-partials launch.

`value` is the step's algorithmic bytes over its time (effective GB/s of the
whole step); `roofline` is the decode-partials kernel's algorithmic bytes over
its own event-timed duration, against the 8 TB/s HBM peak; `traffic` is the
HBM traffic rocprofv3 counters measured for that kernel (profiles/), reported
only while the kernel sources still hash to the ones measured. `quantize` is
the flush (quantize + pack) rate over the workload's whole quantized prefix:
every token appended into one ring, then one kvq_flush_residual, timed.
"""
from __future__ import annotations

import argparse
import hashlib
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
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def quantized_prefix(S, R, G):
    return G * (max(S - R, 0) // G)


def fp8_record_bytes(w):
    return 2 * w.k_group * w.head_dim + 4 * w.k_group


def partial_bytes(w, lengths, record_bytes, sink=0, fp8_blocks=0):
    """Algorithmic HBM bytes the decode-partials launch must move: packed codes and
    fp16 scale/zero of every quantized token (the FP8 records of the FP8 tier's
    blocks instead), the full-precision ring and sink tokens, q."""
    per_tok = record_bytes / w.k_group
    total = 0.0
    for S in lengths:
        post = max(S - sink, 0)
        Q = quantized_prefix(post, w.residual, w.k_group)
        n8 = min(Q // w.k_group, fp8_blocks)
        total += w.num_kv_heads * ((Q - n8 * w.k_group) * per_tok + n8 * fp8_record_bytes(w)
                                   + (S - Q) * w.head_dim * 2 * 2)
    total += w.batch * w.num_q_heads * w.head_dim * 2
    return total


def out_bytes(w):
    return w.batch * w.num_q_heads * w.head_dim * 4


def append_flush_bytes(w, lengths_before, record_bytes, sink=0, T=1, fp8_blocks=0):
    """Algorithmic bytes of appending T tokens per sequence (read K, V rows, write
    them to the ring or the sink) and of flushing the blocks that leave the window
    (read the block's ring rows, write its record)."""
    row = w.head_dim * 2
    total = 0.0
    for S0 in lengths_before:
        total += T * w.num_kv_heads * 2 * row * 2       # read new k, v; write to the ring
        q0 = quantized_prefix(max(S0 - sink, 0), w.residual, w.k_group)
        q1 = quantized_prefix(max(S0 + T - sink, 0), w.residual, w.k_group)
        blocks = (q1 - q0) // w.k_group
        total += blocks * w.num_kv_heads * (w.k_group * 2 * row + record_bytes)
        total += min(blocks, fp8_blocks) * w.num_kv_heads * fp8_record_bytes(w)   # their FP8 records
    return total


def source_hash() -> str:
    """sha256 over the library sources (kernels and header); names the build the
    counters in profiles/ were taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_append_amd", "csrc")
    paths = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".h", ".hip")))
    paths.append(os.path.join(ROOT, "include", "kvq.h"))
    for p in paths:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode-partials launch from the counter summary in profiles/,
    or None if there is none or the sources changed since it was taken."""
    path = os.path.join(PROFILES, f"decode_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def quantize_rate(w, inp, lengths, dev, reps=5, rotate=0):
    """Full-prefix flush: all of every sequence's tokens appended into a ring
    that holds them, then one kvq_flush_residual quantizes and packs every
    complete block past the window (event-timed, median of `reps`). Bytes are
    the fp16/bf16 rows read plus the records written."""
    import torch
    from quantized_kv_cache_append_amd.cache import cache_for_workload
    S = max(lengths)
    c = cache_for_workload(w, lengths, S, device=dev, rotate=rotate)
    lens = torch.tensor(list(lengths), dtype=torch.int32, device=dev)
    k, v = inp.k[:, :, :S].contiguous(), inp.v[:, :, :S].contiguous()
    ts = []
    for _ in range(reps):
        c.state.zero_()
        c.append(k, v, lens)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        c.flush()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    if c.read_device_error():
        raise SystemExit("device error word set by the quantize measurement")
    q_tok = sum(quantized_prefix(s, w.residual, w.k_group) for s in lengths) * w.num_kv_heads
    nbytes = q_tok * w.head_dim * 2 * 2 + (q_tok // w.k_group) * c.record_bytes
    t = sorted(ts)[len(ts) // 2]
    del c, k, v
    torch.cuda.empty_cache()
    gbps = nbytes / t / 1e9
    return {"value": round(gbps, 1), "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "us_per_flush": round(t * 1e6, 1), "bytes": int(nbytes), "kernel": "flush_kernel",
            "sample": f"one flush of every pair's whole quantized prefix ({q_tok} token-heads), median of {reps}"}


# (query rows per kv head, key bits, value bits, G, G_V, dtype) of the matrix-core
# kernel's instantiations (csrc/decode_fast_dispatch.hip)
FAST_CONFIGS = {(4, 4, 4, 32, 32, "bf16"), (4, 2, 2, 32, 32, "bf16"), (8, 2, 2, 64, 64, "bf16"),
                (6, 4, 2, 16, 32, "bf16"), (4, 2, 2, 32, 32, "f16"), (8, 2, 2, 32, 32, "f16"),
                (8, 2, 2, 32, 32, "bf16"), (8, 4, 4, 32, 32, "bf16")}


def decode_kernel_name(w, T=1, rotate=0) -> str:
    """The decode-partials kernel a workload's configuration runs (T query tokens
    per sequence; the same with a rotated cache)."""
    del rotate
    rows = w.n_g * T
    if w.head_dim != 128:
        return "decode_generic_kernel"
    if rows == 1:
        mx = (w.k_bits, w.v_bits, w.k_group, w.v_group) == (2, 2, 32, 32)
        return "decode_mx_kernel" if mx else "decode_mha_kernel"
    if (rows, w.k_bits, w.v_bits, w.k_group, w.v_group, w.dtype) in FAST_CONFIGS:
        return "decode_fast_kernel"
    return "decode_generic_kernel"


def host_description():
    """The host the oracle runs on: logical CPUs, the ones this process may use,
    and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"host_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model}


def cpu_baseline(w, inp, lengths, budget_s=15.0, sink=0, quant_budget_s=4.0, rotate=0):
    """Time the oracle on the host, one thread: its decode attention on a bounded
    sample of (sequence, kv head) pairs of the same workload (GB/s of the same
    algorithmic bytes), and its quantizer (formula F + packing) over the blocks
    of one pair (GB/s of rows read + records written). Also reports, ungated,
    the fidelity of the quantized cache: the oracle's quantized attention
    against exact attention on the unquantized inputs, over the sampled pairs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kivi
    spec = kivi.CacheSpec(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.k_bits, w.v_bits,
                          w.k_group, w.v_group, w.residual, w.residual + w.k_group, w.dtype, sink=sink,
                          rotate=rotate)
    q = inp.q.float().cpu().numpy()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    done, nbytes, t_used = 0, 0.0, 0.0
    per_tok = kivi.record_bytes(spec) / w.k_group
    n_g = w.num_q_heads // w.num_kv_heads
    diff2 = ref2 = 0.0
    max_abs = 0.0
    with threadpool_limits(limits=1):
        for b, h in pairs:
            S = lengths[b]
            k = inp.k[b, h, :S].float().cpu().numpy()[None, None]
            v = inp.v[b, h, :S].float().cpu().numpy()[None, None]
            qp = q[b:b + 1, h * n_g:(h + 1) * n_g]
            one = kivi.CacheSpec(1, n_g, 1, w.head_dim, w.k_bits, w.v_bits, w.k_group, w.v_group,
                                 w.residual, w.residual + w.k_group, w.dtype, sink=sink, rotate=rotate)
            t0 = time.perf_counter()
            got = kivi.decode_attention(one, qp, k, v, [S])
            t_used += time.perf_counter() - t0
            exact = kivi.exact_attention(one, qp, k, v, [S])
            diff2 += float(np.sum((got - exact) ** 2))
            ref2 += float(np.sum(exact ** 2))
            max_abs = max(max_abs, float(np.max(np.abs(got - exact))))
            Q = quantized_prefix(max(S - sink, 0), w.residual, w.k_group)
            nbytes += Q * per_tok + (S - Q) * w.head_dim * 4 + n_g * w.head_dim * 6
            done += 1
            if t_used > budget_s:
                break
        # the quantizer: formula F and packing of one pair's blocks, as many as fit the budget
        b0, h0 = pairs[0]
        kq = inp.k[b0, h0].float().cpu().numpy()
        vq = inp.v[b0, h0].float().cpu().numpy()
        G = w.k_group
        nblk = quantized_prefix(lengths[b0], w.residual, G) // G
        qt, qblk = 0.0, 0
        for j in range(nblk):
            t0 = time.perf_counter()
            kivi.block_to_bytes(kivi.quantize_block(spec, kq[j * G:(j + 1) * G], vq[j * G:(j + 1) * G]))
            qt += time.perf_counter() - t0
            qblk += 1
            if qt > quant_budget_s:
                break
    qbytes = qblk * (G * w.head_dim * 2 * 2 + kivi.record_bytes(spec))
    res = {"value": nbytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"numpy fp64 oracle decode attention (quantize+dequantize+attend) on {done} of "
                     f"{len(pairs)} (sequence, kv head) pairs of one {w.name} step, {t_used:.1f} s, "
                     f"BLAS limited to 1 thread",
           "blas_threads": 1,
           "quantize": {"value": qbytes / qt / 1e9, "unit": "GB/s",
                        "sample": f"oracle formula F + packing of {qblk} blocks of one (sequence, kv head), "
                                  f"{qt:.1f} s"},
           "fidelity_vs_unquantized": {"rel_l2": (diff2 / ref2) ** 0.5 if ref2 > 0 else 0.0, "max_abs": max_abs,
                                       "pairs": done,
                                       "note": "oracle attention on the quantized cache against exact attention "
                                               "on the unquantized inputs (ungated: the bits-vs-fidelity trade)"}}
    res.update(host_description())
    return res


def copy_probe(mb, dev):
    """Device-to-device copies of a known size, for scaling the HBM traffic
    counters (a profiling aid: runs after the timed region)."""
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 device-to-device copies of {n} bytes")
    del src, dst


def bench_layers(w, args, dev):
    """The full multi-layer decode step: one resident cache per layer; a step
    is, for every layer in turn, append+flush of the new token, decode partials
    and combine, on one stream."""
    import torch

    from quantized_kv_cache_append_amd import workloads as W
    from quantized_kv_cache_append_amd.cache import cache_for_workload

    L = args.layers or w.layers
    lengths0 = W.sequence_lengths(w)
    total_steps = args.warmup + 2 * args.steps
    chunk = 8192
    log(f"[bench] workload {w.name}: {w.description}; {L} layers")
    caches, toks, qs = [], [], []
    t0 = time.perf_counter()
    for layer in range(L):
        inp = W.make_layer(w, device=dev, layer=layer, lengths=lengths0)
        c = cache_for_workload(w, lengths0, chunk, extra_tokens=total_steps + 1, device=dev, rotate=args.rotate)
        c.prefill(inp.k, inp.v, lengths0, chunk)
        # this layer's decode tokens for the steps (distinct per layer and step)
        toks.append([W.new_tokens(w, inp, 1, device=dev, step=layer * 100003 + s) for s in range(4)])
        caches.append(c)
        if layer == 0:
            inp0 = inp   # kept for the quantize rate and the oracle sample
        del inp
        torch.cuda.synchronize()
    rec = caches[0].record_bytes
    log(f"[bench] {L} layer caches of {caches[0].blocks.numel() / 1e6:.1f} MB of records each, "
        f"prefilled in {time.perf_counter() - t0:.1f} s")
    max_len = max(lengths0) + total_steps + 1
    ws = torch.empty(caches[0].workspace_bytes(max_len), dtype=torch.uint8, device=dev)
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)

    def step(i, evs=None):
        for layer, c in enumerate(caches):
            kn, vn, q = toks[layer][i % 4]
            c.append_flush(kn, vn)
            if evs is not None:
                evs[layer][0].record()
            c.decode_partials(q, max_seq_tokens=max_len, workspace=ws)
            if evs is not None:
                evs[layer][1].record()
            c.decode_combine(out=out, max_seq_tokens=max_len, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one HIP graph per token set: the whole step (3 launches per layer) in
        # one submission; every call takes the fixed max_seq_tokens and workspace
        graphs = []
        for k in range(4):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        torch.cuda.synchronize()
        run = lambda i: graphs[i % 4].replay()   # noqa: E731
        log(f"[bench] step captured as a HIP graph of {3 * L} launches")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for j in range(args.steps):
        run(args.warmup + j)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    part_ms = []
    for j in range(args.steps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
        step(args.warmup + args.steps + j, evs)
        torch.cuda.synchronize()
        part_ms += [a.elapsed_time(b) for a, b in evs]
    err = max(c.read_device_error() for c in caches)
    if err:
        raise SystemExit(f"device error word {err} after the timed steps")
    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    # algorithmic bytes: every layer sees the same lengths
    lens = list(lengths0)
    step_bytes, part_bytes = [], []
    for i in range(total_steps):
        after = [s + 1 for s in lens]
        if args.warmup <= i < args.warmup + args.steps:
            step_bytes.append(L * (append_flush_bytes(w, lens, rec) + partial_bytes(w, after, rec) + out_bytes(w)))
        elif i >= args.warmup + args.steps:
            part_bytes.append(partial_bytes(w, after, rec))
        lens = after
    avg_step_bytes = sum(step_bytes) / len(step_bytes)
    avg_part_bytes = sum(part_bytes) / len(part_bytes)
    part_avg_ms = sum(part_ms) / len(part_ms)
    value = avg_step_bytes / (ms_step * 1e-3) / 1e9
    achieved = avg_part_bytes / (part_avg_ms * 1e-3) / 1e9
    log(f"[bench] {ms_step * 1e3:.1f} us/step over {L} layers ({avg_step_bytes / 1e6:.1f} MB) -> {value:.0f} GB/s; "
        f"decode partials per layer {part_avg_ms * 1e3:.1f} us (x{L} = {part_avg_ms * L:.2f} ms), "
        f"{avg_part_bytes / 1e6:.1f} MB -> {achieved:.0f} GB/s ({achieved / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s); "
        f"sources {source_hash()}")
    traffic = measured_traffic(w.name)
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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "hip_graph": bool(args.graph), "batch": w.batch,
                   "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": max(lengths0),
                   "input_dtype": w.dtype, "k_bits": w.k_bits, "v_bits": w.v_bits, "k_group": w.k_group,
                   "v_group": w.v_group, "residual": w.residual, "paged": w.paged, "rotate": args.rotate,
                   "cache_copies_rotated": 1},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": decode_kernel_name(w, 1, args.rotate), "us_per_launch": round(part_avg_ms * 1e3, 2),
                     "bytes_per_launch": int(avg_part_bytes), "launches_per_step": L},
        "quantize": None,
        "cpu_baseline": None,
    }
    del caches, ws
    torch.cuda.empty_cache()
    result["quantize"] = quantize_rate(w, inp0, lengths0, dev, rotate=args.rotate)
    result["quantize"]["sample"] += " (one layer)"
    log(f"[bench] quantize (one layer): full-prefix flush {result['quantize']['us_per_flush']:.1f} us, "
        f"{result['quantize']['bytes'] / 1e6:.1f} MB -> {result['quantize']['value']:.0f} GB/s")
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, inp0, list(lengths0), rotate=args.rotate)
        cb["sample"] += f"; layer 0 only (a step is {L} such layers)"
        result["cpu_baseline"] = cb
        log(f"[bench] oracle on the host: {cb['value']:.3f} GB/s")
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama-70b-128k-80layer")
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto, > 3x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run device-to-device copies of this many MiB (counter calibration)")
    ap.add_argument("--query-tokens", type=int, default=1,
                    help="tokens per sequence per step, attended causally as one block")
    ap.add_argument("--fp8-blocks", type=int, default=0,
                    help="keep the W most recent quantized blocks also as FP8 records, read by decode")
    ap.add_argument("--layers", type=int, default=0,
                    help="multi-layer workloads: time this many layers instead of all (profiling runs; "
                         "the JSON line's config.layers says how many were timed)")
    ap.add_argument("--rotate", type=int, default=0, choices=(0, 1, 2, 3),
                    help="Walsh-Hadamard pre-rotation of keys (1), values (2) or both (3) before quantization")
    ap.add_argument("--graph", type=int, default=0, choices=(0, 1),
                    help="replay the timed steps as HIP graphs (1) or launch them one by one (0); the graphs "
                         "measured no faster on this path (the launches already queue back to back)")
    ap.add_argument("--sink", type=int, default=0,
                    help="keep the first SINK tokens of every sequence in full precision (attention sink)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no multi-GPU path",
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
    dev = torch.device("cuda:0")
    if w.layers != 1:
        if args.sink or args.query_tokens != 1 or args.fp8_blocks:
            raise SystemExit("--sink, --query-tokens and --fp8-blocks are measured on single-layer workloads")
        return bench_layers(w, args, dev)
    P = args.sink
    W8 = args.fp8_blocks
    T = args.query_tokens
    torch.cuda.set_device(dev)
    lengths0 = W.sequence_lengths(w)
    total_steps = args.warmup + 2 * args.steps
    log(f"[bench] workload {w.name}: {w.description}")

    inp = W.make_layer(w, device=dev, lengths=lengths0)
    chunk = 512
    probe = cache_for_workload(w, lengths0, chunk, extra_tokens=0, device=dev, sink=P, fp8_blocks=W8,
                               rotate=args.rotate)
    rec = probe.record_bytes
    per_copy = probe.blocks.numel() + 2 * probe.k_ring.numel() * 2 + \
        (2 * probe.k_sink.numel() * 2 if probe.k_sink is not None else 0) + \
        (probe.fp8.numel() if probe.fp8 is not None else 0)
    del probe
    copies = args.copies or max(1, math.ceil(3 * MALL_BYTES / per_copy))
    steps_per_copy = (math.ceil(total_steps / copies) + 1) * T
    caches = []
    t_fill = 0.0
    for i in range(copies):
        c = cache_for_workload(w, lengths0, chunk, extra_tokens=steps_per_copy, device=dev, sink=P, fp8_blocks=W8,
                               rotate=args.rotate)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c.prefill(inp.k, inp.v, lengths0, chunk)
        torch.cuda.synchronize()
        t_fill += time.perf_counter() - t0
        caches.append(c)
    log(f"[bench] {copies} cache copies of {per_copy / 1e6:.1f} MB, prefill {t_fill / copies * 1e3:.1f} ms/copy")

    # decode-step inputs, drawn before timing
    pool = 16
    toks = [W.new_tokens(w, inp, T, device=dev, step=s) for s in range(pool)]
    if T > 1:   # a query per new token: [B][H_q][T][d]
        gq = torch.Generator(device=dev).manual_seed(4242)
        toks = [(kn, vn, torch.randn(w.batch, w.num_q_heads, T, w.head_dim, generator=gq, device=dev)
                 .to(w.torch_dtype)) for kn, vn, _ in toks]
    outs = [torch.empty(w.batch, w.num_q_heads, *((T,) if T > 1 else ()), w.head_dim, dtype=torch.float32,
                        device=dev) for _ in caches]
    max_len = max(lengths0) + steps_per_copy
    ws_bytes = max(c.workspace_bytes(max_len) for c in caches)
    if T > 1:
        ws_bytes = max(ws_bytes, binding.kvq_workspace_size_multi(caches[0].cfg, max_len, T))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        c = caches[i % copies]
        kn, vn, q = toks[i % pool]
        c.append_flush(kn, vn)
        if ev is not None:
            ev[0].record()
        if T > 1:
            c.decode_multi(q, out=outs[i % copies], max_seq_tokens=max_len, workspace=ws)
        else:
            c.decode_partials(q, max_seq_tokens=max_len, workspace=ws)
        if ev is not None:
            ev[1].record()
        if T == 1:
            c.decode_combine(out=outs[i % copies], max_seq_tokens=max_len, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one HIP graph per (cache copy, token set) pair of the step sequence
        period = math.lcm(copies, pool)
        graphs = {}
        for j in range(args.steps):
            k = (args.warmup + j) % period
            if k not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(k)
                graphs[k] = g
        torch.cuda.synchronize()
        run = lambda i: graphs[i % period].replay()   # noqa: E731
        log(f"[bench] steps captured as {len(graphs)} HIP graphs")
    # the K timed steps: one event pair around all of them (events between the
    # launches would add their own gaps to the step)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for j in range(args.steps):
        run(args.warmup + j)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    # then K more steps with an event pair around each decode-partials launch,
    # on the stream it runs on, for the kernel's own duration
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for j in range(args.steps):
        step(args.warmup + args.steps + j, evs[j])
    torch.cuda.synchronize()
    err = max(c.read_device_error() for c in caches)
    if err:
        raise SystemExit(f"device error word {err} after the timed steps")

    # algorithmic bytes of every step, from the lengths each launch saw
    lens = [list(lengths0) for _ in caches]
    step_bytes, part_bytes = [], []
    for i in range(total_steps):
        ci = i % copies
        before = lens[ci]
        after = [s + T for s in before]
        # the T-token block reads T query rows and, when T > 1, writes its T output rows in the timed window
        q_extra = (T - 1) * w.batch * w.num_q_heads * w.head_dim * 2
        if args.warmup <= i < args.warmup + args.steps:
            step_bytes.append(append_flush_bytes(w, before, rec, P, T, W8) + partial_bytes(w, after, rec, P, W8)
                              + q_extra + T * out_bytes(w))
        elif i >= args.warmup + args.steps:
            part_bytes.append(partial_bytes(w, after, rec, P, W8) + (q_extra + T * out_bytes(w) if T > 1 else 0))
        lens[ci] = after

    ms_step = ms_total / args.steps
    part_ms = [a.elapsed_time(b) for a, b in evs]
    part_avg_ms = sum(part_ms) / len(part_ms)
    avg_step_bytes = sum(step_bytes) / len(step_bytes)
    avg_part_bytes = sum(part_bytes) / len(part_bytes)
    value = avg_step_bytes / (ms_step * 1e-3) / 1e9
    achieved = avg_part_bytes / (part_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    log(f"[bench] {ms_step * 1e3:.1f} us/step ({avg_step_bytes / 1e6:.1f} MB) -> {value:.0f} GB/s; "
        f"decode partials {part_avg_ms * 1e3:.1f} us, {avg_part_bytes / 1e6:.1f} MB -> {achieved:.0f} GB/s "
        f"({achieved / PEAK_HBM_GBPS * 100:.1f}% of 8 TB/s); sources {source_hash()}")

    if args.copy_probe_mb > 0:
        copy_probe(args.copy_probe_mb, dev)

    kernel = decode_kernel_name(w, T, args.rotate)
    if T > 1:   # the multi-token call's window holds its combine launch too
        kernel += "+combine_kernel"
        log(f"[bench] {T} query tokens per sequence per step (causal block); the decode time covers {kernel}")
    if W8 > 0:   # the partials window then holds the FP8 tier's launch too
        kernel = "fp8_kernel+" + kernel
        log(f"[bench] FP8 tier of {W8} blocks: the decode-partials time covers the FP8 kernel too")
    if P > 0:   # and the sink kernel's
        kernel = "sink_kernel+" + kernel
        log(f"[bench] sink of {P} tokens: the decode-partials time covers the sink kernel too")
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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": max(lengths0),
                   "input_dtype": w.dtype, "k_bits": w.k_bits, "v_bits": w.v_bits, "k_group": w.k_group,
                   "v_group": w.v_group, "residual": w.residual, "paged": w.paged, "sink": P, "query_tokens": T,
                   "fp8_blocks": W8, "rotate": args.rotate, "hip_graph": bool(args.graph),
                   "cache_copies_rotated": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": kernel, "us_per_launch": round(part_avg_ms * 1e3, 2),
                     "bytes_per_launch": int(avg_part_bytes)},
        "quantize": None,
        "cpu_baseline": None,
    }
    result["quantize"] = quantize_rate(w, inp, lengths0, dev, rotate=args.rotate)
    log(f"[bench] quantize: full-prefix flush {result['quantize']['us_per_flush']:.1f} us, "
        f"{result['quantize']['bytes'] / 1e6:.1f} MB -> {result['quantize']['value']:.0f} GB/s")
    if not args.no_cpu_baseline and T > 1:
        log("[bench] the oracle baseline times single-token decode; skipped for --query-tokens > 1")
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, [s + 0 for s in lengths0], sink=P, rotate=args.rotate)
        log(f"[bench] oracle on the host: {result['cpu_baseline']['value']:.3f} GB/s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
