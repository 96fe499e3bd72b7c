"""Host-side checks of bench.py's measurement bookkeeping: the algorithmic
bytes it divides by, and the name of the kernel it reports."""
import importlib.util
import os
import re

from quantized_kv_cache_append_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_of_the_llama2_layer():
    # 8 x 32 pairs of 3968 INT2 tokens (96 B each) and 128 fp16 window tokens
    # (512 B each), the fp16 query and the fp32 output: 114,491,392 bytes
    b = _bench()
    w = W.WORKLOADS["llama2-7b-layer"]
    rec = 96 * w.k_group
    total = b.partial_bytes(w, [4096] * 8, rec) + b.out_bytes(w)
    assert total == 8 * 32 * (3968 * 96 + 128 * 512) + 8 * 32 * 128 * 2 + 8 * 32 * 128 * 4 == 114_491_392


def test_decode_bytes_with_a_sink_and_an_fp8_tier():
    b = _bench()
    w = W.WORKLOADS["llama2-7b-layer"]
    rec = 96 * w.k_group
    # sink of 4: 4092 tokens after it -> 3936 quantized, 156 in the window; 4 more fp16 rows
    with_sink = b.partial_bytes(w, [4096], rec, sink=4)
    assert with_sink == 32 * (3936 * 96 + (4096 - 3936) * 512) + 8 * 32 * 128 * 2
    # FP8 tier of 4 blocks: 128 of the 3968 quantized tokens read at 260 B instead of 96 B
    tier = b.partial_bytes(w, [4096], rec, fp8_blocks=4)
    assert tier == 32 * (3840 * 96 + 4 * (2 * 32 * 128 + 4 * 32) + 128 * 512) + 8 * 32 * 128 * 2


def test_append_flush_bytes_count_the_flushed_block():
    b = _bench()
    w = W.WORKLOADS["llama2-7b-layer"]
    rec = 96 * w.k_group
    row = 128 * 2
    # 4096 -> 4097 tokens: one token appended, no block completes (Q stays 3968)
    assert b.append_flush_bytes(w, [4096], rec) == 32 * 2 * row * 2
    # 4127 -> 4128: Q goes 3968 -> 4000, the block of tokens 3968..3999 leaves the window
    assert b.append_flush_bytes(w, [4127], rec) == 32 * 2 * row * 2 + 32 * (32 * 2 * row + rec)


def test_kernel_names_follow_the_dispatch_table():
    b = _bench()
    src = open(os.path.join(ROOT, "quantized_kv_cache_append_amd", "csrc", "decode_fast_dispatch.hip")).read()
    entries = set()
    for m in re.finditer(r"KVQ_MFMA\((\d+), (\d+), (\d+), (\d+), (\d+), (true|false)\)", src):
        ng, kb, vb, g, gv, bf = m.groups()
        if "#define" in src[max(0, m.start() - 40):m.start()]:
            continue
        entries.add((int(ng), int(kb), int(vb), int(g), int(gv), "bf16" if bf == "true" else "f16"))
    assert entries == b.FAST_CONFIGS
    assert b.decode_kernel_name(W.WORKLOADS["llama2-7b-layer"]) == "decode_mx_kernel"
    assert b.decode_kernel_name(W.WORKLOADS["llama2-7b-layer"], T=4) == "decode_fast_kernel"
    assert b.decode_kernel_name(W.WORKLOADS["llama3-8b-gqa-int2"]) == "decode_fast_kernel"
    assert b.decode_kernel_name(W.WORKLOADS["tiny"]) == "decode_generic_kernel"


def test_more_than_one_gpu_is_refused_with_a_message():
    # the bench measures one GPU; --gpus N > 1 exits before touching torch or a GPU
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_the_default_workload_is_the_80_layer_70b_step():
    b = _bench()
    import inspect
    src = inspect.getsource(b.main)
    assert re.search(r'"--workload", default="llama-70b-128k-80layer"', src)
    assert W.WORKLOADS["llama-70b-128k-80layer"].layers == 80
