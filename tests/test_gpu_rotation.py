"""The Walsh-Hadamard pre-rotation on the GPU (patricehuetz.fr, "TurboQuant : les
cinq innovations", innovation 1): records of rotated key and/or value rows
bit for bit against the oracle (the flush's fp32 butterflies follow the oracle's
order), and decode attention within max-abs 2e-3 / relative L2 1e-3 of the fp64
oracle on the same dequantized cache, for every decode path that takes
rotated caches: the GQA matrix-core kernel (dense and paged, G = 32 and the
70B shape's G = 64), the block-scaled multi-head kernel (fp16 and bf16 INT2),
the multi-head vector kernel (INT4) and the generic kernel (d = 64); steps
across flushes of the fused append+flush, a sink, and a multi-token query."""
import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides, lengths, rotate)
    "gqa-int2-both": ("llama3-8b-gqa-int2", dict(batch=3, num_q_heads=16, num_kv_heads=4), [700, 1500, 33], 3),
    "gqa-int4-keys": ("llama3-8b-gqa-int4", dict(batch=2, num_q_heads=8, num_kv_heads=2), [1100, 400], 1),
    "gqa-int2-values": ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2), [900, 260], 2),
    "70b-g64-both": ("llama-70b-128k-80layer", dict(batch=2, num_q_heads=16, num_kv_heads=2, layers=1),
                     [2100, 500], 3),
    "mha-fp16-both": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4), [1000, 300], 3),
    "mha-bf16-keys": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, dtype="bf16"), [1000, 300], 1),
    "mha-int4-both": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, k_bits=4, v_bits=4),
                      [800, 260], 3),
    "paged-ng6-both": ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2), [37, 300, 1111], 3),
    "tiny-d64-both": ("tiny", dict(batch=2), [512, 200], 3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_rotated_records_and_decode_match_the_oracle(name):
    wname, over, lengths, rot = CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    print(f"[rotation {name}] rotate={rot} lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=61, lengths=lengths)
    cache = make_cache(w, lengths, 128, rotate=rot)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 128)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    spec = spec_of(w, cache.cfg.res_capacity, rotate=rot)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    n = check_records(cache, spec, k_np, v_np, lengths, pairs)
    assert n > 0
    max_abs, rel = check_decode(out, spec, to_np(inp.q), k_np, v_np, lengths, scale=default_scale(w.head_dim))
    # the records do differ from the unrotated ones (first block of the longest sequence)
    b = int(np.argmax(lengths))
    plain = kivi.expected_blocks(spec_of(w, cache.cfg.res_capacity), k_np[b, 0], v_np[b, 0], lengths[b])
    assert not np.array_equal(cache.record(b, 0, 0).cpu().numpy(), plain[0])
    print(f"[rotation {name}] {n} records bit-exact; decode max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)


@pytest.mark.parametrize("wname,over", [
    ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2)),
    ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2)),
])
def test_rotated_decode_steps_across_flushes(wname, over):
    w = W.WORKLOADS[wname].replace(**over)
    lengths = [300, 170]
    steps = 40
    full = [s + steps for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=62, lengths=full)
    cache = make_cache(w, lengths, 64, extra_tokens=steps, rotate=3)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    spec = spec_of(w, cache.cfg.res_capacity, rotate=3)
    cur = list(lengths)
    for st in range(steps):
        kn = torch.stack([inp.k[b, :, cur[b]:cur[b] + 1] for b in range(w.batch)]).contiguous()
        vn = torch.stack([inp.v[b, :, cur[b]:cur[b] + 1] for b in range(w.batch)]).contiguous()
        cache.append_flush(kn.cuda(), vn.cuda())
        cur = [s + 1 for s in cur]
        if st in (0, 17, steps - 1):
            out = cache.decode(inp.q.cuda())
            check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), cur, scale=default_scale(w.head_dim))
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), cur, pairs)


def test_rotation_with_a_sink():
    w = W.WORKLOADS["llama3-8b-gqa-int2"].replace(batch=2, num_q_heads=8, num_kv_heads=2)
    lengths, P = [800, 90], 5
    inp = W.make_layer(w, device="cpu", seed=63, lengths=lengths)
    cache = make_cache(w, lengths, 128, sink=P, rotate=3)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 128)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    spec = spec_of(w, cache.cfg.res_capacity, sink=P, rotate=3)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, pairs)
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths, scale=default_scale(w.head_dim))


def test_rotation_with_a_multi_token_query():
    w = W.WORKLOADS["llama3-8b-gqa-int2"].replace(batch=2, num_q_heads=8, num_kv_heads=2)
    lengths, T = [900, 300], 2
    inp = W.make_layer(w, device="cpu", seed=64, lengths=lengths)
    cache = make_cache(w, lengths, 128, rotate=3)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 128)
    g = torch.Generator().manual_seed(65)
    q = torch.randn(w.batch, w.num_q_heads, T, w.head_dim, generator=g).to(w.torch_dtype)
    out = cache.decode_multi(q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    spec = spec_of(w, cache.cfg.res_capacity, rotate=3)
    ref = kivi.decode_attention_multi(spec, to_np(q), to_np(inp.k), to_np(inp.v), lengths, T,
                                      scale=default_scale(w.head_dim))
    got = out.double().cpu().numpy()
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert float(err.max()) <= 2e-3 and rel <= 1e-3, (float(err.max()), rel)
