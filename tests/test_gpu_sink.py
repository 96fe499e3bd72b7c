"""Parity of the attention-sink prefix (the first P tokens of every sequence
kept in full precision) with the CPU oracle, through the C ABI, on every
decode path: the block-scaled multi-head kernel (INT2), the vector multi-head
kernel (INT4), the GQA matrix-core kernel (dense, paged, G = 64) and the
generic kernel (d = 64). Records, ring, sink rows and lengths bit-exact;
attention within the usual max-abs 2e-3 / rel-L2 1e-3."""
import pytest
import torch

from quantized_kv_cache_append_amd import binding as B
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu

SINK_CASES = {
    # name: (workload, overrides, lengths or None, chunk, sink tokens P)
    "mha-int2": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4), [2, 700, 1500], 256, 4),
    "mha-int4": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, k_bits=4, v_bits=4), [1000, 64],
                 256, 64),
    "gqa-int2": ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2), [2100, 9], 512, 16),
    "70b-g64": ("llama-70b-128k-80layer", dict(batch=1, num_q_heads=16, num_kv_heads=2, layers=1), [3000], 512, 4),
    "paged": ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2), [37, 300, 1111], 256, 5),
    "tiny-d64": ("tiny", {}, None, 128, 3),
    # a sink longer than every sequence: nothing is quantized, nothing is in the ring
    "covers-all": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [100, 250], 256, 256),
}


def _run(name, seed=0):
    wname, over, lengths, chunk, P = SINK_CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    if lengths is None:
        lengths = W.sequence_lengths(w, seed)
    print(f"[sink case {name}] P={P} lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=seed, lengths=lengths)
    cache = make_cache(w, lengths, chunk, sink=P)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, chunk)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    return w, cache, inp, lengths, out, spec_of(w, cache.cfg.res_capacity, sink=P)


@pytest.mark.parametrize("name", list(SINK_CASES))
def test_sink_records_ring_and_sink_bit_exact(name):
    w, cache, inp, lengths, _, spec = _run(name)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, pairs)


@pytest.mark.parametrize("name", list(SINK_CASES))
def test_sink_decode_matches_oracle(name):
    w, cache, inp, lengths, out, spec = _run(name)
    max_abs, rel = check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths,
                                scale=default_scale(w.head_dim))
    print(f"[sink case {name}] max_abs={max_abs:.2e} rel_l2={rel:.2e}")


@pytest.mark.parametrize("name", ["mha-int2", "gqa-int2"])
def test_sink_two_phase_decode_equals_one_call(name):
    w, cache, inp, lengths, out, spec = _run(name)
    cache.decode_partials(inp.q.cuda())
    out2 = cache.decode_combine()
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("fused", [False, True])
def test_sink_decode_steps_across_the_sink_and_a_flush(fused):
    """Decode steps of one token each: one sequence fills its sink (2 -> 14
    tokens with P = 4), another crosses its first flush (P + R + G = 84)."""
    w = W.WORKLOADS["ragged-paged"].replace(batch=3, num_q_heads=12, num_kv_heads=2)
    P, steps = 4, 12
    lengths = [2, 3, 78]
    full = [s + steps for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=9, lengths=full)
    cache = make_cache(w, lengths, 64, extra_tokens=steps, sink=P)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    spec = spec_of(w, cache.cfg.res_capacity, sink=P)
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    for st in range(steps):
        idx = [s + st for s in lengths]
        kn = torch.stack([inp.k[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]).contiguous()
        vn = torch.stack([inp.v[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]).contiguous()
        if fused:
            cache.append_flush(kn.cuda(), vn.cuda())
        else:
            cache.append(kn.cuda(), vn.cuda())
            cache.flush()
        q = W.new_tokens(w, inp, 1, device="cpu", seed=9, step=st)[2]
        out = cache.decode(q.cuda())
        cur = [s + st + 1 for s in lengths]
        if st in (0, 1, 2, 5, 6, 7, steps - 1):
            check_decode(out, spec, to_np(q), k_np, v_np, cur, scale=default_scale(w.head_dim))
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, k_np, v_np, full, pairs)


def test_sink_multi_token_append_straddles_the_sink():
    # one append whose rows go partly to the sink and partly to the ring
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=2, num_q_heads=2, num_kv_heads=2)
    P = 10
    lengths = [3, 0]
    inp = W.make_layer(w, device="cpu", seed=10, lengths=[40, 40])
    cache = make_cache(w, [40, 40], 64, sink=P)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    counts = torch.tensor([30, 25], dtype=torch.int32)
    kn = torch.stack([inp.k[0, :, 3:33], inp.k[1, :, 0:30]]).contiguous()
    vn = torch.stack([inp.v[0, :, 3:33], inp.v[1, :, 0:30]]).contiguous()
    cache.append(kn.cuda(), vn.cuda(), counts.cuda())
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    cur = [33, 25]
    spec = spec_of(w, cache.cfg.res_capacity, sink=P)
    pairs = [(b, h) for b in range(2) for h in range(2)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), cur, pairs)
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), cur, scale=default_scale(w.head_dim))


def test_sink_ring_overflow_counts_tokens_after_the_sink():
    # ring capacity R + G - 1 + 32 = 191: with a sink of 20, 211 rows fit a
    # fresh sequence in one append; 212 can never fit and are refused on the host
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=1, num_q_heads=1, num_kv_heads=1)
    cache = make_cache(w, [400], 32, sink=20)
    kk = torch.zeros(1, 1, 211, 128, dtype=torch.float16, device="cuda")
    cache.append(kk, kk)
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0 and cache.lengths() == ([0], [211])
    with pytest.raises(B.KVQError) as e:
        big = torch.zeros(1, 1, 212, 128, dtype=torch.float16, device="cuda")
        cache.append(big, big)
    assert e.value.status == B.KVQ_ERR_CAPACITY
    # 150 rows leave 130 in the ring after the sink's 20: 61 more fit, 62 overflow on the device
    for n2, full in ((61, False), (62, True)):
        cache = make_cache(w, [400], 32, sink=20)
        first = torch.zeros(1, 1, 150, 128, dtype=torch.float16, device="cuda")
        second = torch.zeros(1, 1, n2, 128, dtype=torch.float16, device="cuda")
        cache.append(first, first)
        cache.append(second, second)
        torch.cuda.synchronize()
        assert bool(cache.read_device_error() & 1) == full
        assert cache.lengths() == ([0], [150 if full else 150 + n2])
