"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Packed codes, fp16 scales/zero-points, the ring and the lengths must match
bit for bit; decode attention must be within max-abs 2e-3 and relative L2 1e-3
of the fp64 oracle evaluated on the same dequantized cache. Sizes here are
small enough for the oracle to finish in seconds yet span several blocks,
several splits and a ragged tail; the full workload sizes are covered on
sampled (sequence, kv head) pairs in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from quantized_kv_cache_append_amd import binding as B
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides, lengths or None, chunk)
    "tiny-full": ("tiny", {}, None, 128),
    "llama2-reduced": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4), [1000, 1000], 256),
    "llama3-int4-reduced": ("llama3-8b-gqa-int4", dict(batch=2, num_q_heads=8, num_kv_heads=2), [2100, 2100], 512),
    "llama3-int2-reduced": ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2), [2100, 2100], 512),
    "llama70b-reduced": ("llama-70b-128k-80layer", dict(batch=1, num_q_heads=16, num_kv_heads=2, layers=1),
                         [3000], 512),
    "ragged-paged-reduced": ("ragged-paged", dict(batch=5, num_q_heads=12, num_kv_heads=2),
                             [37, 300, 1111, 2048, 517], 256),
    # the other instantiations of the multi-head paths (one query head per kv
    # head): bf16 and paged INT2, ragged lengths; INT4
    "mha-bf16-paged": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4, dtype="bf16", paged=True),
                       [700, 1500, 2123], 256),
    "mha-f16-paged": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, paged=True), [1000, 1337], 256),
    "mha-bf16-dense": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4, dtype="bf16"),
                       [95, 900, 1800], 256),
    "mha-int4": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, k_bits=4, v_bits=4), [1000, 1000],
                 256),
    # many pairs of very different lengths: the waves' static unit ranges cut
    # across pairs and through runs of one pair's units
    "mha-ragged-many": ("llama2-7b-layer", dict(batch=8, num_q_heads=8, num_kv_heads=8),
                        [33, 160, 191, 500, 1024, 2049, 3000, 4100], 256),
}


def _run_case(name, seed=0):
    wname, over, lengths, chunk = CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    if lengths is None:
        lengths = W.sequence_lengths(w, seed)
    print(f"[case {name}] lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=seed, lengths=lengths)
    cache = make_cache(w, lengths, chunk)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, chunk)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    return w, cache, inp, lengths, out


@pytest.mark.parametrize("name", list(CASES))
def test_records_and_ring_bit_exact(name):
    w, cache, inp, lengths, _ = _run_case(name)
    spec = spec_of(w, cache.cfg.res_capacity)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    n = check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, pairs)
    assert n == sum((max(S - w.residual, 0) // w.k_group) for S in lengths) * w.num_kv_heads


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    w, cache, inp, lengths, out = _run_case(name)
    spec = spec_of(w, cache.cfg.res_capacity)
    max_abs, rel = check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths,
                                scale=default_scale(w.head_dim))
    print(f"[case {name}] max_abs={max_abs:.2e} rel_l2={rel:.2e}")


@pytest.mark.parametrize("name", ["llama3-int2-reduced", "mha-bf16-paged"])
def test_decode_is_deterministic(name):
    w, cache, inp, lengths, out = _run_case(name)
    again = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, again)


@pytest.mark.parametrize("name", ["llama2-reduced", "mha-bf16-paged", "llama3-int2-reduced", "ragged-paged-reduced",
                                  "tiny-full"])
def test_two_phase_decode_equals_one_call(name):
    # kvq_decode_partials + kvq_decode_combine is the same computation as
    # kvq_decode_attention: the unit partition depends only on the lengths
    w, cache, inp, lengths, out = _run_case(name)
    q = inp.q.cuda()
    cache.decode_partials(q)
    out2 = cache.decode_combine()
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("S", [1, 40, 127, 128, 159, 160, 161, 191, 192])
def test_window_boundaries(S):
    # R = 128, G = 32: nothing is quantized until S reaches R + G = 160
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=1, num_q_heads=2, num_kv_heads=2)
    inp = W.make_layer(w, device="cpu", seed=3, lengths=[S])
    cache = make_cache(w, [S], 64)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), [S], 64)
    out = cache.decode(inp.q.cuda())
    spec = spec_of(w, cache.cfg.res_capacity)
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), [S], [(0, 0), (0, 1)])
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), [S], scale=default_scale(w.head_dim))


@pytest.mark.parametrize("wname", ["llama3-8b-gqa-int4", "llama2-7b-layer"])
def test_empty_sequence_in_batch_gives_zero_output(wname):
    over = dict(batch=3, num_q_heads=8, num_kv_heads=2) if wname != "llama2-7b-layer" else \
        dict(batch=3, num_q_heads=2, num_kv_heads=2)
    w = W.WORKLOADS[wname].replace(**over)
    lengths = [500, 0, 300]
    inp = W.make_layer(w, device="cpu", seed=4, lengths=[500, 1, 300])
    cache = make_cache(w, lengths, 128)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 128)
    out = cache.decode(inp.q.cuda())
    assert torch.count_nonzero(out[1]) == 0
    spec = spec_of(w, cache.cfg.res_capacity)
    pairs = [(b, h) for b in (0, 2) for h in range(w.num_kv_heads)]
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths, pairs=pairs,
                 scale=default_scale(w.head_dim))


def test_constant_groups_quantize_exactly():
    # constant key channels and constant value groups: scale 0, codes 0, zero = value
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=1, num_q_heads=2, num_kv_heads=2)
    S = 400
    inp = W.make_layer(w, device="cpu", seed=5, lengths=[S])
    k = inp.k.clone()
    v = inp.v.clone()
    k[:, :, :, 7] = 1.25                          # channel 7 constant everywhere
    v[:, :, 10:20, 32:64] = -0.5                  # value group 1 constant on tokens 10..19
    cache = make_cache(w, [S], 128)
    cache.prefill(k.cuda(), v.cuda(), [S], 128)
    out = cache.decode(inp.q.cuda())
    spec = spec_of(w, cache.cfg.res_capacity)
    check_records(cache, spec, to_np(k), to_np(v), [S], [(0, 0), (0, 1)])
    check_decode(out, spec, to_np(inp.q), to_np(k), to_np(v), [S], scale=default_scale(w.head_dim))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("wname", ["llama2-7b-layer", "ragged-paged"])
def test_decode_steps_across_flush(wname, fused):
    """Prefill, then decode steps of append(1) -> flush -> attention, across a
    block boundary; every step's output and the final records match."""
    over = dict(batch=2, num_q_heads=4, num_kv_heads=2) if wname == "llama2-7b-layer" else \
        dict(batch=3, num_q_heads=12, num_kv_heads=2)
    w = W.WORKLOADS[wname].replace(**over)
    lengths = [w.residual + 3 * w.k_group - 2] * w.batch if not w.paged else [90, 143, 500]
    steps = w.k_group + 3
    full = [s + steps for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=6, lengths=full)
    cache = make_cache(w, lengths, 64, extra_tokens=steps)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    spec = spec_of(w, cache.cfg.res_capacity)
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    for st in range(steps):
        idx = torch.tensor(lengths) + st
        kn = torch.stack([inp.k[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]).contiguous()
        vn = torch.stack([inp.v[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]).contiguous()
        if fused:
            cache.append_flush(kn.cuda(), vn.cuda())
        else:
            cache.append(kn.cuda(), vn.cuda())
            cache.flush()
        q = W.new_tokens(w, inp, 1, device="cpu", seed=6, step=st)[2]
        out = cache.decode(q.cuda())
        cur = [s + st + 1 for s in lengths]
        if st in (0, w.k_group - 3, w.k_group - 2, w.k_group - 1, steps - 1):
            check_decode(out, spec, to_np(q), k_np, v_np, cur, scale=default_scale(w.head_dim))
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, k_np, v_np, full, pairs)


def test_ring_overflow_sets_device_error():
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=1, num_q_heads=1, num_kv_heads=1)
    cache = make_cache(w, [300], 32)   # ring capacity R + G - 1 + 32 = 191
    # one append of more rows than the ring has slots is refused on the host
    kk = torch.zeros(1, 1, 200, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(B.KVQError) as e:
        cache.append(kk, kk)
    assert e.value.status == B.KVQ_ERR_CAPACITY
    # two appends that fit one by one but not together overflow on the device
    first = torch.zeros(1, 1, 150, 128, dtype=torch.float16, device="cuda")
    second = torch.zeros(1, 1, 50, 128, dtype=torch.float16, device="cuda")
    cache.append(first, first)
    cache.append(second, second)
    torch.cuda.synchronize()
    assert cache.read_device_error() & 1
    assert cache.lengths() == ([0], [150])


def test_fused_append_flush_ragged_counts_match_separate_calls():
    """Ragged n_new through the fused call gives the same cache bytes as
    append + flush, and both match the oracle."""
    w = W.WORKLOADS["ragged-paged"].replace(batch=4, num_q_heads=12, num_kv_heads=2)
    lengths = [70, 81, 200, 64]
    full = [s + 40 for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=8, lengths=full)
    caches = []
    for fused in (False, True):
        cache = make_cache(w, lengths, 64, extra_tokens=40)   # ring R + G - 1 + 64 takes 58 new rows
        cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
        cur = list(lengths)
        for step, n in enumerate([1, 3, 0, 7, 29]):
            counts = torch.tensor([n, max(n - 1, 0), n, 2 * n], dtype=torch.int32)
            nmax = int(counts.max())
            kn = torch.zeros(w.batch, w.num_kv_heads, max(nmax, 1), w.head_dim, dtype=w.torch_dtype)
            vn = torch.zeros_like(kn)
            for b in range(w.batch):
                c = int(counts[b])
                kn[b, :, :c] = inp.k[b, :, cur[b]:cur[b] + c]
                vn[b, :, :c] = inp.v[b, :, cur[b]:cur[b] + c]
            if fused:
                cache.append_flush(kn[:, :, :max(nmax, 1)].contiguous().cuda(),
                                   vn[:, :, :max(nmax, 1)].contiguous().cuda(), counts.cuda())
            else:
                cache.append(kn.cuda(), vn.cuda(), counts.cuda())
                cache.flush()
            cur = [cur[b] + int(counts[b]) for b in range(w.batch)]
        torch.cuda.synchronize()
        assert cache.read_device_error() == 0
        caches.append(cache)
    assert torch.equal(caches[0].blocks, caches[1].blocks)
    assert caches[0].lengths() == caches[1].lengths()
    spec = spec_of(w, caches[1].cfg.res_capacity)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(caches[1], spec, to_np(inp.k), to_np(inp.v), cur, pairs)
