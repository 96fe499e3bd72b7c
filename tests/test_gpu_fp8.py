"""Parity of the FP8 tier (the W most recent quantized blocks of every
(sequence, kv head) also kept as FP8 records, and read there) with the CPU
oracle, through the C ABI: low-bit records, FP8 records, ring and lengths
bit-exact; attention within the usual max-abs 2e-3 / rel-L2 1e-3 -- on every
decode path and with the sink and the multi-token query."""
import pytest
import torch

from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import (ATOL, RTOL_L2, check_decode, check_records, default_scale, errors, make_cache, spec_of,
                         to_np)
from oracle import kivi

pytestmark = pytest.mark.gpu

FP8_CASES = {
    # name: (workload, overrides, lengths, chunk, W, sink P)
    "mha-int2-w4": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4), [100, 700, 1500], 256, 4, 0),
    "mha-int4-w2": ("llama2-7b-layer", dict(batch=2, num_q_heads=4, num_kv_heads=4, k_bits=4, v_bits=4),
                    [1000, 333], 256, 2, 0),
    "gqa-int2-w2": ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2), [2100, 400], 512, 2, 0),
    "70b-g64-w1": ("llama-70b-128k-80layer", dict(batch=1, num_q_heads=16, num_kv_heads=2, layers=1), [3000], 512,
                   1, 0),
    "paged-w3": ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2), [37, 300, 1111], 256, 3, 0),
    "tiny-d64-w2": ("tiny", {}, None, 128, 2, 0),
    "sink-and-tier": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [5, 900], 256, 3, 4),
    # a window wider than every sequence's blocks: all quantized blocks read in FP8
    "all-fp8": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [400, 1100], 256, 64, 0),
}


def _run(name, seed=0):
    wname, over, lengths, chunk, Wt, P = FP8_CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    if lengths is None:
        lengths = W.sequence_lengths(w, seed)
    print(f"[fp8 case {name}] W={Wt} P={P} lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=seed, lengths=lengths)
    cache = make_cache(w, lengths, chunk, sink=P, fp8_blocks=Wt)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, chunk)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    return w, cache, inp, lengths, out, spec_of(w, cache.cfg.res_capacity, sink=P, fp8_blocks=Wt)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_tier_records_bit_exact(name):
    w, cache, inp, lengths, _, spec = _run(name)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, pairs)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_tier_decode_matches_oracle(name):
    w, cache, inp, lengths, out, spec = _run(name)
    max_abs, rel = check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths,
                                scale=default_scale(w.head_dim))
    print(f"[fp8 case {name}] max_abs={max_abs:.2e} rel_l2={rel:.2e}")


@pytest.mark.parametrize("fused", [False, True])
def test_fp8_window_slides_with_decode_steps(fused):
    """One-token steps across two flushes with W = 2: blocks leave the tier
    (read from their low-bit records from then on) as new ones enter it."""
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=2, num_q_heads=2, num_kv_heads=2)
    Wt, steps = 2, 2 * w.k_group + 3
    lengths = [w.residual + 3 * w.k_group - 2, w.residual + 2 * w.k_group + 5]
    full = [s + steps for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=12, lengths=full)
    cache = make_cache(w, lengths, 64, extra_tokens=steps, fp8_blocks=Wt)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    spec = spec_of(w, cache.cfg.res_capacity, fp8_blocks=Wt)
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
        q = W.new_tokens(w, inp, 1, device="cpu", seed=12, step=st)[2]
        out = cache.decode(q.cuda())
        cur = [s + st + 1 for s in lengths]
        if st in (0, 1, 2, w.k_group, w.k_group + 1, steps - 1):
            check_decode(out, spec, to_np(q), k_np, v_np, cur, scale=default_scale(w.head_dim))
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    check_records(cache, spec, k_np, v_np, full, [(b, h) for b in range(2) for h in range(2)])


def test_fp8_tier_with_a_multi_token_block():
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=2, num_q_heads=2, num_kv_heads=2)
    T, Wt, lengths = 4, 3, [600, 1300]
    inp = W.make_layer(w, device="cpu", seed=13, lengths=lengths)
    cache = make_cache(w, lengths, 256, fp8_blocks=Wt)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    g = torch.Generator().manual_seed(77)
    q = torch.randn(w.batch, w.num_q_heads, T, w.head_dim, generator=g).to(w.torch_dtype)
    out = cache.decode_multi(q.cuda())
    torch.cuda.synchronize()
    spec = spec_of(w, cache.cfg.res_capacity, fp8_blocks=Wt)
    ref = kivi.decode_attention_multi(spec, to_np(q), to_np(inp.k), to_np(inp.v), lengths, T,
                                      scale=default_scale(w.head_dim))
    max_abs, rel = errors(out.double().cpu().numpy(), ref)
    assert max_abs <= ATOL and rel <= RTOL_L2, f"max_abs={max_abs:.3e} rel_l2={rel:.3e}"
