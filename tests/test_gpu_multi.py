"""Parity of the multi-token query (the T newest tokens of every sequence,
causal within the block) with the CPU oracle, through the C ABI: the T tokens
are appended (and flushed) first, then kvq_decode_attention_multi. Attention
within the usual max-abs 2e-3 / rel-L2 1e-3 of the fp64 oracle on the same
cache state."""
import pytest
import torch

from quantized_kv_cache_append_amd import workloads as W
from quantized_kv_cache_append_amd.binding import KVQError

from kvq_harness import check_records, default_scale, errors, make_cache, spec_of, to_np, ATOL, RTOL_L2
from oracle import kivi

pytestmark = pytest.mark.gpu

MULTI_CASES = {
    # name: (workload, overrides, lengths after the block, T, sink P)
    "mha-f16-t4": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4), [300, 1111, 2000], 4, 0),
    "mha-bf16-paged-t8": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2, dtype="bf16", paged=True),
                          [700, 1500], 8, 0),
    "gqa-int4-t2": ("llama3-8b-gqa-int4", dict(batch=2, num_q_heads=8, num_kv_heads=2), [2100, 333], 2, 0),
    "70b-g64-t1": ("llama-70b-128k-80layer", dict(batch=1, num_q_heads=16, num_kv_heads=2, layers=1), [3000], 1, 0),
    "tiny-d64-t3": ("tiny", {}, [512], 3, 0),
    # the block straddles the sink (P = 6): tokens 3..8 are the queries of a 9-token sequence
    "sink-straddle-t6": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [9, 600], 6, 6),
    # a sink on the matrix-core path (4 rows): the block of the 5-token sequence straddles it
    "sink-t4": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [5, 900], 4, 3),
    # a sequence shorter than the block: its first queries see nothing
    "short-t4": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2), [2, 400], 4, 0),
}


def _queries(w, T, seed):
    g = torch.Generator().manual_seed(1000 + seed)
    return torch.randn(w.batch, w.num_q_heads, T, w.head_dim, generator=g).to(w.torch_dtype)


def _run(name, seed=0):
    wname, over, lengths, T, P = MULTI_CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    print(f"[multi case {name}] T={T} P={P} lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=seed, lengths=lengths)
    before = [max(S - T, 0) for S in lengths]
    cache = make_cache(w, lengths, 256, sink=P)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), before, 256)
    # the block: T rows per sequence (fewer where the sequence is shorter), appended and flushed in one call
    counts = torch.tensor([S - s0 for S, s0 in zip(lengths, before)], dtype=torch.int32)
    kn = torch.zeros(w.batch, w.num_kv_heads, T, w.head_dim, dtype=w.torch_dtype)
    vn = torch.zeros_like(kn)
    for b in range(w.batch):
        c = int(counts[b])
        kn[b, :, :c] = inp.k[b, :, before[b]:before[b] + c]
        vn[b, :, :c] = inp.v[b, :, before[b]:before[b] + c]
    cache.append_flush(kn.cuda(), vn.cuda(), counts.cuda())
    q = _queries(w, T, seed)
    out = cache.decode_multi(q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    return w, cache, inp, lengths, T, q, out, spec_of(w, cache.cfg.res_capacity, sink=P)


@pytest.mark.parametrize("name", list(MULTI_CASES))
def test_multi_token_query_matches_oracle(name):
    w, cache, inp, lengths, T, q, out, spec = _run(name)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, pairs)
    ref = kivi.decode_attention_multi(spec, to_np(q), to_np(inp.k), to_np(inp.v), lengths, T,
                                      scale=default_scale(w.head_dim))
    got = out.double().cpu().numpy()
    max_abs, rel = errors(got, ref)
    print(f"[multi case {name}] max_abs={max_abs:.2e} rel_l2={rel:.2e}")
    assert max_abs <= ATOL and rel <= RTOL_L2, f"max_abs={max_abs:.3e} rel_l2={rel:.3e}"


def test_one_token_block_is_the_decode():
    w, cache, inp, lengths, T, q, out, spec = _run("70b-g64-t1")
    single = cache.decode(q[:, :, 0].contiguous().cuda())
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0], single)


def test_too_many_query_rows_is_refused():
    # n_g = 6 with T = 2 would need 12 query rows per kv head
    w = W.WORKLOADS["ragged-paged"].replace(batch=2, num_q_heads=12, num_kv_heads=2)
    cache = make_cache(w, [100, 100], 64)
    q = torch.zeros(w.batch, w.num_q_heads, 2, w.head_dim, dtype=w.torch_dtype, device="cuda")
    with pytest.raises(KVQError):
        cache.decode_multi(q)
