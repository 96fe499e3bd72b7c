"""Limits of the path through the C ABI: a batch of several hundred ragged
sequences (the unit plan takes 64 sequences per pass; empty sequences among
them), a sequence longer than the caller's max_seq_tokens (flagged on the
device, its work capped to what the workspace was sized for), out-of-range
page-table entries met by decode and by the bulk flush, and a bulk flush that
needs more blocks than the store holds."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wname,over", [
    ("llama2-7b-layer", dict(num_q_heads=1, num_kv_heads=1)),                  # block-scaled MHA kernel
    ("llama3-8b-gqa-int2", dict(num_q_heads=4, num_kv_heads=1)),               # GQA matrix-core kernel
])
def test_several_hundred_ragged_sequences(wname, over):
    rng = np.random.default_rng(17)
    B = 300
    lengths = [int(x) for x in rng.integers(0, 700, size=B)]
    lengths[5] = lengths[77] = lengths[200] = 0
    w = W.WORKLOADS[wname].replace(batch=B, **over)
    print(f"[limits] {wname} B={B}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=18, lengths=lengths)
    cache = make_cache(w, lengths, 256)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    assert torch.count_nonzero(out[5]) == 0 and torch.count_nonzero(out[200]) == 0
    spec = spec_of(w, cache.cfg.res_capacity)
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths, scale=default_scale(w.head_dim))
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), lengths, [(b, 0) for b in range(0, B, 37)])


def test_sequence_longer_than_the_bound_is_flagged():
    w = W.WORKLOADS["llama2-7b-layer"].replace(batch=2, num_q_heads=2, num_kv_heads=2)
    lengths = [1000, 300]
    inp = W.make_layer(w, device="cpu", seed=19, lengths=lengths)
    cache = make_cache(w, lengths, 256)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    out = cache.decode(inp.q.cuda(), max_seq_tokens=500)   # sequence 0 holds 27 blocks, the bound allows 11
    torch.cuda.synchronize()
    assert cache.read_device_error() & 16
    assert torch.all(torch.isfinite(out))
    # the sequence within the bound is still exact
    spec = spec_of(w, cache.cfg.res_capacity)
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), lengths, pairs=[(1, 0), (1, 1)],
                 scale=default_scale(w.head_dim))


@pytest.mark.parametrize("wname,over", [
    ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2)),                     # GQA kernel, n_g = 6
    ("llama3-8b-gqa-int2", dict(batch=3, num_q_heads=8, num_kv_heads=2, paged=True)),   # GQA kernel, n_g = 4
    ("llama2-7b-layer", dict(batch=3, num_q_heads=2, num_kv_heads=2, paged=True)),      # block-scaled MHA kernel
])
def test_out_of_range_page_skips_its_block(wname, over):
    """A page-table entry outside [0, num_pages) drops that block from the
    attention of its sequence; the other blocks and sequences are unchanged."""
    from oracle import kivi
    w = W.WORKLOADS[wname].replace(**over)
    lengths = [600, 1111, 300]
    print(f"[limits] bad page {wname}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=21, lengths=lengths)
    cache = make_cache(w, lengths, 256)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    G = w.k_group
    bad = {5: cache.cfg.num_pages, 20: -1}   # quantized blocks of sequence 1
    assert max(bad) < (lengths[1] - w.residual) // G
    for j, page in bad.items():
        cache.page_table[1, j] = page
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    spec = spec_of(w, cache.cfg.res_capacity)
    q_np, k_np, v_np = to_np(inp.q), to_np(inp.k), to_np(inp.v)
    scale = default_scale(w.head_dim)
    ref = kivi.decode_attention(spec, q_np, k_np, v_np, lengths, scale=scale,
                                pairs=[(b, h) for b in (0, 2) for h in range(w.num_kv_heads)])
    ng = w.num_q_heads // w.num_kv_heads
    keep = np.ones(lengths[1], bool)
    for j in bad:
        keep[j * G:(j + 1) * G] = False
    for h in range(w.num_kv_heads):
        kh, vh = kivi.pair_cache_fp64(spec, k_np[1, h], v_np[1, h], lengths[1])
        ref[1, h * ng:(h + 1) * ng] = kivi.attention_fp64(q_np[1, h * ng:(h + 1) * ng], kh[keep], vh[keep], scale)
    diff = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert diff.max() <= 2e-3 and rel <= 1e-3, (diff.max(), rel)


def test_bulk_flush_past_max_blocks_is_flagged():
    """A flush that needs more blocks than the store has quantizes the blocks
    that fit, caps Q_b there and flags KVQ_DEV_BLOCKS_FULL; sequences that fit
    are flushed in full."""
    from oracle import kivi
    from quantized_kv_cache_append_amd import binding as B
    from quantized_kv_cache_append_amd.cache import QuantizedKVCache
    w = W.WORKLOADS["llama3-8b-gqa-int2"].replace(batch=3, num_q_heads=8, num_kv_heads=2)
    lengths = [1500, 300, 700]
    G, R = w.k_group, w.residual
    print("[limits] flush past max_blocks", flush=True)
    inp = W.make_layer(w, device="cpu", seed=23, lengths=lengths)
    cache = QuantizedKVCache(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, k_bits=w.k_bits, v_bits=w.v_bits,
                             k_group=G, v_group=w.v_group, residual=R, dtype=w.torch_dtype, max_tokens=16 * G,
                             res_capacity=2048)
    S = max(lengths)
    counts = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    cache.append(inp.k[:, :, :S].contiguous().cuda(), inp.v[:, :, :S].contiguous().cuda(), counts)
    cache.flush()
    torch.cuda.synchronize()
    assert cache.read_device_error() == B.KVQ_DEV_BLOCKS_FULL
    Qs, Ss = cache.lengths()
    want_Q = [min(16, (s - R) // G) * G for s in lengths]
    assert Qs == want_Q and Ss == lengths, (Qs, Ss)
    spec = spec_of(w, cache.cfg.res_capacity)
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    for b, s in enumerate(lengths):
        for h in range(w.num_kv_heads):
            exp = kivi.expected_blocks(spec, k_np[b, h], v_np[b, h], s)
            for j in range(want_Q[b] // G):
                assert np.array_equal(cache.record(b, h, j).cpu().numpy(), exp[j]), (b, h, j)


def test_bulk_flush_skips_an_out_of_range_page():
    """A page-table entry outside [0, num_pages) met by the bulk flush: that
    block is skipped (KVQ_DEV_BAD_PAGE), every other block of every pair is
    written bit for bit and the lengths advance as usual."""
    from oracle import kivi
    from quantized_kv_cache_append_amd import binding as B
    w = W.WORKLOADS["ragged-paged"].replace(batch=3, num_q_heads=12, num_kv_heads=2)
    lengths = [600, 1111, 300]
    G = w.k_group
    print("[limits] flush over a bad page", flush=True)
    inp = W.make_layer(w, device="cpu", seed=29, lengths=lengths)
    cache = make_cache(w, lengths, 256)
    cache.page_table[1, 5] = cache.cfg.num_pages
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    torch.cuda.synchronize()
    assert cache.read_device_error() == B.KVQ_DEV_BAD_PAGE
    spec = spec_of(w, cache.cfg.res_capacity)
    Qs, Ss = cache.lengths()
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    checked = 0
    for b, s in enumerate(lengths):
        _, Q, _ = kivi.stream_split(spec, s)
        assert Qs[b] == Q and Ss[b] == s
        for h in range(w.num_kv_heads):
            exp = kivi.expected_blocks(spec, k_np[b, h], v_np[b, h], s)
            for j in range(Q // G):
                if (b, j) == (1, 5):
                    continue
                assert np.array_equal(cache.record(b, h, j).cpu().numpy(), exp[j]), (b, h, j)
                checked += 1
    assert checked > 100
