"""Parity at the full workload sizes, on sampled (sequence, kv head) pairs.

The caches are filled and decoded exactly as the benchmark does (same chunked
append/flush, same decode launch); the oracle then recomputes the sampled
pairs one by one: every record of those pairs bit for bit, and their decode
outputs within max-abs 2e-3 / relative L2 1e-3 of the fp64 oracle.
"""
import pytest
import torch

from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu

SAMPLES = {
    "llama2-7b-layer": [(0, 0), (3, 17), (7, 31)],
    "llama3-8b-gqa-int4": [(0, 0), (13, 5), (31, 7)],
    "llama3-8b-gqa-int2": [(0, 0), (21, 3), (31, 7)],
    "ragged-paged": None,   # chosen from the lengths: shortest, median, longest
}


def _pairs_np(inp, pairs):
    """CPU copies of only the sampled pairs, indexed like the full tensors."""
    k = {}
    v = {}
    for b, h in pairs:
        k[(b, h)] = to_np(inp.k[b, h])
        v[(b, h)] = to_np(inp.v[b, h])
    return k, v


class _Sparse:
    """Indexable view [b, h] over a dict of per-pair arrays (oracle input)."""

    def __init__(self, d):
        self.d = d

    def __getitem__(self, key):
        b, h = key[0], key[1]
        a = self.d[(b, h)]
        return a[key[2:]] if len(key) > 2 else a


def _check_fullsize(w, lengths, pairs, chunk, seed=0, layer=0):
    print(f"[fullsize {w.name} layer {layer}] B={w.batch} S_max={max(lengths)} pairs={pairs}", flush=True)
    inp = W.make_layer(w, device="cuda", seed=seed, layer=layer, lengths=lengths)
    cache = make_cache(w, lengths, chunk)
    cache.prefill(inp.k, inp.v, lengths, chunk)
    out = cache.decode(inp.q)
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    spec = spec_of(w, cache.cfg.res_capacity)
    kd, vd = _pairs_np(inp, pairs)
    k_np, v_np = _Sparse(kd), _Sparse(vd)
    n = check_records(cache, spec, k_np, v_np, lengths, pairs)
    q_np = to_np(inp.q)
    max_abs, rel = check_decode(out, spec, q_np, k_np, v_np, lengths, pairs=pairs,
                                scale=default_scale(w.head_dim))
    print(f"[fullsize {w.name}] {n} records bit-exact; decode max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    del cache, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama2-7b-layer", "llama3-8b-gqa-int4", "llama3-8b-gqa-int2"])
def test_fullsize_dense(name):
    w = W.WORKLOADS[name]
    _check_fullsize(w, W.sequence_lengths(w), SAMPLES[name], chunk=2048)


def test_fullsize_ragged_paged():
    w = W.WORKLOADS["ragged-paged"]
    lengths = W.sequence_lengths(w)
    order = sorted(range(w.batch), key=lambda b: lengths[b])
    pairs = [(order[0], 0), (order[len(order) // 2], 3), (order[-1], 7)]
    _check_fullsize(w, lengths, pairs, chunk=2048)


@pytest.mark.parametrize("layer", [0, 39, 79])
def test_fullsize_70b_layers(layer):
    w = W.WORKLOADS["llama-70b-128k-80layer"]
    _check_fullsize(w, W.sequence_lengths(w), [(0, 0), (3, 7)], chunk=4096, layer=layer)
