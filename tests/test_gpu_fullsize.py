"""Parity at the full workload sizes.

The caches are filled and decoded exactly as the benchmark does (same chunked
append/flush, same decode launch). The oracle then recomputes, per (sequence,
kv head) pair, every record bit for bit and the pair's decode outputs; the
outputs of all checked pairs must be within max-abs 2e-3 / relative L2 1e-3 of
the fp64 oracle, the L2 taken over all of them together.

Coverage:
  - Llama-2-7B-shaped layer: every (sequence, kv head) pair (256);
  - Llama-3-8B-shaped GQA layer, INT4 and INT2: every kv head of 8 sequences
    spread over the batch (64 of 256 pairs);
  - ragged paged batch: every kv head of 8 sequences spread over the lengths,
    the shortest and the longest among them (64 of 512 pairs);
  - 70B-shaped model: layers 0, 39 and 79 in full (all 32 pairs, records and
    attention), and one pair of every other layer (its records).

The oracle runs on host worker processes forked before any of them touches
the GPU (numpy only), one pair per task.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import ATOL, RTOL_L2, default_scale, make_cache, spec_of

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(12, (os.cpu_count() or 2) - 2))


def _pool():
    return cf.ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("fork"))


def _host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a fp16/bf16 device tensor, on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def _check_pair(spec, b, h, S, kbits, vbits, recs, kring, vring, q, got, scale, want_decode):
    """One pair against the oracle (runs in a worker): its records, its ring and,
    if asked, its decode outputs. Returns (blocks checked, squared error sum,
    squared reference sum, max abs error)."""
    k = _to_f32(kbits, spec.dtype)
    v = _to_f32(vbits, spec.dtype)
    exp = kivi.expected_blocks(spec, k, v, S)
    assert recs.shape == exp.shape, f"(b={b}, h={h}): {recs.shape[0]} records, want {exp.shape[0]}"
    if not np.array_equal(recs, exp):
        j = int(np.nonzero((recs != exp).any(axis=1))[0][0])
        bad = np.nonzero(recs[j] != exp[j])[0]
        raise AssertionError(f"record (b={b}, h={h}, blk={j}) differs at {bad.size} bytes, first {bad[:8]}")
    _, Q, _ = kivi.stream_split(spec, S)
    slots = kivi.ring_slots(Q, S, spec.res_capacity)
    assert np.array_equal(_to_f32(kring[slots], spec.dtype), k[Q:S]), f"ring K of (b={b}, h={h}) differs"
    assert np.array_equal(_to_f32(vring[slots], spec.dtype), v[Q:S]), f"ring V of (b={b}, h={h}) differs"
    if not want_decode:
        return exp.shape[0], 0.0, 0.0, 0.0
    one = kivi.CacheSpec(1, spec.n_g, 1, spec.head_dim, spec.k_bits, spec.v_bits, spec.k_group, spec.v_group,
                         spec.residual, spec.res_capacity, spec.dtype)
    ref = kivi.decode_attention(one, q[None], k[None, None], v[None, None], [S], scale=scale)[0]
    d = got.astype(np.float64) - ref
    assert np.all(np.isfinite(got)), f"non-finite output for (b={b}, h={h})"
    return exp.shape[0], float(np.sum(d * d)), float(np.sum(ref * ref)), float(np.max(np.abs(d)))


class _Layer:
    """One filled and decoded layer cache, with host copies of what the oracle
    compares against."""

    def __init__(self, w, lengths, chunk, layer=0, seed=0, decode=True):
        self.w, self.lengths = w, lengths
        self.inp = W.make_layer(w, device="cuda", seed=seed, layer=layer, lengths=lengths)
        self.cache = make_cache(w, lengths, chunk)
        self.cache.prefill(self.inp.k, self.inp.v, lengths, chunk)
        self.out = self.cache.decode(self.inp.q).cpu().numpy() if decode else None
        torch.cuda.synchronize()
        assert self.cache.read_device_error() == 0
        Qs, Ss = self.cache.lengths()
        self.spec = spec_of(w, self.cache.cfg.res_capacity)
        for b, S in enumerate(lengths):
            assert Ss[b] == S and Qs[b] == kivi.stream_split(self.spec, S)[1], f"lengths of sequence {b}"
        self.blocks = self.cache.blocks.cpu().numpy()
        self.table = self.cache.page_table.cpu().numpy() if self.cache.page_table is not None else None
        self.rec = self.cache.layout.record
        self.q = self.inp.q.float().cpu().numpy()

    def records(self, b, h):
        c = self.cache.cfg
        nblk = kivi.stream_split(self.spec, self.lengths[b])[1] // c.k_group
        if self.table is None:
            base = ((b * c.num_kv_heads + h) * c.max_blocks) * self.rec
            return self.blocks[base:base + nblk * self.rec].reshape(nblk, self.rec)
        pages = self.table[b, :nblk].astype(np.int64)
        offs = (pages * c.num_kv_heads + h) * self.rec
        return np.stack([self.blocks[o:o + self.rec] for o in offs]) if nblk else \
            np.zeros((0, self.rec), np.uint8)

    def task(self, b, h, decode=True):
        S = self.lengths[b]
        n_g = self.w.n_g
        return (self.spec, b, h, S, _host_bits(self.inp.k[b, h, :S]), _host_bits(self.inp.v[b, h, :S]),
                self.records(b, h), _host_bits(self.cache.k_ring[b, h]), _host_bits(self.cache.v_ring[b, h]),
                self.q[b, h * n_g:(h + 1) * n_g], self.out[b, h * n_g:(h + 1) * n_g] if decode else None,
                default_scale(self.w.head_dim), decode)

    def free(self):
        del self.cache, self.inp
        torch.cuda.empty_cache()


def _run(pool, tasks):
    n = 0
    d2 = r2 = mx = 0.0
    for fut in [pool.submit(_check_pair, *t) for t in tasks]:
        nb, a, b, m = fut.result()
        n, d2, r2, mx = n + nb, d2 + a, r2 + b, max(mx, m)
    return n, d2, r2, mx


def _assert_decode(name, n, d2, r2, mx, pairs):
    rel = (d2 / r2) ** 0.5 if r2 > 0 else 0.0
    print(f"[fullsize {name}] {pairs} pairs, {n} records bit-exact; decode max_abs={mx:.2e} rel_l2={rel:.2e}",
          flush=True)
    assert mx <= ATOL and rel <= RTOL_L2, f"{name}: decode error max_abs={mx:.3e} rel_l2={rel:.3e}"


def _spread(batch, k=8):
    """k sequence indices spread evenly over [0, batch)."""
    return sorted({round(i * (batch - 1) / (k - 1)) for i in range(k)})


def test_fullsize_llama2_every_pair():
    w = W.WORKLOADS["llama2-7b-layer"]
    print(f"[fullsize {w.name}] B={w.batch} S={w.seq_len}: every pair", flush=True)
    L = _Layer(w, W.sequence_lengths(w), chunk=2048)
    with _pool() as pool:
        pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
        res = _run(pool, [L.task(b, h) for b, h in pairs])
    L.free()
    _assert_decode(w.name, *res, len(pairs))


@pytest.mark.parametrize("name", ["llama3-8b-gqa-int4", "llama3-8b-gqa-int2"])
def test_fullsize_gqa_eight_sequences(name):
    w = W.WORKLOADS[name]
    seqs = _spread(w.batch)
    print(f"[fullsize {name}] B={w.batch} S={w.seq_len}: every kv head of sequences {seqs}", flush=True)
    L = _Layer(w, W.sequence_lengths(w), chunk=2048)
    with _pool() as pool:
        pairs = [(b, h) for b in seqs for h in range(w.num_kv_heads)]
        res = _run(pool, [L.task(b, h) for b, h in pairs])
    L.free()
    _assert_decode(name, *res, len(pairs))


def test_fullsize_ragged_paged_eight_sequences():
    w = W.WORKLOADS["ragged-paged"]
    lengths = W.sequence_lengths(w)
    order = sorted(range(w.batch), key=lambda b: lengths[b])
    seqs = sorted({order[i] for i in _spread(w.batch)})
    assert order[0] in seqs and order[-1] in seqs
    print(f"[fullsize ragged-paged] every kv head of sequences {seqs} "
          f"(lengths {[lengths[b] for b in seqs]})", flush=True)
    L = _Layer(w, lengths, chunk=2048)
    with _pool() as pool:
        pairs = [(b, h) for b in seqs for h in range(w.num_kv_heads)]
        res = _run(pool, [L.task(b, h) for b, h in pairs])
    L.free()
    _assert_decode("ragged-paged", *res, len(pairs))


def test_fullsize_70b_layers():
    w = W.WORKLOADS["llama-70b-128k-80layer"]
    lengths = W.sequence_lengths(w)
    full = {0, 39, 79}
    every = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    with _pool() as pool:
        for layer in range(w.layers):
            if layer in full:
                print(f"[fullsize 70b layer {layer}] every pair", flush=True)
                L = _Layer(w, lengths, chunk=4096, layer=layer)
                res = _run(pool, [L.task(b, h) for b, h in every])
                L.free()
                _assert_decode(f"70b layer {layer}", *res, len(every))
            else:
                b, h = every[(layer * 7) % len(every)]
                L = _Layer(w, lengths, chunk=4096, layer=layer, decode=False)
                n, _, _, _ = _run(pool, [L.task(b, h, decode=False)])
                L.free()
                if layer % 10 == 1:
                    print(f"[fullsize 70b layer {layer}] pair ({b}, {h}): {n} records bit-exact", flush=True)
