"""Shared test harness: fill a libkvq cache from a workload and check it against
the oracle (GPU tests only)."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import kivi
from quantized_kv_cache_append_amd import workloads as W
from quantized_kv_cache_append_amd.cache import QuantizedKVCache, cache_for_workload

ATOL = 2e-3     # max-abs error against the fp64 oracle on the same dequantized cache
RTOL_L2 = 1e-3  # relative L2 error over the whole output


def spec_of(w: W.Workload, res_capacity: int, sink: int = 0, fp8_blocks: int = 0, rotate: int = 0) -> kivi.CacheSpec:
    return kivi.CacheSpec(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim=w.head_dim, k_bits=w.k_bits, v_bits=w.v_bits, k_group=w.k_group,
                          v_group=w.v_group, residual=w.residual, res_capacity=res_capacity, dtype=w.dtype,
                          sink=sink, fp8_blocks=fp8_blocks, rotate=rotate)


def make_cache(w: W.Workload, lengths, chunk: int, extra_tokens: int = 0, device="cuda", seed: int = 0,
               sink: int = 0, fp8_blocks: int = 0, rotate: int = 0):
    return cache_for_workload(w, lengths, chunk, extra_tokens=extra_tokens, device=device, seed=seed, sink=sink,
                              fp8_blocks=fp8_blocks, rotate=rotate)


def errors(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got.astype(np.float64) - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def check_records(cache: QuantizedKVCache, spec: kivi.CacheSpec, k_np, v_np, lengths, pairs):
    """Bit-exact comparison of every quantized block of the given (b, h) pairs,
    of their rings and of their sink rows."""
    Qs, Ss = cache.lengths()
    n_blocks = 0
    P = spec.sink
    for b, h in pairs:
        S_b = int(lengths[b])
        s, Q, _ = kivi.stream_split(spec, S_b)
        assert Qs[b] == Q and Ss[b] == S_b, f"lengths of seq {b}: got (Q={Qs[b]}, S={Ss[b]}), want ({Q}, {S_b})"
        exp = kivi.expected_blocks(spec, k_np[b, h], v_np[b, h], S_b)
        for j in range(Q // spec.k_group):
            got = cache.record(b, h, j).cpu().numpy()
            if not np.array_equal(got, exp[j]):
                bad = np.nonzero(got != exp[j])[0]
                raise AssertionError(f"record (b={b}, h={h}, blk={j}) differs at {bad.size} bytes, first {bad[:8]}")
            n_blocks += 1
        # the ring holds the residual tokens bit for bit
        slots = kivi.ring_slots(Q, S_b, spec.res_capacity, sink=P)
        kr = cache.k_ring[b, h].float().cpu().numpy()[slots]
        vr = cache.v_ring[b, h].float().cpu().numpy()[slots]
        assert np.array_equal(kr, k_np[b, h, P + Q:S_b]) and np.array_equal(vr, v_np[b, h, P + Q:S_b]), \
            f"ring of (b={b}, h={h}) differs"
        # the FP8 tier: the records of the W most recent blocks
        if spec.fp8_blocks > 0:
            f0, nblk = kivi.fp8_window(spec, S_b)
            G = spec.k_group
            for j in range(f0, nblk):
                lo = P + j * G
                exp8 = kivi.fp8_record(k_np[b, h, lo:lo + G], v_np[b, h, lo:lo + G])
                got8 = cache.fp8_record(b, h, j).cpu().numpy()
                if not np.array_equal(got8, exp8):
                    bad = np.nonzero(got8 != exp8)[0]
                    raise AssertionError(f"FP8 record (b={b}, h={h}, blk={j}) differs at {bad.size} bytes, "
                                         f"first {bad[:8]}: got {got8[bad[:4]]}, want {exp8[bad[:4]]}")
        # and the sink its tokens
        if P > 0:
            ks = cache.k_sink[b, h, :s].float().cpu().numpy()
            vs = cache.v_sink[b, h, :s].float().cpu().numpy()
            assert np.array_equal(ks, k_np[b, h, :s]) and np.array_equal(vs, v_np[b, h, :s]), \
                f"sink of (b={b}, h={h}) differs"
    return n_blocks


def check_decode(out: torch.Tensor, spec: kivi.CacheSpec, q_np, k_np, v_np, lengths, pairs=None, scale=None):
    """Attention output against the fp64 oracle; returns (max_abs, rel_l2)."""
    ref = kivi.decode_attention(spec, q_np, k_np, v_np, lengths, scale=scale, pairs=pairs)
    got = out.double().cpu().numpy()
    mask = ~np.isnan(ref)
    max_abs, rel = errors(got[mask], ref[mask])
    assert np.all(np.isfinite(got[mask])), "non-finite output"
    assert max_abs <= ATOL and rel <= RTOL_L2, f"decode error max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def default_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


GUARD_BYTE = 0xA5


class Guards:
    """Guard bands around device buffers: each buffer is replaced by a view into
    a larger allocation whose first and last `nbytes` hold GUARD_BYTE. check()
    asserts that no kernel wrote into a band."""

    def __init__(self, nbytes: int = 4096):
        self.nbytes = nbytes
        self.bands = []

    def wrap(self, t: torch.Tensor, name: str) -> torch.Tensor:
        n = t.numel() * t.element_size()
        big = torch.full((n + 2 * self.nbytes,), GUARD_BYTE, dtype=torch.uint8, device=t.device)
        view = big[self.nbytes:self.nbytes + n]
        view.copy_(t.contiguous().view(torch.uint8).reshape(-1))
        self.bands.append((name, big))
        return view.view(t.dtype).view(t.shape)

    def check(self):
        torch.cuda.synchronize()
        for name, big in self.bands:
            lo = big[:self.nbytes].cpu().numpy()
            hi = big[-self.nbytes:].cpu().numpy()
            assert (lo == GUARD_BYTE).all(), f"write below {name}: bytes {np.nonzero(lo != GUARD_BYTE)[0][:8]}"
            assert (hi == GUARD_BYTE).all(), f"write past {name}: bytes {np.nonzero(hi != GUARD_BYTE)[0][:8]}"


def guard_cache(cache: QuantizedKVCache, guards: Guards) -> QuantizedKVCache:
    """Move every device buffer of `cache` inside guard bands and re-point its C
    struct at them."""
    from quantized_kv_cache_append_amd import binding as B
    cache.blocks = guards.wrap(cache.blocks, "block store")
    cache.k_ring = guards.wrap(cache.k_ring, "k_ring")
    cache.v_ring = guards.wrap(cache.v_ring, "v_ring")
    cache.state = guards.wrap(cache.state, "state words")
    if cache.page_table is not None:
        cache.page_table = guards.wrap(cache.page_table, "page table")
    if cache.k_sink is not None:
        cache.k_sink = guards.wrap(cache.k_sink, "k_sink")
        cache.v_sink = guards.wrap(cache.v_sink, "v_sink")
    if cache.fp8 is not None:
        cache.fp8 = guards.wrap(cache.fp8, "fp8 store")
    cache.cache = B.kvq_cache(
        blocks=cache.blocks.data_ptr(),
        block_table=cache.page_table.data_ptr() if cache.page_table is not None else None,
        k_ring=cache.k_ring.data_ptr(), v_ring=cache.v_ring.data_ptr(), state=cache.state.data_ptr(),
        k_sink=cache.k_sink.data_ptr() if cache.k_sink is not None else None,
        v_sink=cache.v_sink.data_ptr() if cache.v_sink is not None else None,
        fp8=cache.fp8.data_ptr() if cache.fp8 is not None else None)
    return cache
