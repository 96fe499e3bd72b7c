"""Edge cases of the quantizer and of buffer bounds, on the GPU.

- A group whose fp16 scale is subnormal (range below 2^-14 * (2^b - 1)): formula
  F still fixes every bit, so the record must match the oracle exactly (the
  error bound |x - x_hat| <= s/2 is only claimed for normal scales).
- Guard bands: every buffer a kernel writes (block store, rings, sink, FP8
  store, state words, workspace, output) sits between bands of a known byte
  pattern, which must be intact after appends, flushes and decodes of every
  kernel family.
"""
import numpy as np
import pytest
import torch

from oracle import kivi
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import (Guards, check_decode, check_records, default_scale, guard_cache, make_cache, spec_of,
                         to_np)

pytestmark = pytest.mark.gpu


def _subnormal_inputs(w, lengths, seed):
    """The workload's inputs with tiny-range groups planted in the first block of
    pair (0, 0): two key channels and two value token groups whose range is a
    few units in the last place of values near 1e-3."""
    inp = W.make_layer(w, device="cpu", seed=seed, lengths=lengths)
    G, gv = w.k_group, w.v_group
    k, v = inp.k.clone(), inp.v.clone()
    step = torch.tensor([0, 1, 3, 4] * (G // 4), dtype=torch.float32)
    for c, sgn in ((5, 1.0), (70, -1.0)):
        col = sgn * (1e-3 + step * (2 ** -20 if w.dtype == "f16" else 2 ** -17))
        k[0, 0, :G, c] = col.to(w.torch_dtype)
    for t, sgn in ((3, 1.0), (17, -1.0)):
        row = sgn * (2e-3 + torch.arange(gv, dtype=torch.float32) % 4 * (2 ** -19 if w.dtype == "f16" else 2 ** -16))
        v[0, 0, t, :gv] = row.to(w.torch_dtype)
    return inp, k, v


@pytest.mark.parametrize("wname,over", [
    ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2)),          # fp16, INT2, block-scaled MFMA
    ("llama3-8b-gqa-int4", dict(batch=2, num_q_heads=8, num_kv_heads=2)),      # bf16, INT4, GQA MFMA
])
def test_subnormal_scale_groups_are_bit_exact(wname, over):
    w = W.WORKLOADS[wname].replace(**over)
    lengths = [300, 257]
    inp, k, v = _subnormal_inputs(w, lengths, seed=21)
    spec = spec_of(w, w.residual + w.k_group - 1 + 64)
    # the planted groups do have subnormal scales in the oracle
    sec = kivi.quantize_block(spec, to_np(k[0, 0, :w.k_group]), to_np(v[0, 0, :w.k_group]))
    ks = sec["k_scale"].astype(np.float64)
    vs = sec["v_scale"].astype(np.float64)
    tiny = 2.0 ** -14
    assert 0 < ks[5] < tiny and 0 < ks[70] < tiny, (ks[5], ks[70])
    assert 0 < vs[0, 3] < tiny and 0 < vs[0, 17] < tiny, (vs[0, 3], vs[0, 17])
    cache = make_cache(w, lengths, 64)
    cache.prefill(k.cuda(), v.cuda(), lengths, 64)
    out = cache.decode(inp.q.cuda())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(k), to_np(v), lengths, pairs)
    check_decode(out, spec, to_np(inp.q), to_np(k), to_np(v), lengths, scale=default_scale(w.head_dim))


CANARY_CASES = {
    # name: (workload, overrides, lengths, sink, fp8 blocks)
    "mha-fp16-int2": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4), [500, 33, 1100], 0, 0),
    "mha-int4-sink": ("llama2-7b-layer", dict(batch=2, num_q_heads=2, num_kv_heads=2, k_bits=4, v_bits=4),
                      [700, 150], 4, 0),
    "gqa-int2-fp8": ("llama3-8b-gqa-int2", dict(batch=2, num_q_heads=8, num_kv_heads=2), [900, 300], 0, 3),
    "70b-shape": ("llama-70b-128k-80layer", dict(batch=2, num_q_heads=16, num_kv_heads=2, layers=1),
                  [1500, 200], 0, 0),
    "paged-ng6": ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2), [37, 300, 1111], 0, 0),
    "tiny-generic": ("tiny", dict(batch=2), [512, 100], 0, 0),
}


@pytest.mark.parametrize("name", list(CANARY_CASES))
def test_guard_bands_stay_intact(name):
    wname, over, lengths, P, W8 = CANARY_CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    steps = 40
    full = [s + steps for s in lengths]
    inp = W.make_layer(w, device="cpu", seed=31, lengths=full)
    guards = Guards()
    cache = guard_cache(make_cache(w, lengths, 64, extra_tokens=steps, sink=P, fp8_blocks=W8), guards)
    cache.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 64)
    msl = max(full)
    ws = guards.wrap(torch.zeros(cache.workspace_bytes(msl), dtype=torch.uint8, device="cuda"), "workspace")
    out = guards.wrap(torch.zeros(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda"), "out")
    cur = list(lengths)
    for st in range(steps):
        kn = torch.stack([inp.k[b, :, cur[b]:cur[b] + 1] for b in range(w.batch)]).contiguous()
        vn = torch.stack([inp.v[b, :, cur[b]:cur[b] + 1] for b in range(w.batch)]).contiguous()
        cache.append_flush(kn.cuda(), vn.cuda())
        cur = [s + 1 for s in cur]
        cache.decode(inp.q.cuda(), out=out, max_seq_tokens=msl, workspace=ws)
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    guards.check()
    spec = spec_of(w, cache.cfg.res_capacity, sink=P, fp8_blocks=W8)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(cache, spec, to_np(inp.k), to_np(inp.v), cur, pairs)
    check_decode(out, spec, to_np(inp.q), to_np(inp.k), to_np(inp.v), cur, scale=default_scale(w.head_dim))
