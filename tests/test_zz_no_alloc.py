"""The decode entry point that allocates nothing (kvq_decode_attention_noalloc,
for callers that cannot allocate) against kvq_decode_attention with a
caller-provided workspace, through the C ABI: equal bit for bit (the same
kernels and the same work partition), on calls in a row whose inputs shrink,
so that the second call reuses the array the first one filled."""
import ctypes

import pytest
import torch

from quantized_kv_cache_append_amd import binding as B
from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import make_cache

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))


def _decode_both(w, lengths, seed):
    print(f"[no-alloc] {w.name} B={w.batch} H_q={w.num_q_heads} H_kv={w.num_kv_heads} lengths={lengths}", flush=True)
    inp = W.make_layer(w, device="cuda", seed=seed, lengths=lengths)
    cache = make_cache(w, lengths, 256)
    cache.prefill(inp.k, inp.v, lengths, 256)
    msl = max(lengths)
    ref = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    ws = torch.empty(cache.workspace_bytes(msl), dtype=torch.uint8, device="cuda")
    B.kvq_decode_attention(cache.cfg, cache.cache, inp.q.data_ptr(), ref.data_ptr(), 0.0, msl, ws.data_ptr(),
                           ws.numel(), _stream())
    out = torch.full_like(ref, float("nan"))
    B.kvq_decode_attention_noalloc(cache.cfg, cache.cache, inp.q.data_ptr(), out.data_ptr(), 0.0, msl, _stream())
    torch.cuda.synchronize()
    assert cache.read_device_error() == 0
    return ref, out


def test_noalloc_decode_equals_the_workspace_call_on_shrinking_inputs():
    gqa = W.WORKLOADS["llama3-8b-gqa-int2"]
    cases = [
        (gqa.replace(batch=6, num_q_heads=16, num_kv_heads=4), [3000, 129, 2048, 4100, 700, 1]),
        (W.WORKLOADS["llama2-7b-layer"].replace(batch=3, num_q_heads=4, num_kv_heads=4), [1100, 40, 600]),
        (gqa.replace(batch=2, num_q_heads=8, num_kv_heads=2), [300, 157]),
    ]
    for i, (w, lengths) in enumerate(cases):
        ref, out = _decode_both(w, lengths, seed=50 + i)
        assert torch.isfinite(out).all()
        assert torch.equal(ref, out), f"case {i}: max abs diff {float((ref - out).abs().max()):.3e}"
