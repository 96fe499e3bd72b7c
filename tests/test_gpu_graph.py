"""A decode step (fused append+flush, then decode attention) captured once in
a HIP graph and replayed step after step must give, at every replay, the
output the same calls give eagerly on a twin cache, bit for bit; the records
it leaves must match the oracle's. The captured calls take a fixed
max_seq_tokens and workspace: the host-side length bound does not advance on
a replay."""
import pytest
import torch

from quantized_kv_cache_append_amd import workloads as W

from kvq_harness import check_decode, check_records, default_scale, make_cache, spec_of, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides, lengths, rotate)
    "mha-int2": ("llama2-7b-layer", dict(batch=3, num_q_heads=4, num_kv_heads=4), [300, 95, 1000], 0),
    "paged-ng6": ("ragged-paged", dict(batch=3, num_q_heads=12, num_kv_heads=2), [37, 300, 1111], 0),
    "70b-rotated": ("llama-70b-128k-80layer", dict(batch=2, num_q_heads=16, num_kv_heads=2, layers=1),
                    [1000, 160], 3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_steps(name):
    wname, over, lengths, rot = CASES[name]
    w = W.WORKLOADS[wname].replace(**over)
    steps = 40                       # every sequence crosses at least one flush
    full = [s + steps for s in lengths]
    cap = max(full)
    print(f"[graph case {name}] lengths={lengths} steps={steps}", flush=True)
    inp = W.make_layer(w, device="cpu", seed=31, lengths=full)
    A = make_cache(w, lengths, 256, extra_tokens=steps, rotate=rot)    # replayed graph
    E = make_cache(w, lengths, 256, extra_tokens=steps, rotate=rot)    # eager twin
    warm = make_cache(w, lengths, 256, extra_tokens=steps, rotate=rot)
    for c in (A, E, warm):
        c.prefill(inp.k.cuda(), inp.v.cuda(), lengths, 256)
    kv_shape = (w.batch, w.num_kv_heads, 1, w.head_dim)
    kn = torch.zeros(kv_shape, dtype=w.torch_dtype, device="cuda")
    vn = torch.zeros(kv_shape, dtype=w.torch_dtype, device="cuda")
    q = torch.zeros(w.batch, w.num_q_heads, w.head_dim, dtype=w.torch_dtype, device="cuda")
    out_a = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    ws_a = torch.empty(A.workspace_bytes(cap), dtype=torch.uint8, device="cuda")
    # first calls outside the capture (one-time kernel set-up)
    warm.append_flush(kn, vn)
    warm.decode(q, max_seq_tokens=cap)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.append_flush(kn, vn)
        A.decode(q, out=out_a, max_seq_tokens=cap, workspace=ws_a)
    torch.cuda.synchronize()

    spec = spec_of(w, A.cfg.res_capacity, rotate=rot)
    k_np, v_np = to_np(inp.k), to_np(inp.v)
    for st in range(steps):
        idx = [s + st for s in lengths]
        kn.copy_(torch.stack([inp.k[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]))
        vn.copy_(torch.stack([inp.v[b, :, idx[b]:idx[b] + 1] for b in range(w.batch)]))
        q.copy_(W.new_tokens(w, inp, 1, device="cpu", seed=31, step=st)[2])
        g.replay()
        E.append_flush(kn, vn)
        out_e = E.decode(q, max_seq_tokens=cap)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_e), f"replay {st} differs from the eager step"
        if st in (0, steps - 1):
            check_decode(out_a, spec, to_np(q), k_np, v_np, [s + st + 1 for s in lengths],
                         scale=default_scale(w.head_dim))
    assert A.read_device_error() == 0 and E.read_device_error() == 0
    assert A.lengths() == E.lengths()
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    check_records(A, spec, k_np, v_np, full, pairs)
