"""Why the matrix-core decode kernels split their real-valued operands in two.

The GQA kernel contracts the exact integer codes with q~ = q' * s_K (scores)
and with p~ = p * s_V (outputs) on bf16 MFMAs. Each real operand is split into
a bf16 high part and a bf16 remainder (about 16 significant bits). These CPU
tests emulate the alternatives on the workloads' own inputs, with every other
step exact (fp64 over the oracle's dequantized cache), and pin that:

- the hi/lo split stays far inside the decode tolerance (max-abs 2e-3);
- one fp16 operand (11 bits) for q~, or for p~, does not.

The quantized blocks come from the oracle's formula F (KIVI: keys per channel,
values per token), the inputs from the seeded workload generators.
"""
import math

import numpy as np
import pytest

from oracle import kivi
from quantized_kv_cache_append_amd import workloads as W
from tests.kvq_harness import ATOL, spec_of


def _bf16(x):
    """Round float32 values to bf16 (nearest, ties to even), returned as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _hi_lo(x):
    x = np.asarray(x, np.float32)
    hi = _bf16(x)
    return hi.astype(np.float64) + _bf16(x - hi).astype(np.float64)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def _worst_error(name, lengths, pairs, q_op, p_op, lag=7.5):
    """Max-abs error of decode attention whose quantized share uses q_op(q~) for
    the scores and p_op(p~) for the outputs, against fp64 on the same cache.
    The probabilities are taken against a running maximum `lag` below the true
    one (the kernels move it lazily, so p reaches up to 2^8)."""
    w = W.WORKLOADS[name]
    spec = spec_of(w, w.residual + w.k_group)
    inp = W.make_layer(w, "cpu", 0, 0, lengths=lengths)
    K, V, q = inp.k.float().numpy(), inp.v.float().numpy(), inp.q.float().numpy()
    d, G, gv, ng = w.head_dim, w.k_group, w.v_group, w.n_g
    scale = np.float32(math.log2(math.e) / math.sqrt(d))
    worst = 0.0
    for b, h in pairs:
        S = lengths[b]
        _, Q, _ = kivi.stream_split(spec, S)
        nb = Q // G
        sec = kivi.quantize_block(spec, K[b, h, :nb * G].reshape(nb, G, d), V[b, h, :nb * G].reshape(nb, G, d))
        kh, vh = (x.reshape(-1, d) for x in kivi.dequantize_block(spec, sec))
        kc = kivi.unpack_lsb_first(sec["k_codes"], spec.k_bits).astype(np.float64)              # [nb][G][d]
        vc = kivi.value_codes_from_stream(kivi.unpack_lsb_first(sec["v_codes"], spec.v_bits), G, d)
        vc = vc.reshape(-1, d).astype(np.float64)
        vs = np.repeat(np.swapaxes(sec["v_scale"], -1, -2), gv, axis=-1).reshape(-1, d).astype(np.float32)
        vz = np.repeat(np.swapaxes(sec["v_zero"], -1, -2), gv, axis=-1).reshape(-1, d).astype(np.float64)
        kr, vr = K[b, h, nb * G:S].astype(np.float64), V[b, h, nb * G:S].astype(np.float64)
        for hq in range(h * ng, (h + 1) * ng):
            qs = q[b, hq].astype(np.float32) * scale                                              # q' (log2 units)
            s_ex = kh @ qs.astype(np.float64)
            kap = (qs.astype(np.float64)[None, :] * sec["k_zero"].astype(np.float64)).sum(-1)     # q' . z_K per block
            qt = qs[None, :] * sec["k_scale"].astype(np.float32)                                  # q~ per block (fp32)
            s_op = (np.einsum("bgc,bc->bg", kc, q_op(qt)) + kap[:, None]).reshape(-1)
            s_r = kr @ qs.astype(np.float64)
            m = (max(s_ex.max(), s_r.max()) if len(s_r) else s_ex.max()) - lag
            pr = np.exp2(s_r - m)

            def out(sq, split_p):
                pq = np.exp2(sq - m)
                if split_p:
                    o = (p_op(pq.astype(np.float32)[:, None] * vs) * vc).sum(0) + pq @ vz
                else:
                    o = pq @ vh
                return (o + pr @ vr) / (pq.sum() + pr.sum())

            ref = out(s_ex, False)
            worst = max(worst, float(np.abs(out(s_op, True) - ref).max()))
    return worst


def _exact(x):
    return np.asarray(x, np.float64)


@pytest.mark.parametrize("name,lengths,pairs", [
    ("llama3-8b-gqa-int2", [8192] * 4, [(0, 1), (1, 3), (2, 5), (3, 6)]),
    ("llama2-7b-layer", [4096] * 2, [(0, 0), (0, 5), (1, 9), (1, 31)]),
])
def test_hi_lo_split_within_tolerance(name, lengths, pairs):
    err = _worst_error(name, lengths, pairs, _hi_lo, _hi_lo)
    assert err < ATOL / 4, err


def test_single_fp16_query_operand_exceeds_tolerance():
    err = _worst_error("llama3-8b-gqa-int2", [8192] * 4, [(0, 1), (1, 3), (2, 5), (3, 6)], _f16, _exact)
    assert err > ATOL, err


def test_single_fp16_probability_operand_exceeds_tolerance():
    err = _worst_error("llama2-7b-layer", [4096] * 2, [(0, 0), (0, 5), (1, 9), (1, 31)], _exact, _f16)
    assert err > ATOL, err
