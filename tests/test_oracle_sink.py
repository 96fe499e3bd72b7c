"""Pins for the oracle's attention sink: the first P tokens of a sequence stay
in full precision, and quantization and the residual window act on the rest as
if the sequence began at token P (zubnet.ai survey, paragraph on the eviction
family: StreamingLLM's sink tokens plus recent window; encorp.ai, section on
OSCAR: sink and recent tokens in BF16, historical tokens in INT2)."""
import math

import numpy as np
import pytest

from oracle import kivi


def _spec(P, R=4, G=16, d=16, bits=2, Hq=1, Hkv=1):
    return kivi.CacheSpec(batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, k_bits=bits, v_bits=bits,
                          k_group=G, v_group=16 if d >= 16 else d, residual=R, res_capacity=R + G + 64,
                          dtype="f16", sink=P)


def _fsum_attention(q, K, V, scale):
    """Brute-force softmax attention with Python floats and math.fsum."""
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q, k)) for k in K]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    den = math.fsum(e)
    return np.array([math.fsum(e[t] * float(V[t][c]) for t in range(len(K))) / den for c in range(len(V[0]))])


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def test_stream_split_hand_cases():
    sp = _spec(P=4, R=4, G=2)
    # (S) -> (sink tokens, quantized tokens after the sink, ring tokens)
    want = {0: (0, 0, 0), 3: (3, 0, 0), 4: (4, 0, 0), 9: (4, 0, 5), 10: (4, 2, 4), 11: (4, 2, 5), 12: (4, 4, 4)}
    for S, exp in want.items():
        assert kivi.stream_split(sp, S) == exp, S
    # ring slots: tokens P+Q .. S-1 live at (t - P) mod C
    assert list(kivi.ring_slots(2, 10, 6, sink=4)) == [2, 3, 4, 5]
    assert list(kivi.ring_slots(4, 14, 6, sink=4)) == [4, 5, 0, 1, 2, 3]
    assert list(kivi.ring_slots(0, 3, 6, sink=4)) == []


@pytest.mark.parametrize("P,R,G", [(0, 8, 16), (1, 8, 16), (4, 0, 16), (5, 16, 32), (64, 128, 32)])
def test_stream_split_invariants(P, R, G):
    sp = _spec(P=P, R=R, G=G)
    for S in range(0, 400):
        s, Q, r = kivi.stream_split(sp, S)
        assert s + Q + r == S and s == min(S, P) and Q % G == 0
        if S - P >= R:
            assert R <= r < R + G
        else:
            assert Q == 0 and r == max(S - P, 0)
    # no sink: the plain KIVI window
    if P == 0:
        assert all(kivi.stream_split(sp, S)[1] == kivi.quantized_prefix(S, R, G) for S in range(400))


@pytest.mark.parametrize("P,S", [(1, 70), (4, 100), (7, 37), (16, 200)])
def test_sink_shifts_the_quantized_blocks(P, S):
    rng = np.random.default_rng(P * 1000 + S)
    K = _f16(rng.standard_normal((S, 16)) * 2)
    V = _f16(rng.standard_normal((S, 16)))
    with_sink = kivi.expected_blocks(_spec(P=P), K, V, S)
    shifted = kivi.expected_blocks(_spec(P=0), K[P:], V[P:], S - P)
    assert with_sink.shape == shifted.shape and np.array_equal(with_sink, shifted)
    # and the offset matters: the same stream without a sink quantizes other tokens
    unshifted = kivi.expected_blocks(_spec(P=0), K, V, S)
    n = min(len(unshifted), len(with_sink))
    assert n > 0 and not np.array_equal(unshifted[:n], with_sink[:n])


def test_all_sink_is_exact_attention():
    # every token in the sink: the output is softmax attention on the raw tokens
    rng = np.random.default_rng(11)
    S, d = 40, 16
    K, V = _f16(rng.standard_normal((S, d)) * 2), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 1, d)))
    sp = _spec(P=64, R=0, G=16)
    out = kivi.decode_attention(sp, q, K[None, None], V[None, None], [S], scale=0.25)
    ref = _fsum_attention(q[0, 0], K, V, 0.25)
    assert np.max(np.abs(out[0, 0] - ref)) < 1e-12
    # with no sink and R = 0 the same stream is quantized, and the output moves
    out0 = kivi.decode_attention(_spec(P=0, R=0, G=16), q, K[None, None], V[None, None], [S], scale=0.25)
    assert np.max(np.abs(out0[0, 0] - ref)) > 1e-3


def test_equal_keys_give_the_exact_value_mean():
    # identical keys: uniform weights, so the output is the mean of the value
    # rows; the sink's rows enter exactly (INT2 cannot represent these values)
    rng = np.random.default_rng(12)
    S, d, P = 48, 16, 48
    K = np.tile(_f16(rng.standard_normal((1, d))), (S, 1))
    V = _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 1, d)))
    out = kivi.decode_attention(_spec(P=P, R=0, G=16), q, K[None, None], V[None, None], [S])
    assert np.max(np.abs(out[0, 0] - V.astype(np.float64).mean(axis=0))) < 1e-13


def test_dominant_sink_key_returns_its_exact_value():
    # token 1 sits in a 2-token sink and its key dominates every score: the
    # output is its value as stored, not a dequantized one
    rng = np.random.default_rng(13)
    S, d = 100, 16
    K = _f16(rng.standard_normal((S, d)) * 0.1)
    V = _f16(rng.standard_normal((S, d)))
    K[1] = _f16(np.full(d, 8.0))
    q = _f16(np.full((1, 1, d), 8.0))
    out = kivi.decode_attention(_spec(P=2, R=8, G=16), q, K[None, None], V[None, None], [S], scale=1.0)
    assert np.max(np.abs(out[0, 0] - V[1])) < 1e-12
    # without the sink, token 1 is quantized with its block and the output is its dequantized value
    out0 = kivi.decode_attention(_spec(P=0, R=8, G=16), q, K[None, None], V[None, None], [S], scale=1.0)
    assert np.max(np.abs(out0[0, 0] - V[1])) > 1e-2


def test_sink_zero_changes_nothing():
    rng = np.random.default_rng(14)
    S, d = 90, 16
    K, V = _f16(rng.standard_normal((S, d))), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 1, d)))
    a = kivi.decode_attention(_spec(P=0), q, K[None, None], V[None, None], [S])
    sp = _spec(P=0)
    b = kivi.attention_fp64(q[0], *kivi.pair_cache_fp64(sp, K, V, S), 1 / math.sqrt(d))
    assert np.array_equal(a[0], b)
    assert kivi.stream_split(sp, S) == (0, kivi.quantized_prefix(S, sp.residual, sp.k_group),
                                        S - kivi.quantized_prefix(S, sp.residual, sp.k_group))
