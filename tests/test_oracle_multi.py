"""Pins for the oracle's multi-token query: the T newest tokens of a sequence
attend causally, query t to tokens 0 .. S - T + t of the cache (encorp.ai,
section on EpiCache: block-wise prefill; patricehuetz.fr, introduction:
compatible with block decoding)."""
import math

import numpy as np
import pytest

from oracle import kivi


def _spec(R=8, G=16, d=16, Hq=2, Hkv=1, P=0):
    return kivi.CacheSpec(batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, k_bits=2, v_bits=2, k_group=G,
                          v_group=16 if d >= 16 else d, residual=R, res_capacity=R + G + 64, dtype="f16", sink=P)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _fsum_causal(q, K, V, scale, S, T):
    """Brute-force causal attention of the last T tokens with math.fsum."""
    out = []
    for t in range(T):
        n = S - T + t + 1
        s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[t], K[i])) for i in range(n)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        out.append([math.fsum(e[i] * float(V[i][c]) for i in range(n)) / den for c in range(len(V[0]))])
    return np.array(out)


def test_nothing_quantized_is_causal_attention_on_the_raw_tokens():
    # S < R + G: every token exact, so the block's queries see raw tokens causally
    rng = np.random.default_rng(21)
    S, T, d = 20, 5, 16
    K, V = _f16(rng.standard_normal((S, d)) * 2), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 2, T, d)))
    out = kivi.decode_attention_multi(_spec(R=8, G=16), q, K[None, None], V[None, None], [S], T, scale=0.3)
    for hq in range(2):
        ref = _fsum_causal(q[0, hq], K, V, 0.3, S, T)
        assert np.max(np.abs(out[0, hq] - ref)) < 1e-12


@pytest.mark.parametrize("P", [0, 3])
def test_last_query_is_the_single_token_decode(P):
    rng = np.random.default_rng(22)
    S, T, d = 130, 6, 16
    K, V = _f16(rng.standard_normal((S, d))), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 2, T, d)))
    sp = _spec(P=P)
    multi = kivi.decode_attention_multi(sp, q, K[None, None], V[None, None], [S], T)
    single = kivi.decode_attention(sp, q[:, :, T - 1], K[None, None], V[None, None], [S])
    assert np.max(np.abs(multi[:, :, T - 1] - single)) < 1e-13


def test_a_token_is_seen_from_its_own_query_on():
    # a dominant key at position S - T + 2 (in the exact window): queries 0 and 1
    # do not see it, queries 2.. return its value
    rng = np.random.default_rng(23)
    S, T, d = 100, 5, 16
    K = _f16(rng.standard_normal((S, d)) * 0.1)
    V = _f16(rng.standard_normal((S, d)))
    pos = S - T + 2
    K[pos] = _f16(np.full(d, 8.0))
    q = _f16(np.full((1, 2, T, d), 8.0))
    sp = _spec(R=8, G=16)
    out = kivi.decode_attention_multi(sp, q, K[None, None], V[None, None], [S], T, scale=1.0)
    for t in range(T):
        if t < 2:
            assert np.max(np.abs(out[0, 0, t] - V[pos])) > 1e-2
        else:
            assert np.max(np.abs(out[0, 0, t] - V[pos])) < 1e-12
    # and the earlier queries equal the attention of the cache without that token
    K2, V2 = K.copy(), V.copy()
    K2[pos] = _f16(np.full(d, -8.0))   # now it gets no weight from any query
    out2 = kivi.decode_attention_multi(sp, q, K2[None, None], V2[None, None], [S], T, scale=1.0)
    assert np.max(np.abs(out[0, :, :2] - out2[0, :, :2])) < 1e-12


def test_quantized_blocks_are_seen_by_every_query():
    # with T <= R the block's tokens are all in the window, so every query sees
    # the same dequantized blocks: query t equals attention over the first
    # S - T + t + 1 rows of the one cache state
    rng = np.random.default_rng(24)
    S, T, d = 200, 4, 16
    K, V = _f16(rng.standard_normal((S, d))), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 2, T, d)))
    sp = _spec(R=8, G=16)
    _, Q, r = kivi.stream_split(sp, S)
    assert Q > 0 and r >= T
    out = kivi.decode_attention_multi(sp, q, K[None, None], V[None, None], [S], T)
    Kh, Vh = kivi.pair_cache_fp64(sp, K, V, S)
    for t in range(T):
        ref = kivi.attention_fp64(q[0, :, t], Kh[:S - T + t + 1], Vh[:S - T + t + 1], 1 / math.sqrt(d))
        assert np.max(np.abs(out[0, :, t] - ref)) < 1e-13


def test_short_sequence_queries_without_tokens_are_zero():
    rng = np.random.default_rng(25)
    S, T, d = 2, 4, 16
    K, V = _f16(rng.standard_normal((S, d))), _f16(rng.standard_normal((S, d)))
    q = _f16(rng.standard_normal((1, 2, T, d)))
    out = kivi.decode_attention_multi(_spec(), q, K[None, None], V[None, None], [S], T)
    assert np.all(out[0, :, :2] == 0.0)
    assert np.allclose(out[0, :, 2], V[0], atol=1e-12)   # one token seen: its value
