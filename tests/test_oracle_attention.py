"""Pins for the oracle's attention, residual window, cache sizes and closed form."""
import json
import math
import os

import numpy as np
import pytest

from oracle import kivi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fsum_attention(q, K, V, scale):
    """Brute-force softmax attention with Python floats and math.fsum."""
    out = []
    for qi in q:
        s = [scale * math.fsum(float(a) * float(b) for a, b in zip(qi, k)) for k in K]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        out.append([math.fsum(e[t] * float(V[t][c]) for t in range(len(K))) / den
                    for c in range(len(V[0]))])
    return np.array(out)


@pytest.mark.parametrize("T,d,n", [(1, 4, 1), (3, 8, 2), (8, 8, 4), (5, 2, 3)])
def test_attention_matches_brute_force(T, d, n):
    rng = np.random.default_rng(T * 100 + d)
    q, K, V = rng.standard_normal((n, d)), rng.standard_normal((T, d)) * 3, rng.standard_normal((T, d))
    got = kivi.attention_fp64(q, K, V, 1 / math.sqrt(d))
    ref = _fsum_attention(q, K, V, 1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    K, V = rng.standard_normal((7, 8)), rng.standard_normal((7, 8))
    # zero query: uniform weights -> mean of the value rows
    assert np.allclose(kivi.attention_fp64(np.zeros((1, 8)), K, V, 0.3)[0], V.mean(axis=0), atol=1e-14)
    # one token: the output is that token's value
    assert np.allclose(kivi.attention_fp64(rng.standard_normal((2, 8)), K[:1], V[:1], 0.3), V[:1], atol=1e-15)
    # permuting tokens (keys with their values) changes nothing
    q = rng.standard_normal((3, 8))
    p = rng.permutation(7)
    assert np.allclose(kivi.attention_fp64(q, K, V, 0.3), kivi.attention_fp64(q, K[p], V[p], 0.3), atol=1e-14)


def test_quantized_prefix_policy():
    # after a flush R <= r < R+G (all tokens stay exact while S < R+G)
    assert kivi.quantized_prefix(512, 32, 32) == 480
    assert kivi.quantized_prefix(4096, 128, 32) == 3968
    assert kivi.quantized_prefix(131072, 128, 64) == 130944
    assert kivi.quantized_prefix(128 + 32 - 1, 128, 32) == 0
    assert kivi.quantized_prefix(128 + 32, 128, 32) == 32
    assert kivi.quantized_prefix(5, 128, 32) == 0
    for S in range(0, 600):
        Q = kivi.quantized_prefix(S, 64, 16)
        r = S - Q
        assert Q % 16 == 0 and (r < 64 + 16) and (S < 64 or r >= 64)


def _spec(**kw):
    base = dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=32, k_bits=2, v_bits=2,
                k_group=16, v_group=16, residual=16, res_capacity=32, dtype="f16")
    base.update(kw)
    return kivi.CacheSpec(**base)


def test_short_sequences_are_exact():
    # S < R + G: nothing is quantized, decode attention equals exact attention
    spec = _spec()
    rng = np.random.default_rng(11)
    K = rng.standard_normal((2, 2, 40, 32)).astype(np.float16).astype(np.float32)
    V = rng.standard_normal((2, 2, 40, 32)).astype(np.float16).astype(np.float32)
    q = rng.standard_normal((2, 4, 32)).astype(np.float16).astype(np.float32)
    lens = [31, 1]
    a = kivi.decode_attention(spec, q, K, V, lens)
    b = kivi.exact_attention(spec, q, K, V, lens)
    assert np.max(np.abs(a - b)) < 1e-14
    # one token: the output is that token's value for every query head of the group
    assert np.allclose(a[1, 0], V[1, 0, 0]) and np.allclose(a[1, 3], V[1, 1, 0])


def test_lossless_grid_pins_grouping_axes():
    """Inputs that lie exactly on each group's grid are reconstructed exactly, so
    quantized attention equals exact attention -- but only when keys are grouped
    per channel (over G tokens) and values per token (over G_V channels)."""
    spec = _spec(batch=1, num_q_heads=2, num_kv_heads=1, residual=16, k_bits=2, v_bits=4)
    rng = np.random.default_rng(3)
    S, d, G = 16 * 5 + 16, 32, 16
    K = np.zeros((1, 1, S, d), np.float32)
    V = np.zeros((1, 1, S, d), np.float32)
    for blk in range(S // G):
        for c in range(d):   # key channel c: offset + (c+1)/4 * code, every code used
            codes = rng.permutation(np.arange(G) % 4)
            K[0, 0, blk * G:(blk + 1) * G, c] = (c - 7) * 0.5 + codes * (c + 1) * 0.25
    for t in range(S):       # value token t, group j: offset + step_t * code
        for j in range(d // 16):
            codes = rng.permutation(np.arange(16) % 16)
            V[0, 0, t, j * 16:(j + 1) * 16] = (t % 5) - 2 + codes * 0.125 * (1 + t % 3)
    q = rng.standard_normal((1, 2, d)).astype(np.float16).astype(np.float32)
    a = kivi.decode_attention(spec, q, K, V, [S])
    b = kivi.exact_attention(spec, q, K, V, [S])
    assert kivi.quantized_prefix(S, 16, 16) == 80
    assert np.max(np.abs(a - b)) < 1e-12
    # grouping keys per token instead would not be lossless on this input
    s_tok, z_tok, c_tok = kivi.quantize_groups(K[0, 0, :16], 2, axis=1)
    rec = kivi.dequantize(c_tok, s_tok.astype(np.float64)[:, None], z_tok.astype(np.float64)[:, None])
    assert np.max(np.abs(rec - K[0, 0, :16])) > 0.1


def test_quantized_attention_error_is_small_and_nonzero():
    # fidelity trade: INT2 changes the output, but by a bounded amount
    spec = _spec(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=64, k_group=32, v_group=32,
                 residual=32, res_capacity=64)
    rng = np.random.default_rng(0)
    K = rng.standard_normal((1, 1, 512, 64)).astype(np.float16).astype(np.float32)
    V = rng.standard_normal((1, 1, 512, 64)).astype(np.float16).astype(np.float32)
    q = rng.standard_normal((1, 1, 64)).astype(np.float16).astype(np.float32)
    a = kivi.decode_attention(spec, q, K, V, [512])
    b = kivi.exact_attention(spec, q, K, V, [512])
    err = np.max(np.abs(a - b))
    assert 1e-4 < err < 0.5


# --- the memory closed form and the pages' worked numbers -----------------------------

def test_closed_form_reproduces_the_pages_figures():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    m = fig["kv_bytes_per_token_70b_bf16"]["model"]
    per_tok = kivi.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], 1, m["bytes_per_element"])
    assert per_tok == 327680
    assert round(per_tok / 2 ** 20, 2) == fig["kv_bytes_per_token_70b_bf16"]["value_mb"]
    t128 = fig["kv_bytes_128k_70b"]["tokens"]
    tot = kivi.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], t128, 2)
    assert tot / 2 ** 30 == fig["kv_bytes_128k_70b"]["value_gb"]
    assert round(tot / 1e9) == 43 and int(tot / 1e9) == fig["kv_bytes_128k_70b_results_section"]["value_gb"]
    t1m = fig["kv_bytes_1m_70b_lower_bound"]["tokens"]
    assert kivi.kv_cache_bytes(m["layers"], m["kv_heads"], m["head_dim"], t1m, 2) / 1e9 > \
        fig["kv_bytes_1m_70b_lower_bound"]["value_gb_more_than"]
    # counting 64 query heads instead of 8 KV heads would not give 0.31 MB
    assert kivi.kv_cache_bytes(80, 64, 128, 1, 2) / 2 ** 20 > 2.0


def test_residual_window_default_matches_the_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    R = fig["residual_window_tokens"]["value"]
    # with R = 128 and G = 32 the last 128..159 tokens stay exact
    for S in (4096, 4100, 4127):
        assert 128 <= S - kivi.quantized_prefix(S, R, 32) < 160


def test_paged_block_matches_the_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    spec = kivi.CacheSpec(1, 48, 8, 128, 4, 2, fig["paged_block_tokens"]["value"], 32, 64, 128, "bf16")
    assert kivi.record_bytes(spec) == 2304 and kivi.record_bytes(spec) % 16 == 0
