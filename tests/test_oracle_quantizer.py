"""Pins for the oracle's quantizer (formula F) and packing, independent of the oracle.

Each check fixes the oracle to something other than itself: hand-derived
values, the exact-rational nearest code, invariants that the asymmetric min/max
quantizer must satisfy, and the packing density the pages print.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kivi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --- hand-derived cases (the pages print no worked quantization example) -----------

def test_hand_case_int2_tie_goes_to_even():
    # min -1, max 2: range 3, scale 3/3 = 1, zero -1; (x - z)/s = 0, 1, 1.5, 3.
    # 1.5 is a tie between codes 1 and 2 and goes to the even code 2.
    s, z, c = kivi.quantize_groups(np.array([-1, 0, 0.5, 2], np.float32), 2, axis=0)
    assert float(s) == 1.0 and float(z) == -1.0
    assert c.tolist() == [0, 1, 2, 3]


def test_hand_case_int2_tie_two_and_a_half():
    # (x - z)/s = 0, 2.5, 3 -> 2.5 ties between 2 and 3 and goes to 2.
    s, z, c = kivi.quantize_groups(np.array([-1, 1.5, 2], np.float32), 2, axis=0)
    assert c.tolist() == [0, 2, 3]


def test_hand_case_int4_identity_and_tie():
    x = np.arange(16, dtype=np.float32)
    s, z, c = kivi.quantize_groups(x, 4, axis=0)
    assert float(s) == 1.0 and float(z) == 0.0 and c.tolist() == list(range(16))
    # 0, 7.5, 15: scale 1, 7.5 -> 8 (even)
    s, z, c = kivi.quantize_groups(np.array([0, 7.5, 15], np.float32), 4, axis=0)
    assert c.tolist() == [0, 8, 15]


def test_hand_case_constant_group_has_zero_scale_and_codes():
    s, z, c = kivi.quantize_groups(np.full(32, 0.75, np.float32), 2, axis=0)
    assert float(s) == 0.0 and float(z) == 0.75 and not c.any()


def test_hand_case_fp16_scale_rounding():
    # range 1 over 3 steps: fp32(1/3) = 0x3EAAAAAB, fp16 nearest is 1365/4096.
    s, z, c = kivi.quantize_groups(np.array([0.0, 0.25, 1.0], np.float32), 2, axis=0)
    assert Fraction(float(s)) == Fraction(1365, 4096)
    # 0.25 / (1365/4096) = 0.7503 -> 1 ; 1.0 -> 3.0007 -> clamps at 3
    assert c.tolist() == [0, 1, 3]


def test_axis_selects_the_group():
    # Keys are grouped per channel over tokens: axis 0 of [tokens][channels].
    x = np.array([[0, 10], [3, 10], [1, 40]], np.float32)   # 3 tokens, 2 channels
    s, z, c = kivi.quantize_groups(x, 2, axis=0)
    assert s.tolist() == [1.0, 10.0] and z.tolist() == [0.0, 10.0]
    assert c[:, 0].tolist() == [0, 3, 1] and c[:, 1].tolist() == [0, 0, 3]


# --- the exact nearest code, brute force ---------------------------------------------

def _nearest_code_exact(x, s16, z16, qmax):
    """argmin over codes of |x - (z + c*s)| in exact rationals (ties -> even)."""
    best = None
    for cand in range(qmax + 1):
        err = abs(Fraction(float(x)) - (Fraction(float(z16)) + cand * Fraction(float(s16))))
        if best is None or err < best[0] or (err == best[0] and cand % 2 == 0):
            best = (err, cand)
    return best[1]


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_the_exact_nearest_level(bits):
    rng = np.random.default_rng(123)
    qmax = 2 ** bits - 1
    n_checked = 0
    for _ in range(60):
        x = (rng.standard_normal(16) * rng.uniform(0.01, 50)).astype(np.float16).astype(np.float32)
        s, z, c = kivi.quantize_groups(x, bits, axis=0)
        # zero-point: the fp16 value of the exact minimum (fp16 inputs: exact)
        assert float(z) == float(x.min())
        # scale: within one fp16 rounding (plus one fp32 rounding) of (max-min)/qmax
        exact_s = (Fraction(float(x.max())) - Fraction(float(x.min()))) / qmax
        ulp = Fraction(2) ** (int(np.floor(np.log2(float(exact_s)))) - 10)
        assert abs(Fraction(float(s)) - exact_s) <= ulp / 2 * (1 + Fraction(1, 2 ** 12))
        for xi, ci in zip(x, c):
            t = (Fraction(float(xi)) - Fraction(float(z))) / Fraction(float(s))
            frac = t - int(t)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 5):
                continue  # a near-tie: fp32 rounding of t legitimately decides
            n_checked += 1
            assert int(ci) == _nearest_code_exact(xi, s, z, qmax)
    assert n_checked > 800


# --- invariants over many random groups ----------------------------------------------

@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_invariants_random_groups(bits, dtype):
    rng = np.random.default_rng(7 + bits)
    n_groups, gsz = 20000, 32
    scale = np.exp(rng.standard_normal((n_groups, 1)) * 2.0)
    x = (rng.standard_normal((n_groups, gsz)) * scale).astype(np.float32)
    if dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
    else:  # bf16: keep the top 16 bits, rounding to nearest even
        u = x.view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        x = u.astype(np.uint32).view(np.float32)
    s, z, c = kivi.quantize_groups(x, bits, axis=1)
    qmax = 2 ** bits - 1
    assert c.min() >= 0 and c.max() <= qmax
    s64 = s.astype(np.float64)[:, None]
    xhat = kivi.dequantize(c, s.astype(np.float64)[:, None], z.astype(np.float64)[:, None])
    normal = (s.astype(np.float64) >= 2.0 ** -14)[:, None]
    err = np.abs(x.astype(np.float64) - xhat)
    # |x - x_hat| <= scale/2 (tiny slack for the fp32 rounding of t)
    assert np.all(err[normal[:, 0]] <= s64[normal[:, 0]] * (0.5 + 1e-5))
    # the group minimum gets code 0 and is reconstructed exactly
    amin = x.argmin(axis=1)
    assert np.all(c[np.arange(n_groups), amin] == 0)
    assert np.all(xhat[np.arange(n_groups), amin] == x[np.arange(n_groups), amin])
    # the group maximum gets the top code when the scale is a normal fp16
    amax = x.argmax(axis=1)
    top = c[np.arange(n_groups), amax]
    assert np.all(top[normal[:, 0] & (s > 0)] == qmax)


# --- packing --------------------------------------------------------------------------

def test_packing_density_matches_the_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["codes_per_uint32"]
    for bits, key in ((4, "int4"), (2, "int2")):
        codes = np.zeros((1, fig[key]), np.uint8)
        assert kivi.pack_lsb_first(codes, bits).shape == (1, 1)


def test_pack_hand_words():
    c = np.zeros(16, np.uint8)
    c[15] = 3
    assert kivi.pack_lsb_first(c, 2)[0] == 0xC0000000
    c = np.zeros(8, np.uint8)
    c[0] = 15
    assert kivi.pack_lsb_first(c, 4)[0] == 0x0000000F
    assert kivi.pack_lsb_first(np.arange(16) % 4, 2)[0] == 0xE4E4E4E4
    assert kivi.pack_lsb_first(np.arange(8), 4)[0] == 0x76543210


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(bits)
    c = rng.integers(0, 2 ** bits, size=(5, 7, 64)).astype(np.uint8)
    w = kivi.pack_lsb_first(c, bits)
    assert w.shape == (5, 7, 64 * bits // 32)
    assert np.array_equal(kivi.unpack_lsb_first(w, bits), c)


# --- block record layout, by hand -----------------------------------------------------

def _tiny_spec(kb=2, vb=2):
    return kivi.CacheSpec(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=16,
                          k_bits=kb, v_bits=vb, k_group=16, v_group=16,
                          residual=0, res_capacity=32, dtype="f16")


def test_record_layout_hand_offsets():
    spec = _tiny_spec()
    K = np.zeros((16, 16), np.float32)
    V = np.zeros((16, 16), np.float32)
    K[1, 0] = 3.0      # channel 0: values 0..3 -> scale 1, code 3 at token 1
    K[0, 15] = 3.0     # channel 15: code 3 at token 0
    V[2, 5] = 3.0      # token 2, group 0 (channels 0..15): code 3 at channel 5
    rec = kivi.block_to_bytes(kivi.quantize_block(spec, K, V))
    # K codes: 16 tokens x 1 word; K scale 16 fp16; K zero 16 fp16;
    # V codes: 16 channels x 1 word; V scale 1x16 fp16; V zero 1x16 fp16
    assert rec.size == 64 + 32 + 32 + 64 + 32 + 32 == kivi.record_bytes(spec)
    w = rec[:64].view(np.uint32)
    assert w[0] == 0xC0000000 and w[1] == 0x00000003 and not w[2:].any()
    ks = rec[64:96].view(np.float16)
    assert ks[0] == 1.0 and ks[15] == 1.0 and not ks[1:15].any()
    # V codes, 8-token chunks: (t=2, c=5) at position ((0*16 + 5)*1 + 0)*8 + 2 = 42
    # -> bit 84 -> word 2, bit 20
    vw = rec[128:192].view(np.uint32)
    assert vw[2] == (3 << 20) and not np.delete(vw, 2).any()
    vs = rec[192:224].view(np.float16)
    assert vs[2] == 1.0 and not np.delete(vs, 2).any()


def test_record_sizes_per_token_match_the_design_table():
    # bytes per token per kv head: codes + fp16 scale/zero
    cases = [((2, 2, 32, 32), 96), ((4, 4, 32, 32), 160), ((2, 2, 64, 64), 80), ((4, 2, 16, 32), 144)]
    for (kb, vb, G, gv), per_tok in cases:
        spec = kivi.CacheSpec(1, 1, 1, 128, kb, vb, G, gv, 128, 256, "bf16")
        assert kivi.record_bytes(spec) == per_tok * G
        # the same figure from the layout's parts, per token: d*(b_K + b_V)/8 code bytes,
        # 2*2*d/G bytes of key scale/zero shared by the block, 2*2*d/G_V of value scale/zero
        assert kivi.quantized_bytes_per_token(spec) == 128 * (kb + vb) / 8 + 4 * 128 / G + 4 * 128 / gv == per_tok


def test_code_bandwidth_divisor_matches_the_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["code_bandwidth_divisor_vs_fp16"]
    for bits, key in ((4, "int4"), (2, "int2")):
        spec = kivi.CacheSpec(1, 1, 1, 128, bits, bits, 32, 32, 128, 256, "f16")
        codes = kivi.record_sections(spec)["k_codes"] + kivi.record_sections(spec)["v_codes"]
        fp16 = 2 * 32 * 128 * 2
        assert fp16 / codes == fig[key]


def test_record_layout_value_scales_are_group_major():
    # d = 32, G_V = 16: two value groups per token. Token 2, channel 21 (group 1)
    # holds the only non-zero value, so only scale[group 1][token 2] is non-zero.
    spec = kivi.CacheSpec(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=32, k_bits=4, v_bits=2,
                          k_group=16, v_group=16, residual=0, res_capacity=32, dtype="f16")
    K = np.zeros((16, 32), np.float32)
    V = np.zeros((16, 32), np.float32)
    V[2, 21] = 1.5
    rec = kivi.block_to_bytes(kivi.quantize_block(spec, K, V))
    kc = 16 * 32 * 4 // 8            # 256 B of key codes (4 words per token)
    vc_off = kc + 2 * 64             # after key scale and zero (32 fp16 each)
    # (t=2, c=21): position ((0*16 + 5)*2 + 1)*8 + 2 = 90 -> bit 180 -> word 5, bit 20
    vw = rec[vc_off:vc_off + 32 * 4].view(np.uint32)
    assert vw[5] == (3 << 20) and not np.delete(vw, 5).any()
    vs = rec[vc_off + 128:vc_off + 128 + 64].view(np.float16).reshape(2, 16)
    assert vs[1, 2] == np.float16(0.5) and np.count_nonzero(vs) == 1
    vz = rec[vc_off + 192:vc_off + 256].view(np.float16)
    assert not vz.any()


def test_record_layout_value_codes_second_token_chunk_int4():
    # G = 16, d = 16, 4-bit values: token 9 (second 8-token chunk), channel 3.
    spec = _tiny_spec(kb=2, vb=4)
    K = np.zeros((16, 16), np.float32)
    V = np.zeros((16, 16), np.float32)
    V[9, 3] = 15.0                  # group of token 9: range 15 over 15 steps -> code 15
    rec = kivi.block_to_bytes(kivi.quantize_block(spec, K, V))
    vc_off = 64 + 32 + 32           # after 16 key words and key scale/zero
    vw = rec[vc_off:vc_off + 128].view(np.uint32)   # 16 tokens x 16 channels x 4 bits
    # position ((1*16 + 3)*1 + 0)*8 + 1 = 153 -> bit 612 -> word 19, bit 4
    assert vw[19] == (15 << 4) and not np.delete(vw, 19).any()


@pytest.mark.parametrize("kb,vb,G,gv", [(2, 2, 32, 32), (4, 4, 32, 32), (2, 2, 64, 64), (4, 2, 16, 32)])
def test_blocks_at_once_equal_blocks_one_by_one(kb, vb, G, gv):
    # quantize_block over a leading block axis takes the same steps on each block
    rng = np.random.default_rng(7)
    spec = kivi.CacheSpec(1, 1, 1, 128, kb, vb, G, gv, 128, 128 + G, "bf16")
    k = (rng.standard_normal((5, G, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    v = rng.standard_normal((5, G, 128)).astype(np.float32)
    k[2] = 1.5   # a constant block: zero scales and codes
    many = kivi.block_to_bytes(kivi.quantize_block(spec, k, v))
    one = np.stack([kivi.block_to_bytes(kivi.quantize_block(spec, k[j], v[j])) for j in range(5)])
    assert many.shape == (5, kivi.record_bytes(spec)) and np.array_equal(many, one)
    kh, vh = kivi.dequantize_block(spec, kivi.quantize_block(spec, k, v))
    for j in range(5):
        kj, vj = kivi.dequantize_block(spec, kivi.quantize_block(spec, k[j], v[j]))
        assert np.array_equal(kh[j], kj) and np.array_equal(vh[j], vj)
