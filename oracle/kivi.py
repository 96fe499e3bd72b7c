"""Plain CPU oracle for KIVI-style quantized KV-cache append and decode attention.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import this module. The product path (the HIP library and
its Python binding) never imports it, and this module imports nothing from the
product path: it works on plain numpy arrays.

Written slowly and directly so that a reader can check it against the pages:

  [P2] zubnet.ai -- "KV cache compression techniques for LLM inference
       (H2O, KIVI, MLA, StreamingLLM)", paragraph on the quantization family.
  [P3] encorp.ai -- "La compression du cache KV est une décision
       d'infrastructure, pas un débat sur les modèles", section on HBM, not
       FLOPs, being the ceiling.
  [P4] patricehuetz.fr -- "Quantification du KV-Cache : TurboQuant et l'état de
       l'art en 2026": section "Le problème : le KV-cache, gouffre silencieux"
       (memory formula), section "KIVI (2024) — la quantification asymétrique
       par canal", innovation 3 "Bit-packing dense : INT4 et INT2 en mémoire
       GPU" and innovation 4 "Fenêtre résiduelle".
  [P1] ai-automate.fr -- "KV-cache compressé et modèles 4-bit ...", section on
       Minima-KV (partial attention states merged by an online softmax).
  [P2'] the same zubnet.ai survey, paragraph on the eviction family:
       StreamingLLM keeps the first tokens, which act as attention sinks,
       beside a sliding window of recent ones.
  [P3'] the same encorp.ai page, section "OSCAR compte parce que quelqu'un a
       effectivement livré les parties brouillonnes": OSCAR keeps the sink
       tokens and the recent tokens in BF16 and compresses the historical ones
       to INT2.
  [P1'] the same ai-automate.fr page, section "Minima-KV : la compression sans
       éviction": a mixed-format hierarchy in which recent and protected
       pages stay in FP8 and older pages are compacted to low bits, partial
       attention states of both merged by one online softmax.
  [P3''] the same encorp.ai page, section on EpiCache (long prompts and long
       conversations are different systems problems): block-wise prefill;
       [P4] introduction: compatible with block decoding.

What the pages fix: keys are quantized per channel, values per token [P2; P4
KIVI]; each channel carries its own min/max parameters [P4 KIVI]; codes are
INT2 (or INT4) packed 16 (or 8) to a 32-bit word [P4 innovation 3]; the most
recent tokens stay in full precision [P4 KIVI; P4 innovation 4]; the cache size
is 2*L*H*d*S*bytes [P4 "Le problème"].

What the pages leave open is taken here as follows (each reading is one line
of the readings list kept with the design notes):
  * the quantizer is asymmetric uniform min/max: scale = (max-min)/(2^b-1),
    zero-point = min, x_hat = code*scale + zero; scale and zero are stored as
    fp16;
  * formula F fixes every rounding in fp32: see quantize_groups();
  * a constant group (scale rounds to 0) gets all-zero codes;
  * LSB-first packing: slot i of a word sits at bits [i*b, (i+1)*b);
  * keys are grouped over G consecutive tokens (one block), values over G_V
    consecutive channels of one token;
  * the residual window keeps R <= r < R+G tokens: after a flush, the oldest
    complete G-token blocks beyond R are quantized, so Q = G*floor(max(S-R,0)/G);
  * attention uses softmax scale 1/sqrt(d) by default, query head h' reads kv
    head floor(h'/n_g), and is evaluated in fp64 on the dequantized cache;
  * a multi-token query (block-wise prefill or the check of T drafted
    tokens) [P3''; P4 introduction]: the T newest tokens of a sequence of S
    tokens are queries, and query t (0 <= t < T) attends to tokens
    0 .. S - T + t of the same cache state (causal within the block);
  * an FP8 tier of W blocks (W = 0: none) [P1']: the W most recent quantized
    blocks of a sequence are also kept in FP8 (e4m3, one fp16 scale per token
    row, formula F8 below) and attention reads them there; older blocks are
    read from their low-bit records, which are still quantized from the
    original values;
  * an attention sink of P tokens (P = 0: none) [P2'; P3']: the first min(S, P)
    tokens of a sequence stay in full precision and are never quantized; the
    quantized blocks and the residual window cover the tokens after them,
    exactly as if the sequence started at token P. The pages give no count, so
    P is a parameter;
  * a Walsh-Hadamard pre-rotation (rotate = 0: none; bit 1 keys, bit 2
    values) [P4w]: before formula F every key (and/or value) token vector x of
    d channels is replaced by R(x) = H x / 8, H the d x d Sylvester Hadamard
    matrix, computed in fp32 by radix-2 butterflies in the order of fwht_f32();
    attention reads the dequantized vectors back through H y / (d / 8), R's
    inverse (H H = d I). The page's rotation is orthonormal, H / sqrt(d);
    splitting that factor into the powers of two 1/8 and 8/d keeps both sides
    free of extra rounding, and formula F commutes with a power-of-two scale of
    its group. The residual window and the sink stay in the original
    coordinates.

  [P4w] the same patricehuetz.fr page, "TurboQuant : les cinq innovations",
       innovation 1 "Rotation Walsh-Hadamard : normaliser la distribution": a
       WHT of the key and value vectors before quantization spreads outliers
       over all dimensions; it is orthogonal and is inverted on the
       dequantized vectors when attention is computed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# Configuration of one cache layer (plain data; mirrors the C struct fields).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class CacheSpec:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    k_bits: int
    v_bits: int
    k_group: int          # G: tokens per key group (= tokens per block)
    v_group: int          # G_V: channels per value group
    residual: int         # R
    res_capacity: int     # ring slots per (sequence, kv head)
    dtype: str            # "f16" or "bf16"
    sink: int = 0         # P: leading tokens kept in full precision (attention sink)
    fp8_blocks: int = 0   # W: most recent quantized blocks also kept (and read) in FP8
    rotate: int = 0       # Walsh-Hadamard pre-rotation: bit 1 keys, bit 2 values

    @property
    def n_g(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# ---------------------------------------------------------------------------
# Formula F: asymmetric min/max quantization of one group, fixed in fp32.
# [P4, section "KIVI (2024)"]: every channel (keys) or token (values) has its
# own min/max parameters; the rounding steps are this oracle's reading.
# ---------------------------------------------------------------------------
def quantize_groups(x: np.ndarray, bits: int, axis: int):
    """Quantize groups of a float32 array that lie along `axis`.

    Steps, each an IEEE fp32 operation rounded to nearest-even (no fused
    multiply-add anywhere):
      mn, mx = min, max of the group
      z16 = fp16(mn)                                  (round to nearest even)
      s16 = fp16( fp32(mx - mn) / fp32(2^b - 1) )
      if s16 == 0: every code is 0
      else: inv = fp32(1 / fp32(s16))
            t = fp32( fp32(x - fp32(z16)) * inv )
            code = clamp(round_half_even(t), 0, 2^b - 1)

    Returns (s16, z16, codes) with s16/z16 float16 arrays of the reduced shape
    and codes uint8 of x's shape.
    """
    x = np.asarray(x, dtype=F32)
    qmax = F32(2 ** bits - 1)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    z16 = mn.astype(np.float16)
    s16 = ((mx - mn) / qmax).astype(np.float16)
    s32 = s16.astype(F32)
    z32 = z16.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = F32(1.0) / s32
        t = (x - z32) * inv
        codes = np.clip(np.rint(t), F32(0.0), qmax)
    codes = np.where(s32 == 0, F32(0.0), codes).astype(np.uint8)
    return np.squeeze(s16, axis=axis), np.squeeze(z16, axis=axis), codes


def dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x_hat = code * scale + zero, in fp64 (exact for these operands)."""
    return codes.astype(np.float64) * s16.astype(np.float64) + z16.astype(np.float64)


# ---------------------------------------------------------------------------
# Dense bit-packing [P4, innovation 3]: 32/b codes per uint32, LSB first.
# ---------------------------------------------------------------------------
def pack_lsb_first(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack the last axis of `codes` into uint32 words, slot i at bits [i*b, (i+1)*b)."""
    per = 32 // bits
    c = np.asarray(codes, dtype=np.uint32)
    n = c.shape[-1]
    if n % per:
        raise ValueError(f"last axis {n} is not a multiple of {per}")
    c = c.reshape(c.shape[:-1] + (n // per, per))
    words = np.zeros(c.shape[:-1], dtype=np.uint32)
    for i in range(per):
        words |= (c[..., i] & np.uint32(2 ** bits - 1)) << np.uint32(i * bits)
    return words


def unpack_lsb_first(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_lsb_first: uint32 words -> codes along a longer last axis."""
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty(w.shape + (per,), dtype=np.uint8)
    for i in range(per):
        out[..., i] = (w >> np.uint32(i * bits)) & np.uint32(2 ** bits - 1)
    return out.reshape(w.shape[:-1] + (w.shape[-1] * per,))


# ---------------------------------------------------------------------------
# Walsh-Hadamard pre-rotation [P4w, innovation 1].
# ---------------------------------------------------------------------------
ROT_KEYS, ROT_VALUES = 1, 2
ROT_SHIFT = 3   # the stored side is H x * 2^-3


def hadamard(d: int) -> np.ndarray:
    """The d x d Sylvester Hadamard matrix (d a power of two): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]]. Symmetric, entries +-1, H H = d I."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == d, "d must be a power of two"
    return h


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """H x along the last axis, in float32: for h = 1, 2, 4, ..., d/2, every
    pair (i, i + h) with bit h of i clear becomes (x_i + x_{i+h}, x_i - x_{i+h}),
    each sum rounded to fp32. This order fixes the roundings the stored codes
    depend on."""
    y = np.array(x, dtype=F32)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        t = y.reshape(lead + (d // (2 * h), 2, h))
        a, b = t[..., 0, :], t[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return y


def rotate_f32(x: np.ndarray) -> np.ndarray:
    """R(x) = H x / 8 in float32 (the division by 8 is exact)."""
    return fwht_f32(x) * F32(2.0 ** -ROT_SHIFT)


def unrotate_f64(y: np.ndarray) -> np.ndarray:
    """R's inverse, H y * 8 / d, in fp64 along the last axis."""
    d = y.shape[-1]
    return (np.asarray(y, np.float64) @ hadamard(d).astype(np.float64)) * (2.0 ** ROT_SHIFT / d)


# ---------------------------------------------------------------------------
# One quantized block: G tokens of one (sequence, kv head).
#
# Record layout (little-endian bytes, sections in this order):
#   K codes  uint32 [G][d*b_K/32]      token-major: word w of token t holds
#                                      channels w*32/b_K ... (LSB first)
#   K scale  fp16   [d]                per channel, over the G tokens
#   K zero   fp16   [d]
#   V codes  8-token chunks: the code of (token t, channel c) sits at bit
#            position pos(t, c) * b_V of the section, with
#              pos(t, c) = ((t//8 * 16 + c%16) * (d//16) + c//16) * 8 + t%8,
#            i.e. for each run of 8 tokens, for each c%16, for each c//16, the 8
#            tokens of that channel LSB first (a little-endian uint32 stream)
#   V scale  fp16   [d/G_V][G]         per (channel group, token)
#   V zero   fp16   [d/G_V][G]
# ---------------------------------------------------------------------------
def record_sections(spec: CacheSpec):
    G, d = spec.k_group, spec.head_dim
    kc = G * d * spec.k_bits // 8
    ks = 2 * d
    vc = d * G * spec.v_bits // 8
    vs = 2 * (d // spec.v_group) * G
    return {"k_codes": kc, "k_scale": ks, "k_zero": ks,
            "v_codes": vc, "v_scale": vs, "v_zero": vs}


def record_bytes(spec: CacheSpec) -> int:
    return sum(record_sections(spec).values())


def value_code_order(G: int, d: int) -> np.ndarray:
    """Stream position of every (token, channel) value code, [G][d] -> int."""
    t = np.arange(G)[:, None]
    c = np.arange(d)[None, :]
    return ((t // 8 * 16 + c % 16) * (d // 16) + c // 16) * 8 + t % 8


def value_code_stream(vcodes: np.ndarray) -> np.ndarray:
    """[..., G, d] codes -> stream in record order along the last axis, [..., G*d]
    (see the record layout; leading axes are independent blocks)."""
    G, d = vcodes.shape[-2:]
    lead = vcodes.shape[:-2]
    out = np.empty(lead + (G * d,), dtype=vcodes.dtype)
    out[..., value_code_order(G, d).ravel()] = vcodes.reshape(lead + (G * d,))
    return out


def value_codes_from_stream(stream: np.ndarray, G: int, d: int) -> np.ndarray:
    """[..., G*d] stream -> [..., G, d] codes."""
    return stream[..., value_code_order(G, d)]


def quantize_block(spec: CacheSpec, kblk: np.ndarray, vblk: np.ndarray):
    """Quantize one block. kblk, vblk: float32 [G][d] (exact input values), or
    [n][G][d] for n independent blocks at once (the same steps on each).

    Keys: one group per channel over the G tokens [P4 KIVI: keys per channel].
    Values: one group per (token, G_V consecutive channels) [P4 KIVI: values
    per token].
    Returns a dict of the section arrays (with the leading block axis, if any).
    """
    G, d, gv = spec.k_group, spec.head_dim, spec.v_group
    assert kblk.shape[-2:] == (G, d) and vblk.shape == kblk.shape
    lead = kblk.shape[:-2]
    if spec.rotate & ROT_KEYS:      # every token's key vector rotated first [P4w]
        kblk = rotate_f32(kblk)
    if spec.rotate & ROT_VALUES:
        vblk = rotate_f32(vblk)
    ks, kz, kcodes = quantize_groups(kblk, spec.k_bits, axis=-2)         # [d], [d], [G][d]
    vs, vz, vcodes = quantize_groups(vblk.reshape(lead + (G, d // gv, gv)), spec.v_bits, axis=-1)
    vcodes = vcodes.reshape(lead + (G, d))                                # [G][d]
    return {
        "k_codes": pack_lsb_first(kcodes, spec.k_bits),                   # [G][d*bK/32]
        "k_scale": ks, "k_zero": kz,                                      # [d]
        "v_codes": pack_lsb_first(value_code_stream(vcodes), spec.v_bits),
        "v_scale": np.ascontiguousarray(np.swapaxes(vs, -1, -2)),         # [d/G_V][G]
        "v_zero": np.ascontiguousarray(np.swapaxes(vz, -1, -2)),
    }


def block_to_bytes(sec) -> np.ndarray:
    """Record bytes of a block's sections ([record_bytes]), or of n blocks'
    ([n][record_bytes])."""
    lead = sec["k_scale"].shape[:-1]
    parts = [np.ascontiguousarray(sec[k]).view(np.uint8).reshape(lead + (-1,))
             for k in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")]
    return np.concatenate(parts, axis=-1)


# ---------------------------------------------------------------------------
# FP8 tier [P1' Minima-KV: recent pages in FP8]. Formula F8, per token row x
# (d values), every step an fp32 IEEE operation rounded to nearest even:
#   s = fp16(max|x| / 448);  s == 0 -> all codes 0;
#   else code_c = e4m3(clamp(fp32(x_c / s), -448, 448)), e4m3 rounding to
#   nearest with ties to the even code; x_hat_c = e4m3_value(code_c) * s.
# e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
# subnormal (m/8 * 2^-6); 0x7f / 0xff are NaN and never produced; 448 is the
# largest finite magnitude.
# ---------------------------------------------------------------------------
def e4m3_value(code) -> np.ndarray:
    """float64 value of e4m3 codes (uint8 array)."""
    c = np.asarray(code, np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(c & 0x80, -mag, mag)


_E4M3_POS = e4m3_value(np.arange(0x7f))   # codes 0x00 .. 0x7e, increasing


def e4m3_encode(y) -> np.ndarray:
    """Nearest e4m3 code (ties to the even code) of float values |y| <= 448."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 0, 0x7e)
    lo = np.clip(hi - 1, 0, 0x7e)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    mag = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    return (mag | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_fp8_rows(x: np.ndarray):
    """Formula F8 on every row of x (float32 [n][d]): (codes uint8 [n][d], s16 [n])."""
    x = np.asarray(x, F32)
    a = np.max(np.abs(x), axis=1)
    s16 = (a / F32(448.0)).astype(F32).astype(np.float16)
    s = s16.astype(F32)
    y = np.zeros_like(x)
    nz = s != 0
    y[nz] = np.clip(x[nz] / s[nz, None], F32(-448.0), F32(448.0))
    codes = e4m3_encode(y)
    codes[~nz] = 0
    return codes, s16


def fp8_record(kblk: np.ndarray, vblk: np.ndarray) -> np.ndarray:
    """FP8 record of one block, as bytes: K codes u8 [G][d] (token-major), K
    scales fp16 [G], V codes u8 [G][d], V scales fp16 [G]."""
    kc, ks = quantize_fp8_rows(kblk)
    vc, vs = quantize_fp8_rows(vblk)
    return np.concatenate([kc.ravel(), ks.view(np.uint8), vc.ravel(), vs.view(np.uint8)])


def fp8_record_bytes(spec: CacheSpec) -> int:
    return 2 * spec.k_group * spec.head_dim + 4 * spec.k_group


def dequantize_fp8_block(kblk: np.ndarray, vblk: np.ndarray):
    """fp64 [G][d] key and value reconstructions of one block through F8."""
    out = []
    for x in (kblk, vblk):
        c, s = quantize_fp8_rows(x)
        out.append(e4m3_value(c) * s.astype(np.float64)[:, None])
    return out[0], out[1]


def fp8_window(spec: CacheSpec, S: int):
    """Quantized blocks of a sequence of S tokens read through FP8: [f0, nblk)."""
    nblk = stream_split(spec, S)[1] // spec.k_group
    return nblk - min(nblk, spec.fp8_blocks), nblk


def dequantize_block(spec: CacheSpec, sec):
    """fp64 [G][d] key and value reconstructions of one block (or [n][G][d] of
    the n blocks of a batched quantize_block), in the rotated coordinates when
    the spec rotates (pair_cache_fp64 takes them back)."""
    G, d, gv = spec.k_group, spec.head_dim, spec.v_group
    kcodes = unpack_lsb_first(sec["k_codes"], spec.k_bits)               # [G][d]
    khat = dequantize(kcodes, sec["k_scale"][..., None, :], sec["k_zero"][..., None, :])
    vcodes = value_codes_from_stream(unpack_lsb_first(sec["v_codes"], spec.v_bits), G, d)  # [G][d]
    vs = np.repeat(np.swapaxes(sec["v_scale"], -1, -2), gv, axis=-1)      # [G][d]
    vz = np.repeat(np.swapaxes(sec["v_zero"], -1, -2), gv, axis=-1)
    vhat = dequantize(vcodes, vs, vz)
    return khat, vhat


# ---------------------------------------------------------------------------
# Residual window policy [P4 KIVI: recent tokens stay fp16; P4 innovation 4:
# the last R tokens stay in full precision and the switch is invisible to the
# attention kernel].  Reading: after a flush R <= r < R+G.
# ---------------------------------------------------------------------------
def quantized_prefix(S: int, R: int, G: int) -> int:
    """Q = number of leading tokens held quantized once the window is flushed."""
    return G * (max(S - R, 0) // G)


def stream_split(spec: CacheSpec, S: int):
    """Where the S tokens of one sequence live once the window is flushed
    [P2'; P3' sink; P4 KIVI window]: (s, Q, r) with tokens [0, s) in the sink,
    [P, P + Q) quantized and [P + Q, S) in the ring; s + Q + r = S."""
    P = spec.sink
    s = min(S, P)
    post = max(S - P, 0)
    Q = quantized_prefix(post, spec.residual, spec.k_group)
    return s, Q, post - Q


# ---------------------------------------------------------------------------
# Expected cache state after appending S_b tokens per sequence and flushing.
# ---------------------------------------------------------------------------
def expected_blocks(spec: CacheSpec, K: np.ndarray, V: np.ndarray, S_b: int):
    """Records of every quantized block of one (sequence, kv head).

    K, V: float32 [>=S_b][d] input values of that pair. Returns uint8
    [Q/G][record_bytes]; block j holds tokens P + jG .. P + jG + G - 1.
    """
    G, P, d = spec.k_group, spec.sink, spec.head_dim
    _, Q, _ = stream_split(spec, S_b)
    if Q == 0:
        return np.zeros((0, record_bytes(spec)), np.uint8)
    # every block at once: block j is row j of the [Q/G][G][d] views
    kb = np.asarray(K[P:P + Q], F32).reshape(Q // G, G, d)
    vb = np.asarray(V[P:P + Q], F32).reshape(Q // G, G, d)
    return block_to_bytes(quantize_block(spec, kb, vb))


def ring_slots(Q: int, S: int, capacity: int, sink: int = 0) -> np.ndarray:
    """Ring-buffer slots holding the residual tokens P+Q .. S-1 of a sequence
    with a sink of P tokens: token t lives at (t - P) mod C."""
    return np.arange(Q, max(S - sink, 0)) % capacity


# ---------------------------------------------------------------------------
# Attention in fp64 [P4 "Le problème": queries read back the stored keys and
# values of every earlier token].
# ---------------------------------------------------------------------------
def attention_fp64(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of queries q [n][d] over keys/values K, V [T][d], fp64."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = float(scale) * (q @ K.T)                      # [n][T]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def pair_cache_fp64(spec: CacheSpec, K: np.ndarray, V: np.ndarray, S_b: int):
    """The attention inputs of one (sequence, kv head), in token order: the exact
    sink tokens, the dequantized blocks (the W newest through F8; rotated
    sides taken back through R's inverse), then the exact residual tokens.
    Returns (Khat, Vhat) [S_b][d]."""
    G, P = spec.k_group, spec.sink
    assert not (spec.rotate and spec.fp8_blocks), "the FP8 tier stores unrotated rows"
    s, Q, _ = stream_split(spec, S_b)
    ks = [np.asarray(K[:s], np.float64)]
    vs = [np.asarray(V[:s], np.float64)]
    f0 = Q // G - min(Q // G, spec.fp8_blocks)   # blocks from here on are read through FP8
    if f0 > 0:   # blocks 0 .. f0-1 through their low-bit records, all at once
        d = spec.head_dim
        kb = np.asarray(K[P:P + f0 * G], F32).reshape(f0, G, d)
        vb = np.asarray(V[P:P + f0 * G], F32).reshape(f0, G, d)
        kh, vh = dequantize_block(spec, quantize_block(spec, kb, vb))
        if spec.rotate & ROT_KEYS:    # back through R's inverse [P4w]
            kh = unrotate_f64(kh)
        if spec.rotate & ROT_VALUES:
            vh = unrotate_f64(vh)
        ks.append(kh.reshape(f0 * G, d))
        vs.append(vh.reshape(f0 * G, d))
    for j in range(f0, Q // G):
        lo = P + j * G
        kh, vh = dequantize_fp8_block(K[lo:lo + G], V[lo:lo + G])
        ks.append(kh)
        vs.append(vh)
    ks.append(np.asarray(K[P + Q:S_b], np.float64))
    vs.append(np.asarray(V[P + Q:S_b], np.float64))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def decode_attention(spec: CacheSpec, q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     lengths, scale: float | None = None, pairs=None) -> np.ndarray:
    """Single-token decode attention over the quantized cache, fp64.

    q: [B][H_q][d]; K, V: [B][H_kv][>=max S][d] float32 input values;
    lengths: S_b per sequence. Query head h' reads kv head h'//n_g.
    `pairs` limits the work to a list of (b, h_kv); other outputs are NaN.
    Returns out [B][H_q][d] float64.
    """
    B, Hq, d = q.shape
    n_g = spec.n_g
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((B, Hq, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(spec.num_kv_heads)]
    for b, h in pairs:
        S_b = int(lengths[b])
        if S_b == 0:
            out[b, h * n_g:(h + 1) * n_g] = 0.0
            continue
        Kh, Vh = pair_cache_fp64(spec, K[b, h], V[b, h], S_b)
        out[b, h * n_g:(h + 1) * n_g] = attention_fp64(q[b, h * n_g:(h + 1) * n_g], Kh, Vh, scale)
    return out


def decode_attention_multi(spec: CacheSpec, q: np.ndarray, K: np.ndarray, V: np.ndarray, lengths, T: int,
                           scale: float | None = None, pairs=None) -> np.ndarray:
    """Attention of the T newest tokens of every sequence over the quantized
    cache, causal within the block [P3'' block-wise prefill; P4 block decoding],
    fp64.

    q: [B][H_q][T][d] (query t of sequence b is token S_b - T + t); K, V, lengths
    as in decode_attention. Query t sees the first S_b - T + t + 1 tokens of the
    cache state after all S_b tokens are in (sink, dequantized blocks, ring, in
    token order); a query with no token to see gets a zero output.
    Returns out [B][H_q][T][d] float64.
    """
    B, Hq, T_, d = q.shape
    assert T_ == T
    n_g = spec.n_g
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((B, Hq, T, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(spec.num_kv_heads)]
    for b, h in pairs:
        S_b = int(lengths[b])
        Kh, Vh = pair_cache_fp64(spec, K[b, h], V[b, h], S_b) if S_b > 0 else (None, None)
        for t in range(T):
            seen = S_b - T + t + 1
            for hq in range(h * n_g, (h + 1) * n_g):
                if seen <= 0:
                    out[b, hq, t] = 0.0
                else:
                    out[b, hq, t] = attention_fp64(q[b, hq, t][None], Kh[:seen], Vh[:seen], scale)[0]
    return out


def exact_attention(spec: CacheSpec, q, K, V, lengths, scale=None, pairs=None):
    """Attention on the unquantized inputs (for the fidelity report only)."""
    B, Hq, d = q.shape
    n_g = spec.n_g
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((B, Hq, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(spec.num_kv_heads)]
    for b, h in pairs:
        S_b = int(lengths[b])
        out[b, h * n_g:(h + 1) * n_g] = attention_fp64(
            q[b, h * n_g:(h + 1) * n_g], K[b, h, :S_b], V[b, h, :S_b], scale)
    return out


# ---------------------------------------------------------------------------
# KV-cache memory [P4 "Le problème"]: 2 * L * H * d * S * bytes per element.
# ---------------------------------------------------------------------------
def kv_cache_bytes(layers: int, heads: int, head_dim: int, tokens: int, bytes_per_elt: float) -> float:
    return 2 * layers * heads * head_dim * tokens * bytes_per_elt


def quantized_bytes_per_token(spec: CacheSpec) -> float:
    """Bytes one quantized token occupies per kv head (codes + scale/zero): the
    per-token cost that replaces 2 * d * bytes of the closed form above."""
    return record_bytes(spec) / spec.k_group
