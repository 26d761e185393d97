"""Pins of the FP8 part of the oracle (oracle/fp8.py): facts fixed by the
OCP E4M3 format, by an independent library (torch's float8_e4m3fn dtype and
its float32 conversion, torch's float64 scaled_dot_product_attention), by
closed forms and by invariants.  Each check takes the module as its argument
so that the mutation tests can hand it a copy with a planted mistake."""

import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ codec
def check_e4m3_decode_matches_torch(F):
    """Every one of the 256 codes decodes to torch's float8_e4m3fn value."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def check_e4m3_closed_forms(F):
    """Values fixed by the format: bias 7, 3 mantissa bits, subnormals in
    steps of 2^-9, largest finite 448, S.1111.111 NaN, no infinity."""
    d = lambda c: float(F.e4m3_decode(np.array([c], np.uint8))[0])
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x40) == 2.0 and d(0x3C) == 1.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x77) == 240.0 and d(0x78) == 256.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF)) and d(0x00) == 0.0
    vals = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0) and np.isfinite(vals).all()


def check_e4m3_encode_matches_torch(F):
    """Round-to-nearest-even to E4M3 equals torch's float32 -> float8_e4m3fn
    conversion on random magnitudes over the whole range (subnormals
    included), on every representable value and on every exact midpoint
    between neighbours (the ties)."""
    rng = _rng(101)
    x = (rng.choice([-1.0, 1.0], 20000) * 2.0 ** rng.uniform(-13, 8.8, 20000))
    x = x.astype(np.float32).astype(np.float64)
    vals = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, vals, -vals, mids, -mids, [0.0, -0.0, 448.0, -448.0]])
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)  # all exact in fp32
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode_rne(x32)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


# ------------------------------------------------------------ quantization
def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def check_quantize_blocks(F):
    """Block quantization: the largest magnitude of each block encodes to
    +-448 (code 0x7E / 0xFE), every value is reconstructed within half an
    E4M3 step (2^-4 relative above 2^-6 s, 2^-10 s below), blocks are 64
    tokens of one head, the last one partial, and an all-zero block gets
    scale 1 and zero codes."""
    rng = _rng(102)
    B, N, H, d = 2, 150, 3, 64
    # block t of head h carries magnitude 2^(t + h): the scale shows which
    # tokens and head each block covers
    mag = np.zeros((B, N, H, 1))
    for h in range(H):
        for t in range(N):
            mag[:, t, h] = 2.0 ** (t // 64 + h)
    x = _bf16(rng.standard_normal((B, N, H, d)) * mag)
    x[1, 64:128, 2] = 0.0
    codes, scales = F.quantize_blocks(x)
    assert codes.dtype == np.uint8 and scales.shape == (B, H, 3)
    for b in range(B):
        for h in range(H):
            for t in range(3):
                blk = x[b, 64 * t:64 * (t + 1), h]
                c = codes[b, 64 * t:64 * (t + 1), h]
                if b == 1 and h == 2 and t == 1:
                    assert scales[b, h, t] == 1.0 and not c.any()
                    continue
                amax = np.abs(blk).max()
                assert abs(scales[b, h, t] * 448.0 / amax - 1) < 1e-6
                assert 2.0 ** (t + h) / 2 < scales[b, h, t] * 448 < 2.0 ** (t + h) * 8
                at = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                assert c[at] in (0x7E, 0xFE)
    deq = F.dequantize(codes, scales)
    s_tok = np.repeat(scales, 64, axis=2)[:, :, :N].transpose(0, 2, 1)[..., None]
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s_tok) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)


def check_quantize_exact_roundtrip(F):
    """Values that are E4M3 values times a power of two whose block maximum
    is 448 times that power come back exactly, with that power as scale."""
    rng = _rng(103)
    codes = rng.integers(0, 0x7F, size=(1, 128, 2, 64)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[0, 0, :, 0] = 0x7E
    codes[0, 64, :, 0] = 0xFE
    codes[(codes & 0x7F) == 0x7F] = 0x00
    e = np.array([-3.0, 5.0])
    x = F.e4m3_decode(codes) * (2.0 ** e)[None, None, :, None]
    c2, s2 = F.quantize_blocks(x)
    assert np.array_equal(s2, np.broadcast_to((2.0 ** e)[None, :, None], s2.shape))
    assert np.array_equal(F.e4m3_decode(c2), F.e4m3_decode(codes))


# ------------------------------------------------------------ rotation
def check_hadamard_rotation(F):
    """H is the Sylvester-Hadamard matrix (H2 by hand, H H^T = d I), the
    rotation x D H / sqrt(d) preserves norms, is undone by y H / sqrt(d) D,
    applies the signs column-wise (a d = 4 case worked by hand) and leaves
    every score Q K^T unchanged."""
    assert np.array_equal(F.sylvester_hadamard(2), [[1, 1], [1, -1]])
    for d in (4, 64, 128):
        H = F.sylvester_hadamard(d)
        assert np.array_equal(H @ H.T, d * np.eye(d))
    # d = 4, signs (1, -1, 1, 1), x = (1, 2, 3, 4): x D = (1, -2, 3, 4);
    # times H4 = [[1,1,1,1],[1,-1,1,-1],[1,1,-1,-1],[1,-1,-1,1]] / 2:
    # (1-2+3+4, 1+2+3-4, 1-2-3-4, 1+2-3+4) / 2
    got = F.rotate(np.array([1.0, 2.0, 3.0, 4.0]), [1, -1, 1, 1])
    assert np.allclose(got, np.array([6.0, 2.0, -8.0, 4.0]) / 2, atol=1e-15)
    rng = _rng(104)
    s = rng.choice([-1.0, 1.0], 128)
    q = rng.standard_normal((37, 128))
    k = rng.standard_normal((29, 128))
    rq, rk = F.rotate(q, s), F.rotate(k, s)
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), atol=1e-12)
    assert np.allclose(rq @ rk.T, q @ k.T, atol=1e-11)
    back = (rq @ F.sylvester_hadamard(128) / np.sqrt(128)) * s
    assert np.allclose(back, q, atol=1e-12)
    assert not np.allclose(F.rotate(q, np.ones(128)), rq)


def check_rotation_spreads_an_outlier(F):
    """The point of the rotation: a row whose mass sits in one coordinate is
    spread evenly (|x D H| / sqrt(d) = |x_c| / sqrt(d) in every coordinate),
    so its block's scale stops being set by the outlier.  With the outlier
    80000 times the typical value, the other rows fall below E4M3's smallest
    normal (2^-6 of the scale) without the rotation and lose their relative
    precision; rotated, they stay normal."""
    rng = _rng(105)
    d = 64
    x = _bf16(rng.standard_normal((1, 64, 1, d)) * 0.0005)
    x[0, 5, 0, 17] = 40.0
    s = rng.choice([-1.0, 1.0], d)
    r = F.rotate(x, s)
    assert np.allclose(np.abs(F.rotate(np.eye(d)[17] * 40.0, s)), 40.0 / 8, atol=1e-12)
    e_plain = np.abs(F.dequantize(*F.quantize_blocks(x)) - x)
    e_rot = np.abs(F.dequantize(*F.quantize_blocks(x, s)) - r)
    rows = np.arange(64) != 5
    assert e_rot[0, rows].mean() < 0.5 * e_plain[0, rows].mean()


# ------------------------------------------------------------ attention
def _sdpa64(q, k, v, scale, causal):
    """torch float64 SDPA on one head: q [n, d], k, v [m, d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale)[0, 0].numpy()


def check_attn_fp8_is_attention_of_dequantized(F):
    """On codes with power-of-two block scales the quantized problem is
    attention of the decoded values times their block's scale: checked
    against torch's float64 SDPA head by head (GQA groups of 2), dense and
    causal, with blocks of different scales inside one sequence."""
    rng = _rng(106)
    B, N, hq, hkv, d = 1, 140, 4, 2, 64

    def codes(shape):
        c = rng.integers(0, 0x77, size=shape).astype(np.uint8)   # |x| <= 240
        return c | (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)

    q8, k8, v8 = codes((B, N, hq, d)), codes((B, N, hkv, d)), codes((B, N, hkv, d))
    sq = 2.0 ** rng.integers(-9, -5, size=(B, hq, 3)).astype(np.float32)
    sk = 2.0 ** rng.integers(-9, -5, size=(B, hkv, 3)).astype(np.float32)
    sv = 2.0 ** rng.integers(-6, -2, size=(B, hkv, 3)).astype(np.float32)
    scale = 1 / 8
    blk = np.arange(N) // 64
    for causal in (False, True):
        o, lse = F.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale, causal)
        for h in range(hq):
            g = h // 2
            qd = F.e4m3_decode(q8[0, :, h]) * sq[0, h, blk][:, None]
            kd = F.e4m3_decode(k8[0, :, g]) * sk[0, g, blk][:, None]
            vd = F.e4m3_decode(v8[0, :, g]) * sv[0, g, blk][:, None]
            assert np.allclose(o[0, :, h], _sdpa64(qd, kd, vd, scale, causal), atol=1e-12)


def check_p_rounding_model(F):
    """The error model of the 8-bit P V product: when every probability is a
    power of two (scores spaced by whole multiples of ln 2), rounding P to
    E4M3 changes nothing; with random scores its error stays within half an
    E4M3 step of every term, |dO| <= 2^-4 sum_j p_ij |V_j|."""
    rng = _rng(107)
    n, d = 24, 64
    # q = e_0 and key j = -i_j e_0 with i_j in 0..5 (exact E4M3 values); at
    # scale ln 2 the scores are -i_j ln 2, so P relative to the row maximum
    # is 2^-(i_j - min i) and P * 2^7 is a power of two from 2^2 to 2^7
    q8 = np.zeros((1, n, 1, d), np.uint8)
    q8[0, :, 0, 0] = 0x38
    k8 = np.zeros((1, n, 1, d), np.uint8)
    ints = rng.integers(0, 6, size=n).astype(np.float64)
    k8[0, :, 0, 0] = F.e4m3_encode_rne(-ints)
    assert np.array_equal(F.e4m3_decode(k8[0, :, 0, 0]), -ints)
    v8 = rng.integers(0, 0x70, size=(1, n, 1, d)).astype(np.uint8)
    one = np.ones((1, 1, 1), np.float32)
    o_exact, _ = F.attn_fwd_fp8(q8, k8, v8, one, one, one, math.log(2.0))
    o_round = F.attn_fwd_fp8_p_rounded(q8, k8, v8, one, one, one, math.log(2.0))
    assert np.allclose(o_round, o_exact, atol=1e-12)
    B, N, hq, hkv = 1, 96, 2, 1
    q8 = rng.integers(0, 0x70, size=(B, N, hq, d)).astype(np.uint8) | (
        rng.integers(0, 2, size=(B, N, hq, d)) << 7).astype(np.uint8)
    k8 = rng.integers(0, 0x70, size=(B, N, hkv, d)).astype(np.uint8) | (
        rng.integers(0, 2, size=(B, N, hkv, d)) << 7).astype(np.uint8)
    v8 = rng.integers(0, 0x70, size=(B, N, hkv, d)).astype(np.uint8)
    s = np.full((B, hq, 2), 2.0 ** -6, np.float32)
    sk = np.full((B, hkv, 2), 2.0 ** -6, np.float32)
    sv = np.array([[[2.0 ** -3, 3 * 2.0 ** -5]]], np.float32)
    o_exact, _ = F.attn_fwd_fp8(q8, k8, v8, s, sk, sv, 0.125, True)
    o_round = F.attn_fwd_fp8_p_rounded(q8, k8, v8, s, sk, sv, 0.125, True)
    vd = F.dequantize(v8, sv)
    qd, kd = F.dequantize(q8, s), F.dequantize(k8, sk)
    for h in range(hq):
        sc = 0.125 * qd[0, :, h] @ kd[0, :, 0].T
        sc = np.where(np.tril(np.ones((N, N), bool)), sc, -np.inf)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        bound = 2.0 ** -4 * (p @ np.abs(vd[0, :, 0])) + 1e-12
        err = np.abs(o_round[0, :, h] - o_exact[0, :, h])
        assert np.all(err <= bound)
        assert err.max() > 0


FP8_CHECKS = [check_e4m3_decode_matches_torch, check_e4m3_closed_forms,
              check_e4m3_encode_matches_torch, check_quantize_blocks,
              check_quantize_exact_roundtrip, check_hadamard_rotation,
              check_rotation_spreads_an_outlier, check_attn_fp8_is_attention_of_dequantized,
              check_p_rounding_model]
