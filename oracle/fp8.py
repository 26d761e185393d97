"""FP8 (OCP E4M3) block quantization, the randomized Hadamard rotation and
attention of the quantized problem, in plain NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that the FA3 variant computes in 8-bit floating point
"with block quantization and incoherent processing" (llms.blog
"FlashAttention: How IO-Aware Tiling and Online Softmax Solved Transformer
Memory Bottlenecks", section "FlashAttention-3: Asynchronous Execution on
Hopper Architectures", the low-precision FP8 bullet; klaylearn.com glossary
"flash-attention", "What changed from FlashAttention to FA2 and FA3?", lists
FP8 among FA3's features).  Readings taken here:

* Format: OCP 8-bit floating point E4M3 ("E4M3FN"): sign, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m * 2^-9; no infinities; S.1111.111 is NaN, so the largest finite value is
  1.75 * 2^8 = 448.
* Block quantization: every block of 64 consecutive tokens of one head (all
  d columns) of Q, K and V gets one fp32 scale.  With amax the block's largest
  |x|, the scale is s = fl32(amax / 448) and the codes are
  RNE_e4m3(clamp(fl32(x * fl32(448 / amax)), -448, 448)): the decisions are
  taken in fp32, as the GPU takes them.  A block whose amax is below 2^-119
  (so that 448 / amax would overflow fp32), or zero, gets s = 1 and zero
  codes.  A block is the unit of one score tile, so per-block scales cost the
  attention kernel one multiply per tile.
* Incoherent processing: before Q and K are quantized, each row (token,
  head) of d values is multiplied by a random +-1 diagonal D (signs drawn by
  the caller) and by the normalised Sylvester-Hadamard matrix H / sqrt(d):
  x -> x D H / sqrt(d).  That matrix is orthogonal and the same for Q and K,
  so (Q D H)(K D H)^T = Q K^T: the scores are unchanged in exact arithmetic,
  while a coordinate with an outlier is spread over all d coordinates before
  the block scale is taken.
* Attention of the quantized problem: S = scale * (sQ Q~)(sK K~)^T,
  P = softmax(S + mask), O = P (sV V~), LSE = ln sum exp S -- the plain
  definition (oracle/attention.py) on the dequantized values, in fp64.
* The GPU also rounds P to E4M3 before the P V product (that product runs on
  the 8-bit matrix cores too), relative to its running row maximum with 2^7
  of headroom.  attn_fwd_fp8_p_rounded applies that rounding relative to the
  exact row maximum: it is the error model the GPU's output is compared with
  statistically, not the definition.
"""

import numpy as np

from .attention import allowed_mask, attn_fwd, kv_head_of

E4M3_MAX = 448.0
BLOCK = 64            # tokens per quantization block
TINY_AMAX = 2.0 ** -119
P_HEADROOM_LOG2 = 7   # P is rounded as P * 2^7 (its largest value 2^7 <= 448)


# ------------------------------------------------------------ E4M3 codec
def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def _positive_table():
    """The 127 finite non-negative E4M3 values, ascending, with their codes
    (code order equals value order for non-negative codes)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3_decode(codes), codes


def e4m3_encode_rne(x):
    """Round values to the nearest E4M3 code, ties to the even code (even
    mantissa); the sign is kept (also for values that round to zero, and for
    -0.0); magnitudes above 448 saturate to 448 (the callers clamp first);
    NaN -> 0x7F.  Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    vals, codes = _positive_table()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = np.abs(a - vals[lo])
    d_hi = np.abs(vals[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    c = np.where(np.signbit(x), c | np.uint8(0x80), c)   # -0.0 keeps its sign
    return np.where(np.isnan(x), np.uint8(0x7F), c).astype(np.uint8)


# ------------------------------------------------------------ rotation
def sylvester_hadamard(d):
    """The d x d Sylvester-Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(d)[:, None] & np.arange(d)[None, :]
    pop = np.zeros_like(i)
    for b in range(int(d).bit_length()):
        pop += (i >> b) & 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotate(x, signs):
    """x D H / sqrt(d) along the last axis (fp64); signs: d values of +-1."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float64)
    return (x * s) @ sylvester_hadamard(d) / np.sqrt(d)


# ------------------------------------------------------------ quantization
def quantize_blocks(x, signs=None, block=BLOCK):
    """Block-quantize x [B, N, H, d] (dense, token-major) to E4M3.

    Returns (codes uint8 [B, N, H, d], scales float32 [B, H, ceil(N/block)]).
    With signs, x is rotated first (fp64) and the rotated values are taken
    in fp32 before quantizing.  Every decision is made on fp32 values with
    fp32 arithmetic: amax, the scale amax/448, the multiplier 448/amax, the
    product and its clamp, then round-to-nearest-even to E4M3."""
    x = np.asarray(x)
    if signs is not None:
        x = rotate(x, signs)
    x = x.astype(np.float32)
    B, N, H, d = x.shape
    nb = -(-N // block)
    codes = np.zeros((B, N, H, d), dtype=np.uint8)
    scales = np.ones((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for t in range(nb):
                blk = x[b, t * block:(t + 1) * block, h]  # [<=block, d] fp32
                amax = np.float32(np.abs(blk).max())
                if not amax >= np.float32(TINY_AMAX):
                    continue  # zero (or negligible) block: scale 1, codes 0
                scales[b, h, t] = np.float32(amax / np.float32(E4M3_MAX))
                inv = np.float32(np.float32(E4M3_MAX) / amax)
                y = np.clip((blk * inv).astype(np.float32), -E4M3_MAX, E4M3_MAX)
                codes[b, t * block:(t + 1) * block, h] = e4m3_encode_rne(y)
    return codes, scales


def dequantize(codes, scales, block=BLOCK):
    """codes [B, N, H, d] uint8, scales [B, H, nb] -> float64 values."""
    codes = np.asarray(codes)
    B, N, H, d = codes.shape
    s = np.asarray(scales, dtype=np.float64)
    per_token = np.repeat(s, block, axis=2)[:, :, :N]          # [B, H, N]
    return e4m3_decode(codes) * per_token.transpose(0, 2, 1)[..., None]


# ------------------------------------------------------------ attention
def attn_fwd_fp8(q8, k8, v8, sq, sk, sv, scale, causal=False, window=0):
    """O, LSE of the quantized problem: exact attention (fp64) of the
    dequantized Q, K, V (dense layouts as oracle.attn_fwd; V token-major)."""
    return attn_fwd(dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv), scale,
                    causal, window)


def attn_fwd_fp8_p_rounded(q8, k8, v8, sq, sk, sv, scale, causal=False, window=0):
    """The error model of the 8-bit P V product: as attn_fwd_fp8, but each
    probability is rounded to E4M3 before it multiplies V, taken relative to
    its row maximum with 2^7 headroom and with each key's V block scale folded
    in relative to the head's largest V scale (the normaliser l stays
    unrounded).  Returns O."""
    q = dequantize(q8, sq)
    k = dequantize(k8, sk)
    vt = e4m3_decode(v8)
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    sv = np.asarray(sv, dtype=np.float64)
    ok = allowed_mask(nq, nk, causal, window)
    o = np.zeros((B, nq, hq, d))
    for b in range(B):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            s = np.where(ok, scale * (q[b, :, h] @ k[b, :, g].T), -np.inf)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            p = np.exp(s - m)                                   # row max -> 1
            l = p.sum(axis=1, keepdims=True)
            sv_key = np.repeat(sv[b, g], BLOCK)[:nk]            # [nk]
            ref = sv[b, g].max()
            pq = e4m3_decode(e4m3_encode_rne(p * 2.0 ** P_HEADROOM_LOG2 * (sv_key / ref)))
            num = pq @ vt[b, :, g] * (ref * 2.0 ** -P_HEADROOM_LOG2)
            o[b, :, h] = np.where(l > 0, num / np.where(l > 0, l, 1.0), 0.0)
    return o
