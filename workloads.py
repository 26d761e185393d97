"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws and rounds data; it holds none of the attention
arithmetic, and neither the CPU oracle nor the HIP library depends on it.

Every tensor is drawn i.i.d. N(0, 1) in float32 with numpy's PCG64
(``numpy.random.default_rng(seed)``), in token-major layout with the head
dimension innermost, then (for bf16 workloads) rounded to bfloat16 by
round-to-nearest-even (fp16 workloads: to IEEE half, nearest even).  The
arrays returned are float32 holding exactly the 16-bit values, so the GPU (after an exact cast to bf16) and the oracle (after an
exact cast to fp64) see identical numbers.

Draw order per workload: sequence lengths (packed batches only), then Q, K, V,
then dO (workloads with a backward pass).  Decode workloads draw the cached
key count of each sequence first, then Q, K, V.
"""

import math

import numpy as np

# The five workloads of the hot path, named by what they are.
#   seed: the rng seed (one per workload; a second seed = seed + 100 is used
#         by tests that want fresh data).
WORKLOADS = {
    # single-head fp32, B=1 H=1 N=128 d=64, non-causal
    "single_head_f32": dict(B=1, Hq=1, Hkv=1, N=128, d=64, dtype="f32",
                            causal=False, window=0, seed=1),
    # multi-head bf16 d=64, B=4 H=16 N=2048, non-causal and causal
    "mha_d64": dict(B=4, Hq=16, Hkv=16, N=2048, d=64, dtype="bf16",
                    causal=False, window=0, seed=2),
    "mha_d64_causal": dict(B=4, Hq=16, Hkv=16, N=2048, d=64, dtype="bf16",
                           causal=True, window=0, seed=2),
    # Llama-style GQA causal prefill, B=1 Hq=32 Hkv=8 N=8192 d=128
    "gqa_causal_prefill": dict(B=1, Hq=32, Hkv=8, N=8192, d=128, dtype="bf16",
                               causal=True, window=0, seed=3),
    # packed batch of 16 sequences, lengths U{256..8192}, causal + window 4096
    "varlen_window": dict(nseq=16, Lmin=256, Lmax=8192, Hq=32, Hkv=8, d=128,
                          dtype="bf16", causal=True, window=4096, seed=4),
    # long causal forward + recomputation backward, B=2 H=16 N=16384 d=128
    "long_fwd_bwd": dict(B=2, Hq=16, Hkv=16, N=16384, d=128, dtype="bf16",
                         causal=True, window=0, seed=5, bwd=True),
    # the GQA prefill shape with a custom additive mask instead of the causal
    # one: one fp32 [N, N] bias shared by every head, N(0, 1) values with a
    # random 10 % of the entries -inf; forward and backward
    "gqa_bias": dict(B=1, Hq=32, Hkv=8, N=8192, d=128, dtype="bf16", causal=False,
                     window=0, seed=7, bwd=True, bias_shape=(1, 1, "Q", "K"),
                     bias_masked=0.1),
    # the GQA causal prefill with dropout p = 0.1 on the probabilities
    # (seeded Philox keep-mask); forward and backward
    "gqa_dropout": dict(B=1, Hq=32, Hkv=8, N=8192, d=128, dtype="bf16", causal=True,
                        window=0, seed=8, bwd=True, dropout_p=0.1, dropout_seed=2024),
}


# 8-bit workloads: E4M3 codes with one fp32 scale per 64 tokens of one head.
FP8_WORKLOADS = {
    # the GQA causal prefill shape with FP8 Q, K, V
    "gqa_causal_prefill_fp8": dict(B=1, Hq=32, Hkv=8, N=8192, d=128, causal=True, window=0,
                                   seed=9),
}


# Decode over a key/value cache (few new query rows per sequence, long cache).
#   kv_lengths: keys in use per sequence, drawn uniformly from [Lmin, Lmax]
#   Nk: cache capacity per sequence (rows past a sequence's length are unused)
DECODE_WORKLOADS = {
    # single-token decode, 16 sequences, GQA 32/8, d=128, 1024..8192 cached keys
    "decode_kv_cache": dict(B=16, Hq=32, Hkv=8, Nq=1, Nk=8192, d=128, Lmin=1024,
                            Lmax=8192, causal=True, window=0, seed=6),
}


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    Works on the bit patterns in place, 16M values at a time: adding 0x7FFF
    plus the lowest kept bit and clearing the low half rounds to nearest even;
    finite values cannot overflow 32 bits on the way, and NaNs are restored."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    u = out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s:s + step]
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        c += np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        c &= np.uint32(0xFFFF0000)
        c[nan] = np.uint32(0x7FC00000)
    return out


def _draw(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":  # IEEE half, nearest even (numpy's conversion)
        return x.astype(np.float16).astype(np.float32)
    return x


def make_inputs(spec, seed=None, with_grad=None):
    """Draw one workload's inputs.

    spec: a WORKLOADS name or a dict with the same keys.  Dense specs need
    B, Hq, Hkv, N (or Nq and Nk), d; packed specs need nseq, Lmin, Lmax (or
    an explicit ``lengths`` list), Hq, Hkv, d.

    Returns a dict with q, k, v (and do when the workload has a backward),
    cu_seqlens (int32, or None), the shape fields, the scale 1/sqrt(d), and
    the mask flags.
    """
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    spec = dict(spec)
    seed = spec.get("seed", 0) if seed is None else seed
    with_grad = spec.get("bwd", False) if with_grad is None else with_grad
    dtype = spec.get("dtype", "bf16")
    rng = np.random.default_rng(seed)
    hq, hkv, d = spec["Hq"], spec["Hkv"], spec["d"]
    out = dict(spec)
    if "nseq" in spec or "lengths" in spec:
        if "lengths" in spec:
            lengths = np.asarray(spec["lengths"], dtype=np.int64)
        else:
            lengths = rng.integers(spec["Lmin"], spec["Lmax"] + 1,
                                   size=spec["nseq"])
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
        qs, ks = (T, hq, d), (T, hkv, d)
        out.update(B=len(lengths), Nq=int(max(lengths.max(), 1)) if len(lengths) else 1,
                   Nk=int(max(lengths.max(), 1)) if len(lengths) else 1,
                   T=T, lengths=lengths, cu_seqlens=cu)
    else:
        B = spec["B"]
        nq = spec.get("Nq", spec.get("N"))
        nk = spec.get("Nk", spec.get("N"))
        qs, ks = (B, nq, hq, d), (B, nk, hkv, d)
        out.update(Nq=nq, Nk=nk, cu_seqlens=None)
    out["q"] = _draw(rng, qs, dtype)
    out["k"] = _draw(rng, ks, dtype)
    out["v"] = _draw(rng, ks, dtype)
    if with_grad:
        out["do"] = _draw(rng, qs, dtype)
    if "bias_shape" in spec:
        out["bias"] = draw_bias(rng, spec["bias_shape"], out, spec.get("bias_masked", 0.1))
    out["scale"] = spec.get("scale", 1.0 / math.sqrt(d))
    out.setdefault("causal", False)
    out.setdefault("window", 0)
    out["dtype"] = dtype
    return out


def draw_bias(rng, shape, geom, masked=0.1):
    """An fp32 additive bias.  shape: four entries, each 1 (broadcast) or one
    of "B", "H", "Q", "K" (the batch, query-head, query and key extents of
    geom).  Values N(0, 1); a fraction `masked` of the entries is -inf, except
    key 0 of every row, so that every row keeps a key.  Drawn in pieces of
    16M entries (values, then the mask of the same piece)."""
    ext = {"B": geom["B"], "H": geom["Hq"], "Q": geom["Nq"], "K": geom["Nk"]}
    dims = tuple(ext[x] if isinstance(x, str) else int(x) for x in shape)
    out = np.empty(dims, dtype=np.float32)
    flat = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        n = min(step, flat.size - s)
        flat[s:s + n] = rng.standard_normal(n, dtype=np.float32)
        flat[s:s + n][rng.random(n, dtype=np.float32) < masked] = -np.inf
    out[..., 0] = np.where(np.isinf(out[..., 0]), 0.0, out[..., 0])
    return out


def make_decode_inputs(spec, seed=None):
    """Draw a decode workload: seqlens_k (int32 [B], drawn first), then q
    [B, Nq, Hq, d], k and v [B, Nk, Hkv, d], all bf16-valued float32."""
    if isinstance(spec, str):
        spec = DECODE_WORKLOADS[spec]
    spec = dict(spec)
    seed = spec.get("seed", 0) if seed is None else seed
    rng = np.random.default_rng(seed)
    B, hq, hkv, nq, nk, d = (spec[x] for x in ("B", "Hq", "Hkv", "Nq", "Nk", "d"))
    if "lengths" in spec:
        lengths = np.asarray(spec["lengths"], dtype=np.int32)
    else:
        lengths = rng.integers(spec["Lmin"], spec["Lmax"] + 1, size=B).astype(np.int32)
    out = dict(spec)
    out["seqlens_k"] = lengths
    out["q"] = _draw(rng, (B, nq, hq, d), "bf16")
    out["k"] = _draw(rng, (B, nk, hkv, d), "bf16")
    out["v"] = _draw(rng, (B, nk, hkv, d), "bf16")
    if "bias_shape" in spec:
        out["bias"] = draw_bias(rng, spec["bias_shape"], out, spec.get("bias_masked", 0.1))
    out["scale"] = spec.get("scale", 1.0 / math.sqrt(d))
    out["dtype"] = "bf16"
    return out


def e4m3_codes(x):
    """float32 values -> OCP E4M3 codes (uint8), by torch's float8_e4m3fn
    cast (nearest even); values must lie within +-448."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_fp8_inputs(spec, seed=None):
    """Draw an 8-bit workload directly in its quantized form: codes of
    N(0, 1) * 112 (clipped to +-448) cast to E4M3 for Q, K and V (V in
    token-major layout), then one scale per block of 64 tokens of each head,
    2^u / 112 with u uniform in [-1/2, 1/2] (so the dequantized values are
    N(0, 1) up to a factor 2^(+-1/2) per block).  Draw order: Q, K, V codes,
    then the Q, K, V scales.  Dense only."""
    if isinstance(spec, str):
        spec = FP8_WORKLOADS[spec]
    spec = dict(spec)
    seed = spec.get("seed", 0) if seed is None else seed
    rng = np.random.default_rng(seed)
    B, hq, hkv, d = spec["B"], spec["Hq"], spec["Hkv"], spec["d"]
    nq = spec.get("Nq", spec.get("N"))
    nk = spec.get("Nk", spec.get("N"))
    out = dict(spec, Nq=nq, Nk=nk)

    def codes(shape):
        x = np.empty(shape, np.float32)
        flat = x.reshape(-1)
        step = 1 << 24
        for s in range(0, flat.size, step):
            n = min(step, flat.size - s)
            flat[s:s + n] = np.clip(rng.standard_normal(n, dtype=np.float32) * 112.0,
                                    -448.0, 448.0)
        return e4m3_codes(x)

    out["q8"] = codes((B, nq, hq, d))
    out["k8"] = codes((B, nk, hkv, d))
    out["v8"] = codes((B, nk, hkv, d))
    scl = lambda h, n: (2.0 ** rng.uniform(-0.5, 0.5, size=(B, h, -(-n // 64))) / 112.0
                        ).astype(np.float32)
    out["sq"], out["sk"], out["sv"] = scl(hq, nq), scl(hkv, nk), scl(hkv, nk)
    out["scale"] = spec.get("scale", 1.0 / math.sqrt(d))
    out.setdefault("causal", False)
    out.setdefault("window", 0)
    out["dtype"] = "fp8"
    return out


def transpose_v8(v8):
    """Token-major V codes [B, N, H, d] -> the V^T layout [B, H, d, ldn]
    (ldn = N rounded up to 64, zero padding) that the FP8 forward reads."""
    B, N, H, d = v8.shape
    ldn = -(-N // 64) * 64
    out = np.zeros((B, H, d, ldn), dtype=np.uint8)
    out[..., :N] = np.transpose(v8, (0, 2, 3, 1))
    return out
