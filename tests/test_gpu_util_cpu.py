"""CPU checks of the derived gradient floor the GPU tests use
(tests/gpu_util.d_rounding_floor): the first-order bound of the dQ/dK error
that forming D = rowsum(dO * O) from the rounded O (bf16, or fp16 for the
fp16 path) causes.

The backward is emulated in fp64 from its definition with exactly that one
change (D from round_bf16(O)); its difference from the exact gradients must
stay inside the floor everywhere, and the floor must not be loose by more
than a small factor (else it would hide real errors)."""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import d_rounding_floor


def _emulated_grads(inp, o_rounded):
    """dQ, dK of one dense batch with D_i = sum_c dO_ic O~_ic from the
    rounded O~ instead of the exact O (no bias, no dropout)."""
    q, k, v, do = (np.asarray(inp[n], np.float64) for n in ("q", "k", "v", "do"))
    scale, causal, window = inp["scale"], inp["causal"], inp["window"]
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    g = hq // hkv
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    ok = oracle.allowed_mask(nq, nk, causal, window)
    for b in range(B):
        for h in range(hq):
            kv = h // g
            s = np.where(ok, scale * q[b, :, h] @ k[b, :, kv].T, -np.inf)
            m = s.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(ok, np.exp(s - m), 0.0)
            l = e.sum(axis=1, keepdims=True)
            p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
            dp = do[b, :, h] @ v[b, :, kv].T
            dd = (do[b, :, h] * o_rounded[b, :, h]).sum(axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, :, h] = scale * ds @ k[b, :, kv]
            dk[b, :, kv] += scale * ds.T @ q[b, :, h]
    return dq, dk


ROUNDINGS = {  # dtype: (rounding of O to nearest, unit of d_rounding_floor)
    "bf16": (lambda x: workloads.round_bf16(x.astype(np.float32)), 2.0 ** -9),
    "f16": (lambda x: x.astype(np.float16), 2.0 ** -12),
}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("spec", [
    dict(B=1, Nq=70, Nk=70, Hq=2, Hkv=1, d=64, causal=True, window=0, seed=41),
    dict(B=2, Nq=33, Nk=90, Hq=4, Hkv=2, d=32, causal=True, window=20, seed=42),
    dict(B=1, Nq=50, Nk=50, Hq=2, Hkv=2, d=16, causal=False, window=0, seed=43),
])
def test_floor_bounds_the_rounded_o_effect(spec, dtype):
    round_o, unit = ROUNDINGS[dtype]
    inp = workloads.make_inputs(dict(spec, bwd=True, dtype=dtype))
    f = lambda n: inp[n].astype(np.float64)
    o, lse = oracle.attn_fwd(f("q"), f("k"), f("v"), inp["scale"], inp["causal"], inp["window"])
    o_r = round_o(o).astype(np.float64)
    dq, dk, _ = oracle.attn_bwd(f("q"), f("k"), f("v"), f("do"), inp["scale"], inp["causal"],
                                inp["window"])
    edq, edk = _emulated_grads(inp, o_r)
    fq, fk = d_rounding_floor(inp, o_r, lse, unit)
    for name, err, fl in (("dQ", np.abs(edq - dq), fq), ("dK", np.abs(edk - dk), fk)):
        # inside the bound (first order: allow 1 % for the second-order terms)
        assert np.all(err <= 1.01 * fl + 1e-12), (name, float((err - fl).max()))
        # and the bound is not vacuous: the largest effect is within 20x of it
        assert err.max() >= fl.max() / 20, (name, float(err.max()), float(fl.max()))


def test_floor_is_zero_without_error_source():
    """dO = 0 leaves D = 0 exactly: the floor is zero."""
    inp = workloads.make_inputs(dict(B=1, Nq=20, Nk=20, Hq=2, Hkv=1, d=16, causal=True,
                                     window=0, seed=44, bwd=True))
    inp["do"] = np.zeros_like(inp["do"])
    f = lambda n: inp[n].astype(np.float64)
    o, lse = oracle.attn_fwd(f("q"), f("k"), f("v"), inp["scale"], True, 0)
    fq, fk = d_rounding_floor(inp, o, lse)
    assert not fq.any() and not fk.any()
