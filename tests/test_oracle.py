"""CPU tests of the oracle against its pins (no GPU, no HIP library)."""

import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from tests import oracle_pins as pins
import workloads


@pytest.mark.parametrize("check", pins.ALL_FORWARD + pins.ALL_BACKWARD,
                         ids=lambda f: f.__name__)
def test_pin(check):
    check(A)


# ----------------------------------------------------------- mutation tests
# Plant a plausible mistake in a copy of the oracle and require that at least
# one pin catches it.  The copy is a fresh module object whose globals are a
# shallow copy of the oracle module's, so the real oracle is never touched.

def _mutant(**overrides):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in A.__dict__.items()
                       if not k.startswith("__")})
    # the copied functions look builtins up through their globals
    m.__dict__["__builtins__"] = A.__dict__["__builtins__"]
    # functions look up globals in their defining module: rebind them
    for name, obj in list(m.__dict__.items()):
        if isinstance(obj, types.FunctionType) and obj.__module__ == A.__name__:
            m.__dict__[name] = types.FunctionType(obj.__code__, m.__dict__, name,
                                                  obj.__defaults__, obj.__closure__)
    m.__dict__.update(overrides)
    return m


def _caught(mutant, checks):
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check(mutant)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return True
    return False


def _bad_window_mask(nq, nk, causal, window):
    i = np.arange(nq)[:, None] + (nk - nq)
    j = np.arange(nk)[None, :]
    ok = np.ones((nq, nk), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (i - j) <= window  # admits W + 1 keys
    return ok


def _top_left_causal(nq, nk, causal, window):
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    ok = np.ones((nq, nk), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def _no_max_softmax(s):
    e = np.exp(s)
    l = e.sum(axis=1)
    return e / l[:, None], np.log(l)


def _lse_without_max(s):
    p, lse = A._softmax_rows(s)
    m = s.max(axis=1)
    return p, lse - np.where(np.isfinite(m), m, 0.0)


def _head_fwd_no_scale(q, k, v, scale, ok, bias=None, keep=None, p_drop=0.0):
    s = q @ k.T + (0.0 if bias is None else bias)
    s = np.where(ok, s, -np.inf)
    p, lse = A._softmax_rows(s)
    return A._dropped(p, keep, p_drop) @ v, lse, p


def _head_bwd_missing_D(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    o, _, p = A._head_fwd(q, k, v, scale, ok, bias, keep, p_drop)
    ds = p * (do @ v.T)
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ do


def _head_bwd_unscaled_dk(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    dq, dk, dv = A._head_bwd(q, k, v, do, scale, ok, bias, keep, p_drop)
    return dq, dk / scale, dv


def _head_bwd_transposed_dv(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    dq, dk, _ = A._head_bwd(q, k, v, do, scale, ok, bias, keep, p_drop)
    _, _, p = A._head_fwd(q, k, v, scale, ok, bias, keep, p_drop)
    return dq, dk, p @ do  # P instead of P^T (the pins use square shapes)


def _head_fwd_bias_scaled(q, k, v, scale, ok, bias=None, keep=None, p_drop=0.0):
    s = scale * (q @ k.T + (0.0 if bias is None else bias))
    p, lse = A._softmax_rows(np.where(ok, s, -np.inf))
    return A._dropped(p, keep, p_drop) @ v, lse, p


def _head_fwd_bias_subtracted(q, k, v, scale, ok, bias=None, keep=None, p_drop=0.0):
    s = scale * (q @ k.T) - (0.0 if bias is None else bias)
    p, lse = A._softmax_rows(np.where(ok, s, -np.inf))
    return A._dropped(p, keep, p_drop) @ v, lse, p


def _head_fwd_bias_transposed(q, k, v, scale, ok, bias=None, keep=None, p_drop=0.0):
    b = 0.0 if bias is None else np.asarray(bias)
    if np.ndim(b) == 2 and b.shape[0] == b.shape[1]:
        b = b.T
    p, lse = A._softmax_rows(np.where(ok, scale * (q @ k.T) + b, -np.inf))
    return A._dropped(p, keep, p_drop) @ v, lse, p


def _head_bwd_bias_dropped(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    return A._head_bwd(q, k, v, do, scale, ok, None, keep, p_drop)


def _bias_of_head_swapped(bias, B, hq, nq, nk):
    if bias is None:
        return None
    return np.broadcast_to(bias, (B, hq, nq, nk))[:, ::-1]


def _dropped_unscaled(p, keep, p_drop):
    return p if keep is None else np.where(keep, p, 0.0)


def _keep_rows_keys_swapped(dropout_p, seed, b, h, rows, nk):
    if dropout_p == 0.0:
        return None
    from oracle import philox
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(nk)[None, :]
    c0 = 2 * (rows >> 4) + ((rows >> 2) & 1)
    slot = 4 * ((rows >> 3) & 1) + (rows & 3)
    w = philox.philox4x32_10(c0, j, h, b, seed & 0xFFFFFFFF, seed >> 32)
    word = slot >> 1
    u = np.select([word == 0, word == 1, word == 2, word == 3], w)
    u16 = (u >> (np.uint64(16) * (slot & 1).astype(np.uint64))) & np.uint64(0xFFFF)
    return u16 >= np.uint64(philox.drop_threshold(dropout_p))


def _keep_slots_from_low_bits(dropout_p, seed, b, h, rows, nk):
    """A plausible mapping mistake: eight consecutive keys share a call
    (counter word j >> 3) and take slot j & 7."""
    if dropout_p == 0.0:
        return None
    from oracle import philox
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(nk)[None, :]
    slot = j & 7
    w = philox.philox4x32_10(j >> 3, rows, h, b, seed & 0xFFFFFFFF, seed >> 32)
    word = slot >> 1
    u = np.select([word == 0, word == 1, word == 2, word == 3], w)
    u16 = (u >> (np.uint64(16) * (slot & 1).astype(np.uint64))) & np.uint64(0xFFFF)
    return u16 >= np.uint64(philox.drop_threshold(dropout_p))


def _keep_head_and_batch_swapped(dropout_p, seed, b, h, rows, nk):
    return A._keep(dropout_p, seed, h, b, rows, nk)


def _keep_halves_swapped(dropout_p, seed, b, h, rows, nk):
    """Slot s read from the other 16-bit half of its word."""
    if dropout_p == 0.0:
        return None
    from oracle import philox
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(nk)[None, :]
    c0 = 2 * (j >> 4) + ((j >> 2) & 1)
    slot = 4 * ((j >> 3) & 1) + (j & 3)
    w = philox.philox4x32_10(c0, rows, h, b, seed & 0xFFFFFFFF, seed >> 32)
    word = slot >> 1
    u = np.select([word == 0, word == 1, word == 2, word == 3], w)
    u16 = (u >> (np.uint64(16) * (1 - (slot & 1)).astype(np.uint64))) & np.uint64(0xFFFF)
    return u16 >= np.uint64(philox.drop_threshold(dropout_p))


def _probabilities_unscaled(q, k, scale, causal=False, window=0):
    return A.probabilities(q, k, 1.0, causal, window)


def _head_bwd_dropout_dp_unmasked(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    o, _, p = A._head_fwd(q, k, v, scale, ok, bias, keep, p_drop)
    dv = A._dropped(p, keep, p_drop).T @ do
    dp = do @ v.T
    ds = p * (dp - (do * o).sum(axis=1)[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


MUTATIONS = {
    "gqa_strided_groups": dict(kv_head_of=lambda h, hq, hkv: h % hkv),
    "window_off_by_one": dict(allowed_mask=_bad_window_mask),
    "causal_top_left": dict(allowed_mask=_top_left_causal),
    "softmax_without_max": dict(_softmax_rows=_no_max_softmax),
    "lse_missing_max": dict(_softmax_rows=_lse_without_max),
    "scale_dropped": dict(_head_fwd=_head_fwd_no_scale),
    "bwd_missing_D": dict(_head_bwd=_head_bwd_missing_D),
    "bwd_dk_unscaled": dict(_head_bwd=_head_bwd_unscaled_dk),
    "bwd_dv_transposed": dict(_head_bwd=_head_bwd_transposed_dv),
    "bias_scaled_with_scores": dict(_head_fwd=_head_fwd_bias_scaled),
    "bias_subtracted": dict(_head_fwd=_head_fwd_bias_subtracted),
    "bias_transposed": dict(_head_fwd=_head_fwd_bias_transposed),
    "bias_dropped_in_bwd": dict(_head_bwd=_head_bwd_bias_dropped),
    "bias_heads_reversed": dict(_bias_of=_bias_of_head_swapped),
    "dropout_unscaled": dict(_dropped=_dropped_unscaled),
    "dropout_rows_keys_swapped": dict(_keep=_keep_rows_keys_swapped),
    "dropout_dp_unmasked": dict(_head_bwd=_head_bwd_dropout_dp_unmasked),
    "dropout_slots_from_low_bits": dict(_keep=_keep_slots_from_low_bits),
    "dropout_head_batch_swapped": dict(_keep=_keep_head_and_batch_swapped),
    "dropout_slot_halves_swapped": dict(_keep=_keep_halves_swapped),
    "probabilities_unscaled": dict(probabilities=_probabilities_unscaled),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mutant = _mutant(**MUTATIONS[name])
    assert _caught(mutant, pins.ALL_FORWARD + pins.ALL_BACKWARD), name


def _slot_words_low_bits(j):
    j = np.asarray(j, dtype=np.int64)
    return j >> 3, (j & 7) >> 1, j & 1


def _slot_words_no_call_pairing(j):
    j = np.asarray(j, dtype=np.int64)
    return j >> 3, (j & 7) >> 1 & 3, (j & 7) & 1


@pytest.mark.parametrize("wrong", [_slot_words_low_bits, _slot_words_no_call_pairing])
def test_golden_slots_catch_a_mapping_mistake_in_the_generator_module(monkeypatch, wrong):
    """A key -> slot mistake inside oracle/philox.py reaches every user of the
    keep-mask at once, so pins that compare the oracle with itself cannot see
    it; the hand-worked golden table must."""
    from oracle import philox
    monkeypatch.setattr(philox, "slot_words", wrong)
    with pytest.raises(AssertionError):
        pins.check_dropout_slots_golden(A)
    # the self-consistency pin passes on the same mistake: it is not a pin
    # of the mapping
    pins.check_dropout_matches_masked_softmax(A)


def test_mutant_harness_is_faithful():
    """An unmutated copy passes every pin (so catches above are real)."""
    assert not _caught(_mutant(), pins.ALL_FORWARD + pins.ALL_BACKWARD)


# ------------------------------------------------------------------- P-7
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 11),
                                           (False, 6)])
def test_online_recurrence_matches_definition(causal, window):
    """The pages' running (m, l, O) recurrence gives the exact result."""
    rng = np.random.default_rng(30)
    nq, nk, d = 45, 77, 16
    q = rng.standard_normal((nq, d)) * 2
    k = rng.standard_normal((nk, d))
    v = rng.standard_normal((nk, d))
    o_ref, l_ref = A.attn_fwd(q[None, :, None], k[None, :, None],
                              v[None, :, None], 0.6, causal, window)
    for trial in range(5):
        sizes = []
        while sum(sizes) < nk:
            sizes.append(int(rng.integers(1, 20)))
        o, lse = oracle.online_attention(q, k, v, 0.6, sizes, causal, window)
        assert np.allclose(o, o_ref[0, :, 0], atol=1e-12, rtol=0)
        assert np.allclose(lse, l_ref[0, 0], atol=1e-12, rtol=0)


# ---------------------------------------------------- sampled oracle paths
def test_rows_path_matches_full():
    rng = np.random.default_rng(31)
    q, k, v = (rng.standard_normal((1, 70, 4, 8)) for _ in range(3))
    k, v = k[:, :, :2], v[:, :, :2]
    for causal, window in [(True, 0), (True, 9), (False, 0)]:
        o, lse = A.attn_fwd(q, k, v, 0.4, causal, window)
        rows = np.array([0, 3, 31, 69])
        for h in range(4):
            g = A.kv_head_of(h, 4, 2)
            orow, lrow = A.attn_fwd_rows(q[0, :, h], k[0, :, g], v[0, :, g], rows,
                                         0.4, causal, window)
            assert np.allclose(orow, o[0, rows, h], atol=1e-13)
            assert np.allclose(lrow, lse[0, h, rows], atol=1e-13)


def test_sampled_backward_matches_full():
    rng = np.random.default_rng(32)
    q = rng.standard_normal((2, 40, 4, 8))
    k = rng.standard_normal((2, 40, 2, 8))
    v = rng.standard_normal((2, 40, 2, 8))
    do = rng.standard_normal(q.shape)
    for causal, window in [(True, 0), (False, 0), (True, 7)]:
        dq, dk, dv = A.attn_bwd(q, k, v, do, 0.3, causal, window)
        qr, kr = np.array([0, 5, 39]), np.array([0, 17, 39])
        for b in range(2):
            for g in range(2):
                sq, sk, sv = A.attn_bwd_sampled(q, k, v, do, 0.3, causal, window,
                                                b, g, qr, kr, chunk=13)
                assert np.allclose(sq, dq[b][qr][:, 2 * g:2 * g + 2], atol=1e-12)
                assert np.allclose(sk, dk[b, kr, g], atol=1e-12)
                assert np.allclose(sv, dv[b, kr, g], atol=1e-12)


def test_nan_poisoning_pattern():
    """NaN in one query row poisons that row only; NaN in a key row poisons
    the rows that see it (non-causal: all; causal: rows at or after it)."""
    rng = np.random.default_rng(33)
    q, k, v = (rng.standard_normal((1, 12, 1, 4)) for _ in range(3))
    q2 = q.copy()
    q2[0, 5, 0, 0] = np.nan
    o, lse = A.attn_fwd(q2, k, v, 0.5)
    assert np.all(np.isnan(o[0, 5])) and np.isnan(lse[0, 0, 5])
    assert np.all(np.isfinite(np.delete(o[0], 5, axis=0)))
    k2 = k.copy()
    k2[0, 7, 0, 1] = np.nan
    o, _ = A.attn_fwd(q, k2, v, 0.5, causal=True)
    assert np.all(np.isfinite(o[0, :7])) and np.all(np.isnan(o[0, 7:]))


# ---------------------------------------------------------------- inputs
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(34)
    x = rng.standard_normal(100000, dtype=np.float32) * 10
    x[:4] = [np.inf, -np.inf, 0.0, -0.0]
    # exact ties (low half 0x8000) with an even and an odd kept bit, and the
    # largest finite float, which rounds up to infinity
    x[4:8] = np.array([0x3F808000, 0x3F818000, 0xBF818000, 0x7F7FFFFF],
                      dtype=np.uint32).view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(workloads.round_bf16(x), ref)
    assert workloads.round_bf16(np.array([np.nan], dtype=np.float32))[0] != 0
    assert np.isnan(workloads.round_bf16(np.array([np.nan, 1.0], dtype=np.float32))[0])


def test_workload_shapes_and_determinism():
    # the lengths are drawn first, so one narrow head gives the same packing
    # as the full packed workload without multi-GB tensors
    narrow = dict(workloads.WORKLOADS["varlen_window"], Hq=2, Hkv=1, d=8)
    a = workloads.make_inputs(narrow)
    b = workloads.make_inputs(narrow)
    assert np.array_equal(a["cu_seqlens"], b["cu_seqlens"])
    assert np.array_equal(a["q"], b["q"])
    assert a["q"].shape == (a["T"], 2, 8) and a["k"].shape == (a["T"], 1, 8)
    L = np.diff(a["cu_seqlens"])
    assert len(L) == 16 and L.min() >= 256 and L.max() <= 8192
    s = workloads.make_inputs({"B": 1, "Hq": 4, "Hkv": 2, "N": 64, "d": 64,
                               "seed": 7, "bwd": True})
    assert s["q"].shape == (1, 64, 4, 64) and s["do"].shape == (1, 64, 4, 64)
    assert np.array_equal(workloads.round_bf16(s["q"]), s["q"])


def test_f16_inputs_are_exact_halves():
    s = workloads.make_inputs({"B": 1, "Hq": 2, "Hkv": 1, "N": 100, "d": 64,
                               "seed": 8, "dtype": "f16"})
    for n in ("q", "k", "v"):
        x = s[n]
        assert x.dtype == np.float32
        assert np.array_equal(x.astype(np.float16).astype(np.float32), x)
        # not merely bf16 values: fp16 keeps bits that bf16 drops
        assert not np.array_equal(workloads.round_bf16(x), x)


def test_sampled_paths_with_bias_and_dropout():
    """The row-sampled forward and backward agree with the full ones when a
    bias and dropout are on."""
    rng = np.random.default_rng(35)
    q = rng.standard_normal((2, 40, 4, 8))
    k = rng.standard_normal((2, 40, 2, 8))
    v = rng.standard_normal((2, 40, 2, 8))
    do = rng.standard_normal(q.shape)
    bias = rng.standard_normal((2, 1, 40, 40))
    kw = dict(bias=bias, dropout_p=0.3, seed=77)
    o, lse = A.attn_fwd(q, k, v, 0.3, True, 0, **kw)
    rows = np.array([0, 9, 39])
    for b in range(2):
        for h in range(4):
            orow, lrow = A.attn_fwd_rows(q[b, :, h], k[b, :, h // 2], v[b, :, h // 2], rows, 0.3,
                                         True, 0, bias=bias[b, 0], dropout_p=0.3, seed=77,
                                         bh=(b, h))
            assert np.allclose(orow, o[b, rows, h], atol=1e-12)
            assert np.allclose(lrow, lse[b, h, rows], atol=1e-12)
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.3, True, 0, **kw)
    qr, kr = np.array([0, 5, 39]), np.array([0, 17, 39])
    for b in range(2):
        for g in range(2):
            sq, sk, sv = A.attn_bwd_sampled(q, k, v, do, 0.3, True, 0, b, g, qr, kr, chunk=13, **kw)
            assert np.allclose(sq, dq[b][qr][:, 2 * g:2 * g + 2], atol=1e-12)
            assert np.allclose(sk, dk[b, kr, g], atol=1e-12)
            assert np.allclose(sv, dv[b, kr, g], atol=1e-12)
