"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each check takes the oracle module (``oracle.attention``) as its argument so
that the mutation tests can hand it a copy with a planted mistake and show that
some check fails.  None of these checks retypes the oracle's formulas: they use
closed forms, invariants, hand-worked values, finite differences, and
independent library routines (torch's scaled_dot_product_attention, logsumexp
and autograd in float64 on the CPU).
"""

import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _dense(rng, B, nq, nk, hq, hkv, d):
    q = rng.standard_normal((B, nq, hq, d))
    k = rng.standard_normal((B, nk, hkv, d))
    v = rng.standard_normal((B, nk, hkv, d))
    return q, k, v


# ---------------------------------------------------------------- P-1
def check_rows_sum_to_one(A):
    """Every row of P with a visible key sums to 1 (softmax definition), and
    P equals torch's float64 softmax of the scaled scores with the causal
    (bottom-right) and window entries filled with -inf."""
    rng = _rng(11)
    q = rng.standard_normal((37, 16))
    k = rng.standard_normal((53, 16))
    for causal, window in [(False, 0), (True, 0), (True, 7), (False, 9)]:
        p = A.probabilities(q, k, 0.7, causal, window)
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
        s = 0.7 * torch.from_numpy(q) @ torch.from_numpy(k).T
        i = torch.arange(37)[:, None] + (53 - 37)
        j = torch.arange(53)[None, :]
        hide = torch.zeros(37, 53, dtype=torch.bool)
        if causal:
            hide |= j > i
        if window > 0:
            hide |= (i - j) >= window
        ref = torch.softmax(s.masked_fill(hide, float("-inf")), dim=1).numpy()
        assert np.allclose(p, ref, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- P-2
def check_identical_keys(A):
    """All keys equal -> O_i is the mean of V over the keys i may see."""
    rng = _rng(12)
    B, n, d = 1, 24, 8
    q = rng.standard_normal((B, n, 2, d))
    k = np.broadcast_to(rng.standard_normal(d), (B, n, 1, d)).copy()
    v = rng.standard_normal((B, n, 1, d))
    o, _ = A.attn_fwd(q, k, v, 0.3, causal=False)
    assert np.allclose(o[0, :, 0], v[0, :, 0].mean(axis=0), atol=1e-12)
    o, _ = A.attn_fwd(q, k, v, 0.3, causal=True)
    prefix = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(o[0, :, 1], prefix, atol=1e-12)


# ---------------------------------------------------------------- P-3
def check_dominant_score(A):
    """k_j* = alpha * q_i with alpha large -> O_i ~= V_j* within the bound."""
    rng = _rng(13)
    n, d = 40, 16
    q, k, v = _dense(rng, 1, n, n, 1, 1, d)
    i, js = 17, 5
    k[0, js, 0] = 60.0 * q[0, i, 0]
    o, _ = A.attn_fwd(q, k, v, 1.0, causal=False)
    s = k[0, :, 0] @ q[0, i, 0]
    gap = s[js] - np.max(np.delete(s, js))
    bound = (n - 1) * math.exp(-gap) * 2 * np.abs(v).max()
    assert gap > 30
    assert np.max(np.abs(o[0, i, 0] - v[0, js, 0])) <= bound + 1e-12


# ---------------------------------------------------------------- P-4
def check_permutation_invariance(A):
    """Permuting K and V rows together leaves non-causal O and LSE unchanged."""
    rng = _rng(14)
    q, k, v = _dense(rng, 2, 19, 31, 4, 2, 8)
    perm = rng.permutation(31)
    o1, l1 = A.attn_fwd(q, k, v, 0.4)
    o2, l2 = A.attn_fwd(q, k[:, perm], v[:, perm], 0.4)
    assert np.allclose(o1, o2, atol=1e-12)
    assert np.allclose(l1, l2, atol=1e-12)


# ---------------------------------------------------------------- P-5
def check_lse_is_logsumexp(A):
    """LSE = ln sum_j exp(S_ij): against long double and torch.logsumexp."""
    rng = _rng(15)
    q, k, v = _dense(rng, 1, 21, 29, 1, 1, 8)
    q *= 3.0  # large scores exercise the max subtraction
    scale = 1.3
    _, lse = A.attn_fwd(q, k, v, scale)
    s = scale * (q[0, :, 0] @ k[0, :, 0].T)
    ld = np.log(np.exp(s.astype(np.longdouble)).sum(axis=1))
    assert np.allclose(lse[0, 0], ld.astype(np.float64), atol=1e-12)
    tl = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(lse[0, 0], tl, atol=1e-12)


# ---------------------------------------------------------------- P-6
def _visible_count(i, nq, nk, causal, window):
    """Number of keys query i sees, by counting (closed form per case)."""
    top = i + (nk - nq)  # last position query i may see when causal
    hi = min(nk - 1, top) if causal else nk - 1
    lo = max(0, top - window + 1) if window > 0 else 0
    return max(0, hi - lo + 1)


def check_scale_zero(A):
    """scale = 0 -> O_i = mean of visible V, LSE_i = ln(#visible keys)."""
    rng = _rng(16)
    for nq, nk, causal, window in [(30, 30, True, 0), (30, 30, True, 7),
                                   (30, 30, False, 7), (12, 30, True, 0),
                                   (12, 30, True, 5), (30, 30, False, 0)]:
        q, k, v = _dense(rng, 1, nq, nk, 1, 1, 4)
        o, lse = A.attn_fwd(q, k, v, 0.0, causal=causal, window=window)
        for i in range(nq):
            cnt = _visible_count(i, nq, nk, causal, window)
            top = i + nk - nq
            hi = min(nk - 1, top) if causal else nk - 1
            lo = max(0, top - window + 1) if window > 0 else 0
            assert cnt == hi - lo + 1
            assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-12
            assert np.allclose(o[0, i, 0], v[0, lo:hi + 1, 0].mean(axis=0),
                               atol=1e-12)
    # window closed form at the diagonal: LSE_i = ln min(i + 1, W)
    q, k, v = _dense(rng, 1, 40, 40, 1, 1, 4)
    _, lse = A.attn_fwd(q, k, v, 0.0, causal=True, window=9)
    assert np.allclose(lse[0, 0], np.log(np.minimum(np.arange(40) + 1, 9)),
                       atol=1e-12)
    # packed batch, non-causal: LSE = ln(sequence length)
    lengths = [5, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, 2, 4))
    k = rng.standard_normal((T, 1, 4))
    v = rng.standard_normal((T, 1, 4))
    o, lse = A.attn_fwd(q, k, v, 0.0, cu_seqlens=cu)
    for s, L in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        assert np.allclose(lse[:, a:b], math.log(L), atol=1e-12)
        assert np.allclose(o[a:b, 0], v[a:b, 0].mean(axis=0), atol=1e-12)


# ---------------------------------------------------------------- P-8
def _torch_sdpa(q, k, v, scale, causal):
    """torch float64 CPU SDPA on the dense layout, GQA by repeating KV heads."""
    G = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def check_against_torch_sdpa(A):
    """Small shapes against torch SDPA (float64, CPU), MHA and GQA."""
    rng = _rng(18)
    for B, n, hq, hkv, d, causal in [(2, 33, 4, 4, 16, False),
                                     (2, 33, 4, 4, 16, True),
                                     (1, 50, 8, 2, 32, True),
                                     (1, 50, 6, 1, 8, False)]:
        q, k, v = _dense(rng, B, n, n, hq, hkv, d)
        scale = 1.0 / math.sqrt(d)
        o, _ = A.attn_fwd(q, k, v, scale, causal=causal)
        assert np.allclose(o, _torch_sdpa(q, k, v, scale, causal), atol=1e-12)


def check_brute_force_tiny(A):
    """N=2, d=1 by hand: O_0 is the sigmoid-weighted mean of v0 and v1."""
    q = np.array([[[[0.7]], [[-1.1]]]])          # [1, 2, 1, 1]
    k = np.array([[[[1.5]], [[-0.4]]]])
    v = np.array([[[[2.0]], [[-3.0]]]])
    o, lse = A.attn_fwd(q, k, v, 1.0)
    for i in range(2):
        s0, s1 = q[0, i, 0, 0] * k[0, 0, 0, 0], q[0, i, 0, 0] * k[0, 1, 0, 0]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(o[0, i, 0, 0] - (w0 * 2.0 + (1 - w0) * -3.0)) < 1e-14
        assert abs(lse[0, 0, i] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-14


def check_hand_worked_golden(A):
    """The hand-worked example in tests/golden/hand_worked_softmax.txt."""
    q = np.array([[1, 0], [0, 1]], float).reshape(1, 2, 1, 2)
    k = np.array([[0, 0], [1, 0], [2, 1]], float).reshape(1, 3, 1, 2)
    v = np.array([[7, 0], [0, 7], [1, 1]], float).reshape(1, 3, 1, 2)
    cases = {"none": (False, 0), "causal": (True, 0), "causal_window2": (True, 2)}
    n = 0
    with open(os.path.join(GOLDEN, "hand_worked_softmax.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            case, row, o0, o1, lse = line.split()
            causal, window = cases[case]
            o, l = A.attn_fwd(q, k, v, math.log(2.0), causal, window)
            r = int(row)
            assert abs(o[0, r, 0, 0] - float(Fraction(o0))) < 1e-12
            assert abs(o[0, r, 0, 1] - float(Fraction(o1))) < 1e-12
            assert abs(l[0, 0, r] - math.log(int(lse[3:-1]))) < 1e-12
            n += 1
    assert n == 6


# ---------------------------------------------------------------- P-9
def check_gqa_is_repeated_mha(A):
    """GQA equals MHA with each KV head repeated over its contiguous group."""
    rng = _rng(19)
    q, k, v = _dense(rng, 2, 17, 17, 8, 2, 8)
    o1, l1 = A.attn_fwd(q, k, v, 0.5, causal=True)
    kr, vr = np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2)
    o2, l2 = A.attn_fwd(q, kr, vr, 0.5, causal=True)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    # query head 1 belongs to KV head 0: changing KV head 1 must not move it
    k2 = k.copy()
    k2[:, :, 1] += 5.0
    o3, _ = A.attn_fwd(q, k2, v, 0.5, causal=True)
    assert np.allclose(o3[:, :, :4], o1[:, :, :4], atol=1e-12)
    # torch check of the grouping (repeat_interleave = contiguous groups)
    assert np.allclose(o1, _torch_sdpa(q, k, v, 0.5, True), atol=1e-12)


# ---------------------------------------------------------------- P-10
def check_varlen_is_concatenation(A):
    """A packed batch equals each sequence run densely, concatenated."""
    rng = _rng(20)
    lengths = [7, 1, 0, 13, 4]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, 4, 8))
    k = rng.standard_normal((T, 2, 8))
    v = rng.standard_normal((T, 2, 8))
    for causal, window in [(False, 0), (True, 0), (True, 3)]:
        o, lse = A.attn_fwd(q, k, v, 0.6, causal, window, cu_seqlens=cu)
        for s, L in enumerate(lengths):
            a, b = cu[s], cu[s + 1]
            if L == 0:
                continue
            od, ld = A.attn_fwd(q[None, a:b], k[None, a:b], v[None, a:b],
                                0.6, causal, window)
            assert np.allclose(o[a:b], od[0], atol=1e-12)
            assert np.allclose(lse[:, a:b], ld[0], atol=1e-12)


# ---------------------------------------------------------------- P-11
def check_key_translation(A):
    """K += 1 c^T leaves O unchanged and shifts LSE_i by scale * q_i . c."""
    rng = _rng(21)
    q, k, v = _dense(rng, 1, 23, 23, 2, 1, 8)
    c = rng.standard_normal(8)
    for causal in (False, True):
        o1, l1 = A.attn_fwd(q, k, v, 0.45, causal)
        o2, l2 = A.attn_fwd(q, k + c, v, 0.45, causal)
        assert np.allclose(o1, o2, atol=1e-11)
        shift = 0.45 * np.einsum("bnhd,d->bhn", q, c)
        assert np.allclose(l2, l1 + shift, atol=1e-11)


# ---------------------------------------------------------------- P-12
def _loss(A, q, k, v, do, scale, causal, window):
    o, _ = A.attn_fwd(q, k, v, scale, causal, window)
    return float((o * do).sum())


def check_backward_finite_differences(A):
    """Central finite differences of sum(O * dO), fp64, tiny shapes."""
    rng = _rng(22)
    for causal, window in [(False, 0), (True, 0), (True, 3)]:
        q, k, v = _dense(rng, 1, 6, 6, 2, 1, 3)
        do = rng.standard_normal(q.shape)
        dq, dk, dv = A.attn_bwd(q, k, v, do, 0.8, causal, window)
        h = 1e-6
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                x[idx] += h
                fp = _loss(A, q, k, v, do, 0.8, causal, window)
                x[idx] -= 2 * h
                fm = _loss(A, q, k, v, do, 0.8, causal, window)
                x[idx] += h
                num[idx] = (fp - fm) / (2 * h)
            err = np.abs(num - g).max() / max(np.abs(num).max(), 1e-30)
            assert err < 1e-6, err


def check_backward_autograd(A):
    """Against torch autograd through float64 SDPA (GQA by repeat)."""
    rng = _rng(23)
    for causal in (False, True):
        q, k, v = _dense(rng, 2, 20, 20, 4, 2, 8)
        do = rng.standard_normal(q.shape)
        dq, dk, dv = A.attn_bwd(q, k, v, do, 0.35, causal)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True)
                      for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq.permute(0, 2, 1, 3),
            tk.permute(0, 2, 1, 3).repeat_interleave(2, dim=1),
            tv.permute(0, 2, 1, 3).repeat_interleave(2, dim=1),
            is_causal=causal, scale=0.35).permute(0, 2, 1, 3)
        (o * torch.from_numpy(do)).sum().backward()
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)


def check_backward_invariants(A):
    """sum_j dK_j = 0 and sum_j dV_j = sum of dO over the group's queries."""
    rng = _rng(24)
    q, k, v = _dense(rng, 1, 15, 15, 4, 2, 8)
    do = rng.standard_normal(q.shape)
    for causal, window in [(False, 0), (True, 0), (True, 4)]:
        _, dk, dv = A.attn_bwd(q, k, v, do, 0.5, causal, window)
        assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-11)
        dsum = do.reshape(1, 15, 2, 2, 8).sum(axis=(1, 3))
        assert np.allclose(dv.sum(axis=1), dsum, atol=1e-11)


# ---------------------------------------------------------------- P-13
def check_causal_row_zero(A):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q0.k0, dQ_0 = 0."""
    rng = _rng(25)
    q, k, v = _dense(rng, 1, 9, 9, 2, 1, 8)
    do = rng.standard_normal(q.shape)
    o, lse = A.attn_fwd(q, k, v, 0.3, causal=True)
    dq, _, _ = A.attn_bwd(q, k, v, do, 0.3, causal=True)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], v[0, 0, 0])
        assert abs(lse[0, h, 0] - 0.3 * q[0, 0, h] @ k[0, 0, 0]) < 1e-14
        assert np.all(dq[0, 0, h] == 0.0)


# ------------------------------------------------- causal alignment (C-6)
def check_chunked_prefill_alignment(A):
    """Nq < Nk causal = the last Nq rows of the full causal problem."""
    rng = _rng(26)
    q, k, v = _dense(rng, 1, 24, 24, 2, 2, 8)
    for window in (0, 5):
        of, lf = A.attn_fwd(q, k, v, 0.5, True, window)
        oc, lc = A.attn_fwd(q[:, 16:], k, v, 0.5, True, window)
        assert np.allclose(oc, of[:, 16:], atol=1e-12)
        assert np.allclose(lc, lf[:, :, 16:], atol=1e-12)


def check_empty_rows(A):
    """A query with no visible key gives O = 0 and LSE = -inf (no NaN)."""
    rng = _rng(27)
    q, k, v = _dense(rng, 1, 4, 2, 1, 1, 4)  # Nq > Nk: rows 0,1 see nothing
    o, lse = A.attn_fwd(q, k, v, 0.5, causal=True)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(o[0, 2:])) and np.all(np.isfinite(lse[0, 0, 2:]))


# ------------------------------------------------ additive mask / bias
def _torch_sdpa_bias(q, k, v, scale, mask):
    """torch float64 SDPA with a float attn_mask added to the scaled scores."""
    G = q.shape[2] // k.shape[2]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(np.array(mask)), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _random_bias(rng, shape, frac_masked=0.2):
    b = rng.standard_normal(shape) * 2.0
    b[rng.random(shape) < frac_masked] = -np.inf
    b[..., 0] = np.where(np.isinf(b[..., 0]), 0.5, b[..., 0])  # every row keeps a key
    return b


def check_bias_against_torch_sdpa(A):
    """Bias of several broadcast shapes, with -inf entries, against torch SDPA
    with the same float attn_mask (plus the causal mask written out)."""
    rng = _rng(40)
    for B, nq, nk, hq, hkv, d in [(2, 19, 27, 4, 2, 8), (1, 15, 15, 2, 1, 8)]:
        _bias_vs_torch(A, rng, B, nq, nk, hq, hkv, d)


def _bias_vs_torch(A, rng, B, nq, nk, hq, hkv, d):
    q, k, v = _dense(rng, B, nq, nk, hq, hkv, d)
    for shape in [(B, hq, nq, nk), (B, 1, nq, nk), (1, hq, 1, nk), (nq, nk)]:
        bias = _random_bias(rng, shape)
        o, _ = A.attn_fwd(q, k, v, 0.4, bias=bias)
        full = np.broadcast_to(bias, (B, hq, nq, nk))
        assert np.allclose(o, _torch_sdpa_bias(q, k, v, 0.4, full), atol=1e-12)
        # causal on top: torch gets the lower-right triangle as -inf entries
        o, _ = A.attn_fwd(q, k, v, 0.4, causal=True, bias=bias)
        j = np.arange(nk)[None, :]
        i = np.arange(nq)[:, None] + (nk - nq)
        both = np.where(j <= i, full, -np.inf)
        assert np.allclose(o, _torch_sdpa_bias(q, k, v, 0.4, both), atol=1e-12)


def check_bias_row_constant(A):
    """A bias constant along each row leaves O alone and adds it to LSE
    (softmax is invariant to a per-row shift)."""
    rng = _rng(41)
    q, k, v = _dense(rng, 1, 13, 21, 2, 1, 8)
    c = rng.standard_normal((1, 2, 13, 1)) * 3.0
    for causal, window in [(False, 0), (True, 5)]:
        o1, l1 = A.attn_fwd(q, k, v, 0.6, causal, window)
        o2, l2 = A.attn_fwd(q, k, v, 0.6, causal, window, bias=c)
        assert np.allclose(o1, o2, atol=1e-12)
        assert np.allclose(l2, l1 + c[..., 0], atol=1e-12)


def check_bias_is_key_shift(A):
    """bias = scale Q W^T gives exactly attention with keys K + W (the bias is
    added to the scaled score of query i and key j); dK and dV agree too."""
    rng = _rng(42)
    B, nq, nk, hq, d = 1, 11, 17, 2, 6
    q, k, v = _dense(rng, B, nq, nk, hq, hq, d)
    w = rng.standard_normal(k.shape)
    do = rng.standard_normal(q.shape)
    bias = 0.7 * np.einsum("bihd,bjhd->bhij", q, w)
    for causal in (False, True):
        o1, l1 = A.attn_fwd(q, k + w, v, 0.7, causal)
        o2, l2 = A.attn_fwd(q, k, v, 0.7, causal, bias=bias)
        assert np.allclose(o1, o2, atol=1e-11) and np.allclose(l1, l2, atol=1e-11)
        _, dk1, dv1 = A.attn_bwd(q, k + w, v, do, 0.7, causal)
        _, dk2, dv2 = A.attn_bwd(q, k, v, do, 0.7, causal, bias=bias)
        assert np.allclose(dk1, dk2, atol=1e-11) and np.allclose(dv1, dv2, atol=1e-11)


def check_bias_mask_equals_causal(A):
    """A {0, -inf} bias shaped like the causal mask equals causal=True, and a
    row that the bias hides completely gives O = 0 and LSE = -inf."""
    rng = _rng(43)
    q, k, v = _dense(rng, 1, 9, 14, 2, 2, 8)
    j = np.arange(14)[None, :]
    i = np.arange(9)[:, None] + 5
    m = np.where(j <= i, 0.0, -np.inf)
    o1, l1 = A.attn_fwd(q, k, v, 0.5, causal=True)
    o2, l2 = A.attn_fwd(q, k, v, 0.5, bias=m)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    m2 = np.zeros((9, 14))
    m2[3] = -np.inf
    o3, l3 = A.attn_fwd(q, k, v, 0.5, bias=m2)
    assert np.all(o3[0, 3] == 0) and np.all(np.isneginf(l3[0, :, 3]))
    assert np.all(np.isfinite(np.delete(o3[0], 3, axis=0)))


def check_bias_backward_autograd(A):
    """Gradients with a constant float mask against torch autograd through
    float64 SDPA, and central finite differences on a tiny case."""
    rng = _rng(44)
    q, k, v = _dense(rng, 2, 12, 16, 4, 2, 8)
    do = rng.standard_normal(q.shape)
    bias = _random_bias(rng, (2, 1, 12, 16))
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.45, bias=bias)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3).repeat_interleave(2, dim=1),
        tv.permute(0, 2, 1, 3).repeat_interleave(2, dim=1),
        attn_mask=torch.from_numpy(np.array(np.broadcast_to(bias, (2, 4, 12, 16)))),
        scale=0.45).permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)
    # finite differences, bias with a window on top
    q, k, v = _dense(rng, 1, 5, 7, 1, 1, 3)
    do = rng.standard_normal(q.shape)
    bias = _random_bias(rng, (5, 7))
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.8, True, 4, bias=bias)
    loss = lambda: float((A.attn_fwd(q, k, v, 0.8, True, 4, bias=bias)[0] * do).sum())
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x[idx] += h
            fp = loss()
            x[idx] -= 2 * h
            fm = loss()
            x[idx] += h
            num[idx] = (fp - fm) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(np.abs(num).max(), 1e-30)


# ------------------------------------------------------------ dropout
def check_philox_known_answers(A):
    """The generator against its published known-answer vectors."""
    from oracle import philox
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            got = [int(x) for x in philox.philox4x32_10(*w[:6])]
            assert got == w[6:], (line, [hex(x) for x in got])
            n += 1
    assert n == 3


def check_dropout_mask_statistics(A):
    """The keep fraction is 1 - p within binomial error, masks of different
    heads, sequences and seeds differ, and every output word is used."""
    from oracle import philox
    for p in (0.1, 0.5, 0.9):
        m = philox.keep_mask(123, 1, 2, np.arange(256), 256, p)
        n = m.size
        assert abs(m.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / n)
    a = philox.keep_mask(7, 0, 0, np.arange(64), 64, 0.5)
    for other in (philox.keep_mask(7, 0, 1, np.arange(64), 64, 0.5),
                  philox.keep_mask(7, 1, 0, np.arange(64), 64, 0.5),
                  philox.keep_mask(8, 0, 0, np.arange(64), 64, 0.5),
                  philox.keep_mask(7 + (1 << 32), 0, 0, np.arange(64), 64, 0.5)):
        assert 0.3 < (a != other).mean() < 0.7
    # keys 4t .. 4t+3 take different slots of a call: not all equal within groups
    g = a.reshape(64, 16, 4)
    assert (g != g[..., :1]).any(axis=2).mean() > 0.5
    # rows restricted to a subset agree with the full mask
    assert np.array_equal(philox.keep_mask(7, 0, 0, [5, 40], 64, 0.5), a[[5, 40]])
    assert philox.keep_mask(7, 0, 0, np.arange(8), 64, 0.0).all()


def load_dropout_golden():
    """Rows of tests/golden/dropout_keep_slots.txt as dicts: the element
    (seed, b, h, i, j), the Philox counter and key written out by hand from
    the mask's definition, the output word and half holding its slot, and
    (zero-counter rows only) the published 16-bit slot value with its keep
    bits at p = 0.5 and p = 0.75."""
    rows = []
    with open(os.path.join(GOLDEN, "dropout_keep_slots.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            elem, ctr, slot, val = (x.split() for x in line.split("|"))
            seed = int(elem[0], 16)
            b, h, i, j = (int(x) for x in elem[1:])
            c = [int(x) for x in ctr[:4]] + [int(x, 16) for x in ctr[4:]]
            u16 = None if val[0] == "-" else int(val[0], 16)
            keeps = None if u16 is None else {0.5: val[1] == "1", 0.75: val[2] == "1"}
            rows.append(dict(seed=seed, b=b, h=h, i=i, j=j, counter=c[:4], key=c[4:],
                             word=int(slot[0]), half=int(slot[1]), u16=u16, keeps=keeps))
    return rows


def golden_slot_value(row):
    """The 16-bit slot of a golden row: the published value, else the
    generator (pinned by its known-answer vectors) at the row's hand-written
    counter and key."""
    from oracle import philox
    if row["u16"] is not None:
        return row["u16"]
    words = philox.philox4x32_10(*row["counter"], *row["key"])
    return (int(words[row["word"]]) >> (16 * row["half"])) & 0xFFFF


def check_dropout_slots_golden(A):
    """The oracle's keep-mask takes each element's decision from the call and
    slot that the hand-worked table assigns it (key -> counter word, output
    word and half; row, head and sequence -> the other counter words; seed ->
    key), at several p; on the zero counter the slots and keep bits are the
    published generator output itself."""
    rows = load_dropout_golden()
    assert len(rows) == 20
    for r in rows:
        u = golden_slot_value(r)
        assert r["seed"] & 0xFFFFFFFF == r["key"][0] and r["seed"] >> 32 == r["key"][1]
        for p in (0.1, 0.5, 0.75, 0.9):
            keep = A._keep(p, r["seed"], r["b"], r["h"], np.array([r["i"]]), r["j"] + 1)
            want = u >= int(p * 65536)
            assert bool(keep[0, r["j"]]) == want, (r, p, hex(u))
            if r["keeps"] is not None and p in r["keeps"]:
                assert want == r["keeps"][p], (r, p)


def _torch_dropout_reference(q, k, v, scale, causal, keep, p):
    """O = (softmax(S) * Z / (1 - p)) V in float64 torch, one head [n, d]."""
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = scale * tq @ tk.T
    if causal:
        n, m = s.shape
        s = s.masked_fill(torch.ones(n, m, dtype=torch.bool).triu(m - n + 1), float("-inf"))
    pr = torch.softmax(s, dim=1)
    return (pr * torch.from_numpy(keep.astype(np.float64)) / (1 - p)) @ tv


def check_dropout_matches_masked_softmax(A):
    """Forward with dropout equals torch's softmax times the keep-mask over
    1 - p, times V; LSE is that of the undropped scores; p = 0 (or a p whose
    threshold is 0) is plain attention.  The p here are multiples of 2^-16,
    for which 1 / (1 - p) is exactly the mask's scale."""
    from oracle import philox
    rng = _rng(45)
    q, k, v = _dense(rng, 2, 13, 18, 4, 2, 8)
    for causal, p in [(False, 0.3125), (True, 0.625)]:
        o, lse = A.attn_fwd(q, k, v, 0.5, causal, dropout_p=p, seed=99)
        _, lse0 = A.attn_fwd(q, k, v, 0.5, causal)
        assert np.allclose(lse, lse0, atol=1e-12)
        for b in range(2):
            for h in range(4):
                keep = philox.keep_mask(99, b, h, np.arange(13), 18, p)
                ref = _torch_dropout_reference(q[b, :, h], k[b, :, h // 2], v[b, :, h // 2],
                                               0.5, causal, keep, p).numpy()
                assert np.allclose(o[b, :, h], ref, atol=1e-12)
    o1, _ = A.attn_fwd(q, k, v, 0.5, True, dropout_p=1e-12, seed=5)
    o2, _ = A.attn_fwd(q, k, v, 0.5, True)
    assert np.allclose(o1, o2, atol=1e-10)


def check_dropout_unbiased(A):
    """Averaged over many seeds the dropped output approaches the plain one
    (E[Z] times the scale is 1), within five standard errors; p = 0.4 is not
    a multiple of 2^-16, so this also pins the scale to the mask's exact keep
    probability."""
    rng = _rng(46)
    q, k, v = _dense(rng, 1, 6, 9, 1, 1, 4)
    o0, _ = A.attn_fwd(q, k, v, 0.7)
    outs = np.stack([A.attn_fwd(q, k, v, 0.7, dropout_p=0.4, seed=s)[0] for s in range(600)])
    err = np.abs(outs.mean(axis=0) - o0)
    se = outs.std(axis=0) / math.sqrt(len(outs))
    assert np.all(err <= 5 * se + 1e-12)


def check_dropout_backward(A):
    """Gradients with dropout against torch autograd through the masked
    softmax (same keep-mask), and central finite differences."""
    from oracle import philox
    rng = _rng(47)
    q, k, v = _dense(rng, 1, 10, 14, 2, 1, 6)
    do = rng.standard_normal(q.shape)
    p = 0.375
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.6, True, dropout_p=p, seed=11)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    loss = 0
    for h in range(2):
        keep = philox.keep_mask(11, 0, h, np.arange(10), 14, p)
        s = 0.6 * tq[0, :, h] @ tk[0, :, 0].T
        s = s.masked_fill(torch.ones(10, 14, dtype=torch.bool).triu(5), float("-inf"))
        o = (torch.softmax(s, 1) * torch.from_numpy(keep.astype(np.float64)) / (1 - p)) @ tv[0, :, 0]
        loss = loss + (o * torch.from_numpy(do[0, :, h])).sum()
    loss.backward()
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)
    q, k, v = _dense(rng, 1, 5, 6, 1, 1, 3)
    do = rng.standard_normal(q.shape)
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.8, False, dropout_p=0.5, seed=3)
    f = lambda: float((A.attn_fwd(q, k, v, 0.8, dropout_p=0.5, seed=3)[0] * do).sum())
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x[idx] += h
            fp = f()
            x[idx] -= 2 * h
            fm = f()
            x[idx] += h
            num[idx] = (fp - fm) / (2 * h)
        assert np.abs(num - g).max() <= 1e-6 * max(np.abs(num).max(), 1e-30)


ALL_FORWARD = [check_rows_sum_to_one, check_identical_keys, check_dominant_score,
               check_permutation_invariance, check_lse_is_logsumexp,
               check_scale_zero, check_against_torch_sdpa, check_brute_force_tiny,
               check_hand_worked_golden, check_gqa_is_repeated_mha,
               check_varlen_is_concatenation, check_key_translation,
               check_causal_row_zero, check_chunked_prefill_alignment,
               check_empty_rows, check_bias_against_torch_sdpa,
               check_bias_row_constant, check_bias_is_key_shift,
               check_bias_mask_equals_causal, check_philox_known_answers,
               check_dropout_mask_statistics, check_dropout_slots_golden,
               check_dropout_matches_masked_softmax,
               check_dropout_unbiased]
ALL_BACKWARD = [check_backward_finite_differences, check_backward_autograd,
                check_backward_invariants, check_bias_backward_autograd,
                check_dropout_backward]
