"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs (workloads.make_inputs), runs the library on
cuda:0 and compares with the oracle on exactly the same (bf16-rounded)
values.  Small cases compare every element; the full-size workloads compare
whole heads plus sampled rows of every head (the oracle computes any row on
its own).  Tolerances: O max|err| <= 2e-2 and mean|err| <= 2e-3, LSE |err| <=
1e-3, gradients max|err| <= 5e-2 * max|ref| (tests/gpu_util.py).
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (check_grad, check_lse, check_o, run_bwd, run_fwd, say,
                            sample_rows, to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()  # fail loudly if the library is missing


def _dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed, dtype="bf16", bwd=False, scale=None):
    spec = dict(B=B, Nq=Nq, Nk=Nk, Hq=Hq, Hkv=Hkv, d=d, causal=causal, window=window,
                dtype=dtype, seed=seed, bwd=bwd)
    if scale is not None:
        spec["scale"] = scale
    return workloads.make_inputs(spec)


def _packed(lengths, Hq, Hkv, d, causal, window, seed, dtype="bf16", bwd=False):
    return workloads.make_inputs(dict(lengths=lengths, Hq=Hq, Hkv=Hkv, d=d, causal=causal,
                                      window=window, dtype=dtype, seed=seed, bwd=bwd))


def _oracle_fwd(inp):
    return oracle.attn_fwd(inp["q"].astype(np.float64), inp["k"].astype(np.float64),
                           inp["v"].astype(np.float64), inp["scale"], inp["causal"],
                           inp["window"], inp.get("cu_seqlens"))


def _compare_full(inp, what):
    say(f"[fwd] {what}")
    dev = run_fwd(inp)
    o_ref, lse_ref = _oracle_fwd(inp)
    check_o(to_np(dev["o"]), o_ref, what)
    check_lse(dev["lse"].cpu().numpy().astype(np.float64), lse_ref, what)
    return dev, o_ref, lse_ref


# ------------------------------------------------------------ small, full compare
DENSE_CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, window
    (2, 300, 300, 4, 2, 128, True, 0),
    (2, 300, 300, 4, 2, 128, False, 0),
    (1, 300, 300, 4, 4, 64, True, 0),
    (2, 200, 200, 4, 2, 64, False, 0),
    (1, 257, 257, 8, 1, 128, True, 0),        # MQA
    (1, 500, 500, 4, 2, 128, True, 100),      # causal + window
    (1, 500, 500, 2, 2, 64, False, 77),       # window only
    (1, 100, 300, 4, 2, 128, True, 0),        # chunked prefill, bottom-right
    (1, 100, 300, 4, 2, 64, True, 40),
    (1, 300, 100, 4, 2, 128, True, 0),        # rows that see no key
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 64, 64, 2, 1, 128, True, 1),          # each query sees only itself
    (3, 128, 128, 2, 2, 128, True, 0),        # exact tile multiples
    (1, 1000, 1000, 2, 1, 128, True, 0),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fwd_dense_small(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    _compare_full(_dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=101), str(case))


PACKED = [0, 1, 63, 64, 65, 129, 300, 2, 128, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 50), (False, 33)])
def test_fwd_packed_small(d, causal, window):
    inp = _packed(PACKED, 4, 2, d, causal, window, seed=102)
    _compare_full(inp, f"packed d={d} causal={causal} window={window}")


@pytest.mark.parametrize("case", [
    (1, 128, 128, 1, 1, 64, False, 0),
    (2, 150, 150, 4, 2, 128, True, 0),
    (1, 200, 200, 2, 2, 64, True, 30),
    (1, 70, 190, 2, 1, 128, True, 0),
], ids=lambda c: "-".join(map(str, c)))
def test_fwd_f32_small(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    inp = _dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=103, dtype="f32")
    dev, o_ref, lse_ref = _compare_full(inp, "f32 " + str(case))
    # fp32 arithmetic: far inside the bf16 bar
    assert np.abs(to_np(dev["o"]) - o_ref).max() < 1e-4


def test_fwd_f32_packed():
    inp = _packed([5, 0, 64, 130], 2, 1, 128, True, 20, seed=104, dtype="f32")
    dev, o_ref, _ = _compare_full(inp, "f32 packed")
    assert np.abs(to_np(dev["o"]) - o_ref).max() < 1e-4


# fp16 operands: P and O carry 11 significant bits instead of bf16's 8, so the
# error sits well inside the bf16 bar; the tighter bound below would fail if
# P or O were rounded to bf16 (and a bf16 reading of fp16 bits fails outright).
F16_CASES = [
    (2, 300, 300, 4, 2, 128, True, 0),
    (1, 260, 260, 4, 4, 64, False, 0),
    (1, 257, 257, 8, 1, 128, True, 0),        # MQA
    (1, 500, 500, 4, 2, 128, True, 100),      # causal + window
    (1, 100, 300, 4, 2, 64, True, 40),        # chunked prefill
    (1, 300, 100, 4, 2, 128, True, 0),        # rows that see no key
]


@pytest.mark.parametrize("case", F16_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fwd_f16_small(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    inp = _dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=112, dtype="f16")
    dev, o_ref, _ = _compare_full(inp, "f16 " + str(case))
    assert np.abs(to_np(dev["o"]) - o_ref).max() < 3e-3


def test_fwd_f16_packed():
    inp = _packed(PACKED, 4, 2, 128, True, 50, seed=113, dtype="f16")
    dev, o_ref, _ = _compare_full(inp, "f16 packed")
    assert np.abs(to_np(dev["o"]) - o_ref).max() < 3e-3


# Short causal grids dispatch each XCD's longest query tiles first across the
# KV-head groups it owns (the launcher's xcd_groups); the condition below
# restates the launcher's so that each case is known to take that path.
def _xcd_groups(B, Nq, Hq, Hkv, d):
    rows = 256 if d == 128 else 128
    nq = -(-Nq // rows)
    n, unit = B * Hq * nq, (Hq // Hkv) * nq
    per, slots = n // 8, 32 * (1 if d == 128 else 3)
    ok = n % 8 == 0 and per % unit == 0 and per // unit > 1 and per <= 2 * slots
    return per // unit if ok else 0


@pytest.mark.parametrize("case", [
    (2, 512, 512, 8, 8, 128, True, 0),
    (4, 600, 600, 8, 4, 128, True, 0),
    (4, 300, 300, 4, 4, 64, True, 100),
    (8, 700, 700, 8, 2, 64, True, 0),
], ids=lambda c: "-".join(map(str, c)))
def test_fwd_xcd_longest_first(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    assert _xcd_groups(B, Nq, Hq, Hkv, d) > 1, case
    _compare_full(_dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=114),
                  "xcd order " + str(case))


# ------------------------------------------------------------ properties
def test_scale_zero_gives_counts():
    """scale = 0: LSE = ln(#visible keys) and O = mean of the visible V."""
    inp = _dense(1, 400, 400, 2, 1, 128, True, 150, seed=105, scale=0.0)
    dev = run_fwd(inp)
    lse = dev["lse"].cpu().numpy()
    n = np.minimum(np.arange(400) + 1, 150)
    assert np.abs(lse[0] - np.log(n)[None]).max() < 1e-4
    o_ref, _ = _oracle_fwd(inp)
    check_o(to_np(dev["o"]), o_ref, "scale=0")


def test_negative_and_large_scale():
    for scale in (-0.3, 2.0):
        inp = _dense(1, 260, 260, 4, 2, 128, True, 0, seed=106, scale=scale)
        _compare_full(inp, f"scale={scale}")


def test_growing_row_maximum():
    """Scores whose row maximum keeps growing along the keys exercise every
    rescale of the running state (keys scaled up along the sequence)."""
    inp = _dense(1, 512, 512, 2, 1, 128, False, 0, seed=107)
    ramp = np.linspace(0.2, 3.0, 512, dtype=np.float32)[None, :, None, None]
    inp["k"] = workloads.round_bf16(inp["k"] * ramp)
    _compare_full(inp, "growing max")


def test_identical_keys_and_dominant_score():
    inp = _dense(1, 256, 256, 2, 1, 128, True, 0, seed=108)
    inp["k"][:] = inp["k"][:, :1]
    dev = run_fwd(inp)
    prefix = np.cumsum(inp["v"][0, :, 0].astype(np.float64), 0) / np.arange(1, 257)[:, None]
    assert np.abs(to_np(dev["o"])[0, :, 0] - prefix).max() < 2e-2
    inp = _dense(1, 256, 256, 1, 1, 128, False, 0, seed=109)
    inp["k"][0, 77, 0] = workloads.round_bf16(inp["q"][0, 5, 0] * 4.0)
    dev = run_fwd(inp)
    assert np.abs(to_np(dev["o"])[0, 5, 0] - inp["v"][0, 77, 0]).max() < 2e-2


def test_nan_poisoning_pattern():
    inp = _dense(1, 300, 300, 1, 1, 128, True, 0, seed=110)
    inp["q"][0, 150, 0, 3] = np.nan
    inp["k"][0, 200, 0, 7] = np.nan
    dev = run_fwd(inp)
    o = to_np(dev["o"])[0, :, 0]
    bad = ~np.isfinite(o).all(axis=1)
    want = np.zeros(300, bool)
    want[150] = True
    want[200:] = True
    assert np.array_equal(bad, want)


def test_deterministic():
    import torch
    inp = _dense(2, 700, 700, 4, 2, 128, True, 0, seed=111, bwd=True)
    a = run_fwd(inp)
    b = run_fwd(inp)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    g1 = run_bwd(inp, a)
    g2 = run_bwd(inp, a)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


# ------------------------------------------------------------ backward, full
BWD_CASES = [
    (2, 300, 300, 4, 2, 128, True, 0),
    (1, 200, 200, 4, 4, 64, False, 0),
    (1, 300, 300, 4, 2, 128, True, 70),
    (1, 100, 300, 4, 2, 128, True, 0),
    (1, 257, 257, 8, 1, 64, True, 0),
    (1, 128, 128, 2, 2, 128, False, 0),
    (1, 300, 333, 4, 2, 128, False, 0),
]


def _oracle_bwd(inp):
    f = lambda n: inp[n].astype(np.float64)
    return oracle.attn_bwd(f("q"), f("k"), f("v"), f("do"), inp["scale"], inp["causal"],
                           inp["window"], inp.get("cu_seqlens"))


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_dense_small(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    inp = _dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=120, bwd=True)
    say(f"[bwd] {case}")
    dev = run_fwd(inp)
    dq, dk, dv = run_bwd(inp, dev)
    rq, rk, rv = _oracle_bwd(inp)
    check_grad(to_np(dq), rq, "dQ")
    check_grad(to_np(dk), rk, "dK")
    check_grad(to_np(dv), rv, "dV")


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 45)])
def test_bwd_packed_small(causal, window):
    inp = _packed([1, 64, 65, 200, 0, 130], 4, 2, 128, causal, window, seed=121, bwd=True)
    say(f"[bwd] packed causal={causal} window={window}")
    dev = run_fwd(inp)
    dq, dk, dv = run_bwd(inp, dev)
    rq, rk, rv = _oracle_bwd(inp)
    check_grad(to_np(dq), rq, "dQ")
    check_grad(to_np(dk), rk, "dK")
    check_grad(to_np(dv), rv, "dV")


# fp16 backward: the same cases in IEEE half.  P and dS are rounded to fp16 as
# MFMA operands (11 significant bits against bf16's 8), so the gradients sit
# well inside the bf16 bar.  F16_GRAD_REL is checked as well: the fp16 path
# measured at most 7.1e-4 of max|ref| on these cases, the bf16 backward of
# the same shapes 1.9e-3 to 5.7e-3, so bf16 operands in the fp16 path would
# fail it.
F16_GRAD_REL = 2e-3


def _bwd_f16_check(inp, what):
    say(f"[bwd f16] {what}")
    dev = run_fwd(inp)
    grads = run_bwd(inp, dev)
    for name, g, r in zip(("dQ", "dK", "dV"), grads, _oracle_bwd(inp)):
        assert g.dtype == dev["q"].dtype
        rel = check_grad(to_np(g), r, f"f16 {what} {name}")
        assert rel <= F16_GRAD_REL, (what, name, rel)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_f16_dense_small(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    _bwd_f16_check(_dense(B, Nq, Nk, Hq, Hkv, d, causal, window, seed=122, dtype="f16",
                          bwd=True), str(case))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 45)])
def test_bwd_f16_packed_small(d, causal, window):
    inp = _packed([1, 64, 65, 200, 0, 130], 4, 2, d, causal, window, seed=123, dtype="f16",
                  bwd=True)
    _bwd_f16_check(inp, f"packed d={d} causal={causal} window={window}")


# ------------------------------------------------------------ full-size workloads
def test_workload_single_head_f32():
    inp = workloads.make_inputs("single_head_f32")
    dev, o_ref, _ = _compare_full(inp, "single_head_f32 B=1 H=1 N=128 d=64")
    assert np.abs(to_np(dev["o"]) - o_ref).max() < 1e-4


@pytest.mark.parametrize("name", ["mha_d64", "mha_d64_causal"])
def test_workload_mha_d64(name):
    _compare_full(workloads.make_inputs(name), name + " B=4 H=16 N=2048 d=64")


def _sampled_heads_compare(inp, dev, full_heads, rows, what):
    """Whole heads `full_heads` and rows `rows` of every head (dense batch)."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    o = to_np(dev["o"])
    lse = dev["lse"].cpu().numpy().astype(np.float64)
    errs_o, errs_ref, errs_l = [], [], []
    for b in range(B):
        for h in range(Hq):
            g = oracle.kv_head_of(h, Hq, Hkv)
            rr = np.arange(Nq) if (b, h) in full_heads else rows
            ro, rl = oracle.attn_fwd_rows(q[b, :, h], k[b, :, g], v[b, :, g], rr,
                                          inp["scale"], inp["causal"], inp["window"])
            errs_o.append(o[b, rr, h])
            errs_ref.append(ro)
            errs_l.append(np.abs(lse[b, h, rr] - rl))
    check_o(np.concatenate(errs_o), np.concatenate(errs_ref), what)
    lmax = max(float(e.max()) for e in errs_l)
    say(f"  {what} LSE max|err|={lmax:.3e}")
    assert lmax <= 1e-3


def test_workload_gqa_causal_prefill():
    inp = workloads.make_inputs("gqa_causal_prefill")
    say("[fwd] gqa_causal_prefill B=1 Hq=32 Hkv=8 N=8192 d=128 causal")
    dev = run_fwd(inp)
    _sampled_heads_compare(inp, dev, {(0, 0), (0, 13)}, sample_rows(8192, count=64, seed=3),
                           "gqa_causal_prefill")


def test_workload_gqa_causal_prefill_f16():
    inp = workloads.make_inputs(dict(workloads.WORKLOADS["gqa_causal_prefill"], dtype="f16"))
    say("[fwd] gqa_causal_prefill fp16 B=1 Hq=32 Hkv=8 N=8192 d=128 causal")
    dev = run_fwd(inp)
    _sampled_heads_compare(inp, dev, {(0, 21)}, sample_rows(8192, count=32, seed=4),
                           "gqa_causal_prefill fp16")


def test_workload_varlen_window():
    inp = workloads.make_inputs("varlen_window")
    say(f"[fwd] varlen_window T={inp['T']} Hq=32 Hkv=8 d=128 causal window=4096")
    dev = run_fwd(inp)
    o = to_np(dev["o"])
    lse = dev["lse"].cpu().numpy().astype(np.float64)
    cu = inp["cu_seqlens"]
    outs, refs, lerr = [], [], 0.0
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        L = e - a
        for h in range(32):
            g = h // 4
            rows = np.arange(L) if h in (0, 29) else sample_rows(L, count=12, seed=s)
            ro, rl = oracle.attn_fwd_rows(inp["q"][a:e, h], inp["k"][a:e, g], inp["v"][a:e, g],
                                          rows, inp["scale"], True, 4096)
            outs.append(o[a + rows, h])
            refs.append(ro)
            lerr = max(lerr, float(np.abs(lse[h, a + rows] - rl).max()))
    check_o(np.concatenate(outs), np.concatenate(refs), "varlen_window")
    say(f"  varlen_window LSE max|err|={lerr:.3e}")
    assert lerr <= 1e-3


def test_workload_long_fwd_bwd():
    inp = workloads.make_inputs("long_fwd_bwd")
    say("[fwd+bwd] long_fwd_bwd B=2 H=16 N=16384 d=128 causal")
    dev = run_fwd(inp)
    _sampled_heads_compare(inp, dev, {(1, 9)}, sample_rows(16384, count=32, seed=5),
                           "long_fwd_bwd fwd")
    dq, dk, dv = run_bwd(inp, dev)
    dq, dk, dv = to_np(dq), to_np(dk), to_np(dv)
    f = lambda n: inp[n]
    for b, g in [(0, 3), (1, 14)]:
        qr = sample_rows(16384, count=24, seed=b)
        kr = sample_rows(16384, count=24, seed=g)
        rq, rk, rv = oracle.attn_bwd_sampled(f("q"), f("k"), f("v"), f("do"), inp["scale"],
                                             True, 0, b, g, qr, kr, chunk=4096)
        check_grad(dq[b][qr][:, g:g + 1], rq, f"dQ b={b} h={g}")
        check_grad(dk[b, kr, g], rk, f"dK b={b} h={g}")
        check_grad(dv[b, kr, g], rv, f"dV b={b} h={g}")


def test_workload_long_bwd_whole_head():
    """Every element of dQ, dK and dV of one (batch, head) of the long
    causal workload (B=2, H=16, N=16384, d=128), against the oracle's full
    backward of that head (S, P and dP materialised in fp64, ~6.5 GB)."""
    inp = workloads.make_inputs("long_fwd_bwd")
    say("[bwd whole head] long_fwd_bwd B=2 H=16 N=16384 d=128 causal, head (b=1, h=9)")
    dev = run_fwd(inp)
    dq, dk, dv = run_bwd(inp, dev)
    b, h = 1, 9
    dq, dk, dv = (to_np(t[b:b + 1, :, h:h + 1]) for t in (dq, dk, dv))
    one = lambda n: inp[n][b:b + 1, :, h:h + 1].astype(np.float64)
    rq, rk, rv = oracle.attn_bwd(one("q"), one("k"), one("v"), one("do"), inp["scale"], True)
    check_grad(dq, rq, "dQ whole head")
    check_grad(dk, rk, "dK whole head")
    check_grad(dv, rv, "dV whole head")


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_bwd_scale_sign(scale):
    """The backward with a negative and with a zero scale (several query and
    key tiles, causal, so diagonal tiles are masked).  With scale 0 the exact
    dQ and dK vanish, and the bar asks for exact zeros."""
    inp = _dense(1, 300, 300, 4, 2, 128, True, 0, seed=121, bwd=True, scale=scale)
    say(f"[bwd] scale={scale}")
    dev = run_fwd(inp)
    dq, dk, dv = run_bwd(inp, dev)
    rq, rk, rv = _oracle_bwd(inp)
    check_grad(to_np(dq), rq, f"scale={scale} dQ")
    check_grad(to_np(dk), rk, f"scale={scale} dK")
    check_grad(to_np(dv), rv, f"scale={scale} dV")
