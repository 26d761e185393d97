"""Seeded random sweep of the forward and backward against the fp64 oracle.

The hand-picked cases elsewhere cover each feature on its own; this sweep
draws 40 configurations that mix them: batch, query and key lengths not
tied to the tile sizes (chunked prefill and rows that see no key included),
GQA group sizes 1-8, d = 64 and 128, causal and window masks, packed
batches, and one of no bias, a bias (per head, shared by the heads, or a
key-padding row) or dropout.  Every element of O, LSE, dQ, dK and dV is
compared at the bars of tests/gpu_util.py (the derived dropout bar for O,
and for dQ and dK the bound of the error that forming D from the bf16 O
carries, which decides only where the exact gradient vanishes).
The configurations come from one fixed generator seed, so a failure names a
case that reproduces.  A second draw runs plain attention in fp16 through
fa_fwd_f16 and fa_bwd_f16, and a third the split-KV decode.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (check_grad, check_lse, check_o, d_rounding_floor,
                            dropout_bar_scale, say, to_dev, to_np)

pytestmark = pytest.mark.gpu

N_CASES = 40
N_DECODE = 16
N_F16 = 12


def _draw_cases(n=N_CASES, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 8]))
        causal = bool(rng.integers(0, 2))
        window = int(rng.integers(1, 200)) if rng.random() < 0.3 else 0
        kind = str(rng.choice(["plain", "bias", "dropout"]))
        packed = kind != "bias" and rng.random() < 0.3
        case = dict(id=c, d=d, Hkv=hkv, Hq=hkv * g, causal=causal, window=window, kind=kind,
                    seed=1000 + c)
        if packed:
            case["lengths"] = [int(x) for x in rng.integers(0, 260, size=int(rng.integers(1, 5)))]
        else:
            case["B"] = int(rng.integers(1, 4))
            case["Nq"] = int(rng.integers(1, 520))
            case["Nk"] = case["Nq"] if rng.random() < 0.6 else int(rng.integers(1, 520))
        if kind == "bias":
            case["bias_shape"] = [("B", "H", "Q", "K"), (1, 1, "Q", "K"), ("B", 1, 1, "K")][
                int(rng.integers(0, 3))]
        if kind == "dropout":
            case["p"] = float(np.float32(rng.choice([0.1, 0.3, 0.6])))
            case["drop_seed"] = int(rng.integers(0, 1 << 62))
        cases.append(case)
    return cases


CASES = _draw_cases()


def _name(c):
    shape = (f"lengths={c['lengths']}" if "lengths" in c
             else f"B={c['B']} Nq={c['Nq']} Nk={c['Nk']}")
    extra = {"bias": f" bias={c.get('bias_shape')}", "dropout": f" p={c.get('p')}",
             "plain": ""}[c["kind"]]
    return (f"case {c['id']}: {shape} Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} "
            f"causal={c['causal']} window={c['window']} {c['kind']}{extra}")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()  # fail loudly if the library is missing


def test_cases_are_varied():
    """The draw exercises every kind, both head dims, masks and packing."""
    kinds = {c["kind"] for c in CASES}
    assert kinds == {"plain", "bias", "dropout"}
    assert {c["d"] for c in CASES} == {64, 128}
    assert any(c["causal"] for c in CASES) and any(not c["causal"] for c in CASES)
    assert any(c["window"] for c in CASES) and any("lengths" in c for c in CASES)


@pytest.mark.parametrize("case", CASES, ids=[f"r{c['id']}" for c in CASES])
def test_random_case(case):
    import torch
    import exact_io_aware_28_amd as fa
    what = _name(case)
    say(f"[random] {what}")
    spec = {k: case[k] for k in ("Hq", "Hkv", "d", "causal", "window", "seed")}
    spec["bwd"] = True
    if "lengths" in case:
        spec["lengths"] = case["lengths"]
    else:
        spec.update(B=case["B"], Nq=case["Nq"], Nk=case["Nk"])
    if case["kind"] == "bias":
        spec["bias_shape"] = case["bias_shape"]
    inp = workloads.make_inputs(spec)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    cu = inp.get("cu_seqlens")
    cu_t = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"])
    okw = {}
    if case["kind"] == "bias":
        bias = torch.from_numpy(np.ascontiguousarray(inp["bias"])).cuda()
        o, lse = fa.fa_fwd_bias(q, k, v, bias, **kw)
        grads = fa.fa_bwd_bias(q, k, v, bias, o, do, lse, **kw)
        okw = dict(bias=inp["bias"])
    else:
        kw.update(cu_seqlens=cu_t, max_seqlen=inp["Nq"] if cu is not None else None)
        if case["kind"] == "dropout":
            p, s = case["p"], case["drop_seed"]
            o, lse = fa.fa_fwd_dropout(q, k, v, p, s, **kw)
            grads = fa.fa_bwd_dropout(q, k, v, o, do, lse, p, s, **kw)
            okw = dict(dropout_p=p, seed=s)
        else:
            o, lse = fa.fa_fwd(q, k, v, **kw)
            grads = fa.fa_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    f = lambda n: inp[n].astype(np.float64)
    o_ref, lse_ref = oracle.attn_fwd(f("q"), f("k"), f("v"), inp["scale"], inp["causal"],
                                     inp["window"], cu, **okw)
    bar = dropout_bar_scale(case["p"]) if case["kind"] == "dropout" else 1.0
    check_o(to_np(o), o_ref, what, bar)
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, what)
    ref = oracle.attn_bwd(f("q"), f("k"), f("v"), f("do"), inp["scale"], inp["causal"],
                          inp["window"], cu, **okw)
    # dQ and dK may also differ by the error of forming D from the bf16 O
    # (d_rounding_floor); it decides only where the exact gradient vanishes
    fq, fk = d_rounding_floor(inp, to_np(o), lse_ref)
    for name, g, r, fl in zip(("dQ", "dK", "dV"), grads, ref, (fq, fk, None)):
        check_grad(to_np(g), r, f"{what} {name}", fl)


# ------------------------------------------------------------ fp16 operands
def _draw_f16(n=N_F16, seed=20261205):
    """Plain attention in IEEE half (fa_fwd_f16 / fa_bwd_f16): the same
    mix of shapes, masks, GQA groups and packing as the bf16 draw."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        hkv = int(rng.choice([1, 2]))
        case = dict(id=c, d=int(rng.choice([64, 128])), Hkv=hkv,
                    Hq=hkv * int(rng.choice([1, 2, 4, 8])), causal=bool(rng.integers(0, 2)),
                    window=int(rng.integers(1, 200)) if rng.random() < 0.3 else 0,
                    seed=3000 + c)
        if rng.random() < 0.3:
            case["lengths"] = [int(x) for x in rng.integers(0, 260, size=int(rng.integers(1, 5)))]
        else:
            case["B"] = int(rng.integers(1, 4))
            case["Nq"] = int(rng.integers(1, 520))
            case["Nk"] = case["Nq"] if rng.random() < 0.6 else int(rng.integers(1, 520))
        cases.append(case)
    return cases


F16_CASES = _draw_f16()


@pytest.mark.parametrize("case", F16_CASES, ids=[f"h{c['id']}" for c in F16_CASES])
def test_random_f16(case):
    """O, LSE, dQ, dK, dV in fp16 against the oracle on the fp16-rounded
    inputs, at the bars of the bf16 sweep (the D floor with fp16's unit)."""
    import torch
    import exact_io_aware_28_amd as fa
    shape = (f"lengths={case['lengths']}" if "lengths" in case
             else f"B={case['B']} Nq={case['Nq']} Nk={case['Nk']}")
    what = (f"f16 case {case['id']}: {shape} Hq={case['Hq']} Hkv={case['Hkv']} d={case['d']} "
            f"causal={case['causal']} window={case['window']}")
    say(f"[random] {what}")
    spec = {k: case[k] for k in ("Hq", "Hkv", "d", "causal", "window", "seed")}
    spec.update(bwd=True, dtype="f16")
    if "lengths" in case:
        spec["lengths"] = case["lengths"]
    else:
        spec.update(B=case["B"], Nq=case["Nq"], Nk=case["Nk"])
    inp = workloads.make_inputs(spec)
    q, k, v, do = (to_dev(inp[n], "f16") for n in ("q", "k", "v", "do"))
    cu = inp.get("cu_seqlens")
    cu_t = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"], cu_seqlens=cu_t,
              max_seqlen=inp["Nq"] if cu is not None else None)
    o, lse = fa.fa_fwd_f16(q, k, v, **kw)
    grads = fa.fa_bwd_f16(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16 and all(g.dtype == torch.float16 for g in grads)
    f = lambda n: inp[n].astype(np.float64)
    o_ref, lse_ref = oracle.attn_fwd(f("q"), f("k"), f("v"), inp["scale"], inp["causal"],
                                     inp["window"], cu)
    check_o(to_np(o), o_ref, what)
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, what)
    ref = oracle.attn_bwd(f("q"), f("k"), f("v"), f("do"), inp["scale"], inp["causal"],
                          inp["window"], cu)
    fq, fk = d_rounding_floor(inp, to_np(o), lse_ref, unit=2.0 ** -12)
    for name, g, r, fl in zip(("dQ", "dK", "dV"), grads, ref, (fq, fk, None)):
        check_grad(to_np(g), r, f"{what} {name}", fl)


# ------------------------------------------------------------ split-KV decode
def _draw_decode(n=N_DECODE, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 4, 8]))
        nk = int(rng.integers(1, 3000))
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(0, nk + 1, size=B)]
        cases.append(dict(id=c, B=B, Hq=hkv * g, Hkv=hkv, Nq=int(rng.integers(1, 5)), Nk=nk,
                          d=int(rng.choice([64, 128])), lengths=lengths,
                          causal=bool(rng.integers(0, 2)),
                          window=int(rng.integers(1, 800)) if rng.random() < 0.3 else 0,
                          splits=int(rng.integers(1, 40)) if rng.random() < 0.5 else None,
                          noalloc=bool(rng.random() < 0.3), seed=2000 + c))
    return cases


DECODE_CASES = _draw_decode()


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"d{c['id']}" for c in DECODE_CASES])
def test_random_decode(case):
    """fa_decode (or fa_decode_noalloc) against attn_fwd on each sequence's
    query rows and its first seqlens_k keys."""
    import torch
    import exact_io_aware_28_amd as fa
    what = (f"decode case {case['id']}: B={case['B']} Hq={case['Hq']} Hkv={case['Hkv']} "
            f"Nq={case['Nq']} Nk={case['Nk']} d={case['d']} lengths={case['lengths']} "
            f"causal={case['causal']} window={case['window']} splits={case['splits']} "
            f"noalloc={case['noalloc']}")
    say(f"[random] {what}")
    inp = workloads.make_decode_inputs({k: case[k] for k in ("B", "Hq", "Hkv", "Nq", "Nk", "d",
                                                            "lengths", "causal", "window",
                                                            "seed")})
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    lens = torch.from_numpy(np.asarray(inp["seqlens_k"], np.int32)).cuda()
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"], seqlens_k=lens)
    if case["noalloc"]:
        o = torch.empty_like(q)
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                          device="cuda")
        fa.fa_decode_noalloc(q, k, v, out=o, lse=lse, num_splits=case["splits"] or 0, **kw)
    else:
        o, lse = fa.fa_decode(q, k, v, num_splits=case["splits"], **kw)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    nq, hq, d = inp["q"].shape[1:]
    for b in range(case["B"]):
        L = int(inp["seqlens_k"][b])
        if L == 0:
            o_ref, l_ref = np.zeros((nq, hq, d)), np.full((hq, nq), -np.inf)
        else:
            o_ref, l_ref = oracle.attn_fwd(inp["q"][b:b + 1].astype(np.float64),
                                           inp["k"][b:b + 1, :L].astype(np.float64),
                                           inp["v"][b:b + 1, :L].astype(np.float64),
                                           inp["scale"], inp["causal"], inp["window"])
            o_ref, l_ref = o_ref[0], l_ref[0]
        check_o(o[b], o_ref, f"{what} seq {b}")
        check_lse(lse[b], l_ref, f"{what} seq {b}")
