"""Helpers shared by the GPU parity tests: moving the seeded inputs to the
device, calling the library through its binding, and the error metrics with
the tolerances the parity bar states."""

import math
import sys

import numpy as np

# Parity bar (bf16 path): O max |err| <= 2e-2 and mean |err| <= 2e-3 over all
# compared elements; LSE |err| <= 1e-3; each of dQ, dK, dV:
# max |err| <= 5e-2 * max |reference|.
O_MAX, O_MEAN, LSE_MAX, GRAD_REL = 2e-2, 2e-3, 1e-3, 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to({"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype])
    return t.cuda()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def run_fwd(inp):
    """Call fa_fwd (fa_fwd_f16, fa_fwd_f32) on a workloads.make_inputs() dict."""
    import torch
    import exact_io_aware_28_amd as fa
    dt = inp.get("dtype", "bf16")
    q, k, v = (to_dev(inp[n], dt) for n in ("q", "k", "v"))
    cu = inp.get("cu_seqlens")
    cu_t = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    fn = {"bf16": fa.fa_fwd, "f16": fa.fa_fwd_f16, "f32": fa.fa_fwd_f32}[dt]
    o, lse = fn(q, k, v, scale=inp["scale"], causal=inp["causal"], window=inp["window"],
                cu_seqlens=cu_t, max_seqlen=inp.get("Nq") if cu is not None else None)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, o=o, lse=lse, cu=cu_t)


def run_bwd(inp, dev):
    """Call fa_bwd (fa_bwd_f16 for fp16 inputs) on the outputs of run_fwd."""
    import torch
    import exact_io_aware_28_amd as fa
    dt = inp.get("dtype", "bf16")
    do = to_dev(inp["do"], dt)
    cu = dev["cu"]
    fn = {"bf16": fa.fa_bwd, "f16": fa.fa_bwd_f16}[dt]
    dq, dk, dv = fn(dev["q"], dev["k"], dev["v"], dev["o"], do, dev["lse"],
                    scale=inp["scale"], causal=inp["causal"], window=inp["window"],
                    cu_seqlens=cu, max_seqlen=inp.get("Nq") if cu is not None else None)
    torch.cuda.synchronize()
    return dq, dk, dv


def o_errors(o, ref):
    err = np.abs(o - ref)
    return float(err.max()), float(err.mean())


def check_o(o, ref, what="", bar_scale=1.0):
    """O against the bars; bar_scale > 1 only where a derived bar applies
    (dropout above p = 0.5, whose kept values grow by 1 / (1 - p))."""
    mx, mn = o_errors(o, ref)
    say(f"  {what} O max|err|={mx:.3e} mean|err|={mn:.3e}"
        + (f" (bars x{bar_scale:.3g})" if bar_scale != 1.0 else ""))
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert mx <= O_MAX * bar_scale and mn <= O_MEAN * bar_scale, (what, mx, mn)
    return mx, mn


def dropout_bar_scale(p):
    """Bar multiplier for O with dropout probability p: 1 (the stated bars)
    for p <= 0.5.  Above that the kept probabilities, O itself and its bf16
    rounding all grow by 1 / (1 - p) (10x at p = 0.9) while the inputs do
    not, so the bars grow by the same factor."""
    return 1.0 if p <= 0.5 else 1.0 / (1.0 - p)


def check_lse(lse, ref, what=""):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref)), f"{what}: -inf pattern"
    mx = float(np.abs(lse[fin] - ref[fin]).max()) if fin.any() else 0.0
    say(f"  {what} LSE max|err|={mx:.3e}")
    assert mx <= LSE_MAX, (what, mx)
    return mx


def check_grad(g, ref, what="", floor=None):
    """Gradient bar: max |err| <= 5e-2 * max |ref|; with `floor` (an array
    shaped like g, d_rounding_floor) each element may also differ by its
    floor, the bound of the error that the bf16 O inside D carries."""
    scale = float(np.abs(ref).max())
    err = np.abs(g - ref)
    mx = float(err.max())
    say(f"  {what} max|err|={mx:.3e} max|ref|={scale:.3e} rel={mx / max(scale, 1e-30):.3e}"
        + ("" if floor is None else f" floor max={float(np.max(floor)):.3e}"))
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    if floor is None:
        assert mx <= GRAD_REL * scale, (what, mx, scale)
    else:
        excess = float((err - (GRAD_REL * scale + floor)).max())
        assert excess <= 0.0, (what, mx, scale, excess)
    return mx / max(scale, 1e-30)


def d_rounding_floor(inp, o, lse_ref, unit=2.0 ** -9):
    """Elementwise first-order bound of the dQ and dK error that comes from
    forming D_i = sum_c dO_ic O_ic from the bf16 O the backward receives (the
    exact gradients use the exact O).  Rounding O to bf16 (to nearest) moves
    D_i by at most e_i = unit sum_c |dO_ic O_ic| (unit = 2^-9, half a bf16
    step; 2^-12 for an fp16 O); through
    dS_ij = P_ij (dP_ij - D_i) that moves dQ_ic by at most
    scale e_i sum_j P_ij |K_jc|, and dK_jc by at most
    scale sum_i P_ij e_i |Q_ic| (summed over the query heads of the KV head).
    P (undropped, with the bias) is rebuilt from the oracle's LSE.  Matters
    where the exact gradient vanishes, e.g. every row seeing one key with
    dropout (D from the rounded O then differs from the kept dP).
    Returns (floor_dq, floor_dk) shaped like Q and K."""
    import oracle
    q, k, do = (np.asarray(inp[n], np.float64) for n in ("q", "k", "do"))
    o = np.asarray(o, np.float64)
    scale, causal, window = inp["scale"], inp["causal"], inp["window"]
    bias = inp.get("bias")
    cu = inp.get("cu_seqlens")
    if cu is None:
        spans = [(b, None) for b in range(q.shape[0])]
    else:
        spans = [(None, (int(cu[s]), int(cu[s + 1]))) for s in range(len(cu) - 1)]
    fq, fk = np.zeros_like(q), np.zeros_like(k)
    hq, hkv = q.shape[-2], k.shape[-2]
    g = hq // hkv
    for b, span in spans:
        if span is None:
            qs, ks, dos, os_ = q[b], k[b], do[b], o[b]
            lse = lambda h: np.asarray(lse_ref[b, h], np.float64)
        else:
            a, e = span
            qs, ks, dos, os_ = q[a:e], k[a:e], do[a:e], o[a:e]
            lse = lambda h, a=a, e=e: np.asarray(lse_ref[h, a:e], np.float64)
        nq, nk = qs.shape[0], ks.shape[0]
        if nq == 0 or nk == 0:
            continue
        ok = oracle.allowed_mask(nq, nk, causal, window)
        for h in range(hq):
            kv = h // g
            s = scale * (qs[:, h] @ ks[:, kv].T)
            if bias is not None:
                s = s + np.broadcast_to(bias, (q.shape[0], hq, nq, nk))[b, h]
            l = lse(h)
            fin = np.isfinite(l)[:, None] & ok
            with np.errstate(invalid="ignore", over="ignore"):  # rows that see no key
                p = np.where(fin, np.exp(np.where(fin, s - l[:, None], -np.inf)), 0.0)
            e_i = unit * np.abs(dos[:, h] * os_[:, h]).sum(axis=1)
            fq_h = scale * e_i[:, None] * (p @ np.abs(ks[:, kv]))
            fk_h = scale * (p * e_i[:, None]).T @ np.abs(qs[:, h])
            if span is None:
                fq[b, :, h] += fq_h
                fk[b, :, kv] += fk_h
            else:
                fq[a:e, h] += fq_h
                fk[a:e, kv] += fk_h
    return fq, fk


def sample_rows(n, tile=128, count=48, seed=0):
    """Rows that cover the first and last rows, tile edges and random rows."""
    rng = np.random.default_rng(seed)
    s = {0, 1, n - 1, n - 2}
    for t in range(tile, n, tile):
        if len(s) > count // 2:
            break
        s.update({t - 1, t})
    s.update(rng.integers(0, n, size=count - len(s) if count > len(s) else 0).tolist())
    return np.array(sorted(x for x in s if 0 <= x < n))


def attention_flops(B, Hq, Nq, Nk, d, causal):
    f = 4.0 * B * Hq * Nq * Nk * d
    return f / 2 if causal else f


def is_close_bits(a, b):
    return a.shape == b.shape and bool((a == b).all())


__all__ = ["say", "to_dev", "to_np", "run_fwd", "run_bwd", "check_o", "check_lse",
           "dropout_bar_scale", "d_rounding_floor",
           "check_grad", "sample_rows", "math"]
