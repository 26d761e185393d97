"""Race check of the LDS double buffers: every kernel that stages tiles by
buffer-to-LDS copies is run from the optimised library and from its
stage-synchronised build (libfa_mi355x_debugsync.so, -DFA_DEBUG_SYNC: every
copy completes and the work-group meets after each copy and after each tile,
so no copy overlaps any read of LDS).  The kernels are deterministic, so a
copy that overwrote a buffer still being read, or a read that ran ahead of
its copy, would show as different bits; the two builds must agree exactly.
One mid-size case per kernel: forward (d = 128 causal, d = 64, packed with a
window, fp16, bias, dropout, FP8), backward (dense, packed with a window,
bias, dropout) and split-KV decode."""

import os

import numpy as np
import pytest

import workloads
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()
    assert os.path.exists(fa.LIB_DEBUG_SYNC_PATH), "build with `build.py --all`"


def _dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    return t.cuda()


def _both(run):
    """run() under the optimised and the stage-synchronised library; the
    outputs (a tuple of tensors) must be equal bit for bit."""
    import torch
    import exact_io_aware_28_amd as fa
    a = run()
    torch.cuda.synchronize()
    with fa.using_library(fa.LIB_DEBUG_SYNC_PATH):
        b = run()
        torch.cuda.synchronize()
    assert len(a) == len(b)
    for i, (x, y) in enumerate(zip(a, b)):
        same = torch.equal(x.view(torch.uint8), y.view(torch.uint8)) if x.dtype.itemsize == 1 \
            else torch.equal(x.view(torch.int16 if x.dtype.itemsize == 2 else torch.int32),
                             y.view(torch.int16 if y.dtype.itemsize == 2 else torch.int32))
        assert same, f"output {i} differs between the two builds"


FWD_BWD = [
    # name, spec, bwd
    ("d128 causal GQA", dict(B=1, N=700, Hq=8, Hkv=2, d=128, causal=True, seed=901), True),
    ("d64 dense", dict(B=2, N=500, Hq=4, Hkv=4, d=64, causal=False, seed=902), True),
    ("packed window", dict(lengths=[1, 190, 64, 333, 77], Hq=4, Hkv=2, d=128, causal=True,
                           window=100, seed=903), True),
]


@pytest.mark.parametrize("name,spec,bwd", FWD_BWD, ids=[c[0] for c in FWD_BWD])
def test_forward_and_backward_same_bits(name, spec, bwd):
    import torch
    import exact_io_aware_28_amd as fa
    inp = workloads.make_inputs(dict(spec, bwd=bwd))
    say(f"[debug-sync] {name}")
    q, k, v, do = (_dev(inp[n]) for n in ("q", "k", "v", "do"))
    cu = inp.get("cu_seqlens")
    cu_t = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    kw = dict(scale=inp["scale"], causal=inp["causal"], window=inp["window"], cu_seqlens=cu_t,
              max_seqlen=inp["Nq"] if cu is not None else None)

    def run():
        o, lse = fa.fa_fwd(q, k, v, **kw)
        return (o, lse) + tuple(fa.fa_bwd(q, k, v, o, do, lse, **kw))
    _both(run)


def test_fp16_bias_dropout_same_bits():
    import torch
    import exact_io_aware_28_amd as fa
    inp = workloads.make_inputs(dict(B=1, N=300, Hq=4, Hkv=2, d=128, causal=True, seed=904,
                                     bwd=True))
    say("[debug-sync] fp16 forward+backward, bias forward+backward (causal; window only),"
        " dropout forward+backward")
    q, k, v, do = (_dev(inp[n]) for n in ("q", "k", "v", "do"))
    qh, kh, vh, doh = (_dev(inp[n], "f16") for n in ("q", "k", "v", "do"))
    bias = torch.from_numpy(np.random.default_rng(905).standard_normal((300, 300)).astype(
        np.float32)).cuda()

    def run():
        out = fa.fa_fwd_f16(qh, kh, vh, causal=True)
        gh = fa.fa_bwd_f16(qh, kh, vh, out[0], doh, out[1], causal=True)
        ob, lb = fa.fa_fwd_bias(q, k, v, bias, causal=True)
        gb = fa.fa_bwd_bias(q, k, v, bias, ob, do, lb, causal=True)
        ow, lw = fa.fa_fwd_bias(q, k, v, bias, window=70)
        od, ld = fa.fa_fwd_dropout(q, k, v, 0.2, 77, causal=True)
        gd = fa.fa_bwd_dropout(q, k, v, od, do, ld, 0.2, 77, causal=True)
        return (out + tuple(gh) + (ob, lb) + tuple(gb) + (ow, lw) + (od, ld) + tuple(gd))
    _both(run)


def test_decode_and_fp8_same_bits():
    import torch
    import exact_io_aware_28_amd as fa
    dec = workloads.make_decode_inputs(dict(B=4, Hq=8, Hkv=2, Nq=2, Nk=2048, d=128, Lmin=100,
                                            Lmax=2048, causal=True, seed=906))
    f8 = workloads.make_fp8_inputs(dict(B=1, N=700, Hq=8, Hkv=2, d=128, causal=True, seed=907))
    say("[debug-sync] split-KV decode, FP8 forward")
    dq, dk, dv = (_dev(dec[n]) for n in ("q", "k", "v"))
    lens = torch.from_numpy(dec["seqlens_k"]).cuda()
    d8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().view(torch.float8_e4m3fn)
    q8, k8, vt8 = d8(f8["q8"]), d8(f8["k8"]), d8(workloads.transpose_v8(f8["v8"]))
    sq, sk, sv = (torch.from_numpy(f8[n]).cuda() for n in ("sq", "sk", "sv"))

    def run():
        o, lse = fa.fa_decode(dq, dk, dv, causal=True, seqlens_k=lens)
        o8, l8 = fa.fa_fwd_fp8(q8, k8, vt8, sq, sk, sv, causal=True)
        return o, lse, o8, l8
    _both(run)
