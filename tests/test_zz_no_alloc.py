"""GPU test of the allocation-free decode entry point (fa_decode_noalloc):
called through the C ABI, it must give the bits of fa_decode (same kernels,
same split count, the partials in the library's static device scratch
instead of a caller workspace) on two calls in a row, the second smaller
than the first, so that what the first call left in the scratch cannot leak
into the second."""

import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_lse, check_o, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()  # fail loudly if the library is missing


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc_c_call(q, k, v, o, lse, lens, scale, causal, window, splits):
    """fa_decode_noalloc straight through ctypes (plain pointers and sizes)."""
    import torch
    import exact_io_aware_28_amd as fa
    B, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    return fa.lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, hq,
                                      hkv, nq, nk, d, float(scale), int(causal), int(window),
                                      _ptr(lens), int(splits),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _case(inp, window, expect_splits=None):
    import torch
    import exact_io_aware_28_amd as fa
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    lens = torch.from_numpy(np.asarray(inp["seqlens_k"], np.int32)).cuda()
    B, nq, hq, d = q.shape
    hkv, nk = k.shape[2], k.shape[1]
    default = fa.fa_decode_num_splits(B, hq, hkv, nq, nk)
    splits = min(default, fa.fa_decode_noalloc_max_splits(B, hq, nq, d))
    if expect_splits is not None:
        assert splits == expect_splits
    say(f"[no-alloc decode] B={B} Nq={nq} Hq={hq} Hkv={hkv} Nk={nk} d={d} window={window} "
        f"splits={splits}")
    o_ref, l_ref = fa.fa_decode(q, k, v, scale=inp["scale"], causal=True, window=window,
                                seqlens_k=lens, num_splits=splits)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
    st = _noalloc_c_call(q, k, v, o, lse, lens, inp["scale"], True, window, 0)
    torch.cuda.synchronize()
    assert st == fa.FA_OK, fa.fa_status_string(st)
    assert torch.equal(o, o_ref), "O differs from fa_decode"
    assert torch.equal(lse, l_ref), "LSE differs from fa_decode"
    # and the oracle's bar on a few sequences, rows at their cache end
    o_np, l_np = to_np(o), lse.cpu().numpy().astype(np.float64)
    outs, refs, lerr = [], [], 0.0
    for b in range(min(B, 3)):
        L = int(inp["seqlens_k"][b])
        for h in range(0, hq, max(1, hq // 4)):
            g = h // (hq // hkv)
            ro, rl = oracle.attn_fwd_rows(inp["q"][b, :, h], inp["k"][b, :L, g],
                                          inp["v"][b, :L, g], np.arange(nq), inp["scale"],
                                          True, window)
            outs.append(o_np[b, :, h])
            refs.append(ro)
            lerr = max(lerr, float(np.abs(l_np[b, h] - rl).max()))
    check_o(np.concatenate(outs), np.concatenate(refs), "no-alloc decode")
    say(f"  LSE max|err|={lerr:.3e}")
    assert lerr <= 1e-3


def test_noalloc_decode_matches_fa_decode_on_two_calls():
    # first: the single-token decode workload (16 sequences, 1024..8192 of
    # 8192 cached keys, Hq 32 / Hkv 8, d 128); second: a smaller chunk of four
    # query rows per sequence over 1000-key caches at d 64 with a window
    big = workloads.make_decode_inputs("decode_kv_cache")
    _case(big, 0, expect_splits=12)
    small = workloads.make_decode_inputs(dict(B=3, Hq=8, Hkv=2, Nq=4, Nk=1000, d=64,
                                              Lmin=17, Lmax=1000, causal=True, window=300,
                                              seed=61))
    _case(small, 300)


def test_noalloc_decode_refuses_oversize_request_before_launch():
    import torch
    import exact_io_aware_28_amd as fa
    # 64 sequences x 16 rows x 64 heads x 128 floats = 32 MiB of partial
    # outputs for one split, plus LSEs: more than the static scratch
    q = torch.zeros(64, 16, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 64, 8, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(64, 64, 16, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_noalloc(q, k, k, o, lse, causal=True)
    assert e.value.status == fa.FA_ERR_TOO_LARGE
