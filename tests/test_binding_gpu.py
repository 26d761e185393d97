"""GPU tests of the binding's stream handling and device checks.

Work launched on a side stream must give the bits of the same work on the
current stream, with the binding's own buffers (outputs, workspace) made on
the side stream, so that allocations on the current stream made while that
work may still run cannot take their memory.  Tensors on the host next to
device tensors are refused before any launch."""

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


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def test_side_stream_gives_the_current_stream_bits():
    import torch
    import exact_io_aware_28_amd as fa
    inp = workloads.make_inputs(dict(B=2, N=700, Hq=8, Hkv=2, d=128, causal=True, seed=81,
                                     bwd=True))
    q, k, v, do = (_dev(inp[n]) for n in ("q", "k", "v", "do"))
    dec = workloads.make_decode_inputs(dict(B=4, Hq=8, Hkv=2, Nq=1, Nk=2048, d=128, Lmin=100,
                                            Lmax=2048, causal=True, seed=82))
    dq_, dk_, dv_ = (_dev(dec[n]) for n in ("q", "k", "v"))
    lens = torch.from_numpy(dec["seqlens_k"]).cuda()
    say("[streams] B=2 N=700 Hq=8 Hkv=2 d=128 causal fwd+bwd, decode B=4 Nk=2048")
    o0, l0 = fa.fa_fwd(q, k, v, causal=True)
    g0 = fa.fa_bwd(q, k, v, o0, do, l0, causal=True)
    d0 = fa.fa_decode(dq_, dk_, dv_, causal=True, seqlens_k=lens)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        o1, l1 = fa.fa_fwd(q, k, v, causal=True, stream=side)
        g1 = fa.fa_bwd(q, k, v, o1, do, l1, causal=True, stream=side)
        d1 = fa.fa_decode(dq_, dk_, dv_, causal=True, seqlens_k=lens, stream=side)
        # allocations and writes on the current stream while the side stream runs
        junk = [torch.full((1 << 20,), float(rep), device="cuda") for _ in range(16)]
        del junk
        side.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1), rep
        for a, b in zip(g0, g1):
            assert torch.equal(a, b), rep
        assert torch.equal(d0[0], d1[0]) and torch.equal(d0[1], d1[1]), rep


def test_host_tensors_next_to_device_tensors_are_refused():
    import torch
    import exact_io_aware_28_amd as fa
    T, H, d = 96, 2, 64
    q = torch.zeros(T, H, d, dtype=torch.bfloat16, device="cuda")
    cu_host = torch.tensor([0, 40, 96], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens must be a device tensor"):
        fa.fa_fwd(q, q, q, cu_seqlens=cu_host, max_seqlen=56)
    qd = torch.zeros(2, 1, 4, 64, dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros(2, 128, 2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="seqlens_k must be a device tensor"):
        fa.fa_decode(qd, kd, kd, seqlens_k=torch.tensor([5, 9], dtype=torch.int32))
    with pytest.raises(ValueError, match="out must be a device tensor"):
        fa.fa_fwd(qd, kd, kd, out=torch.empty(2, 1, 4, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="k must be a device tensor"):
        fa.fa_fwd(qd, kd.cpu(), kd)
