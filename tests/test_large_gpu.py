"""GPU check at a size where every tensor spans more than 4 GiB.

Q, K, V, dO are [1, 131072, 136, 128] bf16 (4.6 GB each) with every head
holding the same single-head data.  Each head's result is computed by the
same code on the same values as a one-head call on that data, so the big
call must reproduce the one-head call bit for bit, head by head; the
one-head forward is also checked against the oracle on sampled rows.  The
staged tiles are bounded by 32-bit buffer descriptors, and a tile's
descriptor spanning everything from the tile to the end of the sequence
would exceed 4 GiB here.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_lse, check_o, say, sample_rows, to_dev, to_np

pytestmark = pytest.mark.gpu

N, H, D = 131072, 136, 128


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()  # fail loudly if the library is missing


def test_tensors_over_4gib_match_one_head():
    import torch
    import exact_io_aware_28_amd as fa
    say(f"[large] B=1 N={N} H={H} d={D} causal: {N * H * D * 2 / 1e9:.2f} GB per tensor")
    one = workloads.make_inputs(dict(B=1, N=N, Hq=1, Hkv=1, d=D, causal=True, seed=55,
                                     bwd=True))
    q1, k1, v1, do1 = (to_dev(one[n]) for n in ("q", "k", "v", "do"))
    big = []
    for t in (q1, k1, v1, do1):
        x = torch.empty((1, N, H, D), dtype=torch.bfloat16, device="cuda")
        x.copy_(t.expand(1, N, H, D))
        big.append(x)
    Q, K, V, dO = big

    o1, l1 = fa.fa_fwd(q1, k1, v1, causal=True)
    O, L = fa.fa_fwd(Q, K, V, causal=True)
    torch.cuda.synchronize()
    for h in (0, 77, H - 1):
        assert torch.equal(O[0, :, h], o1[0, :, 0]), ("O", h)
        assert torch.equal(L[0, h], l1[0, 0]), ("LSE", h)
    rows = sample_rows(N, count=12, seed=9)
    f = lambda n: one[n][0, :, 0].astype(np.float64)
    ro, rl = oracle.attn_fwd_rows(f("q"), f("k"), f("v"), rows, one["scale"], True)
    check_o(to_np(o1)[0, rows, 0], ro, "one head, sampled rows")
    check_lse(l1.cpu().numpy()[0, 0, rows].astype(np.float64), rl, "one head, sampled rows")

    g1 = fa.fa_bwd(q1, k1, v1, o1, do1, l1, causal=True)
    G = fa.fa_bwd(Q, K, V, O, dO, L, causal=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), G, g1):
        for h in (0, 77, H - 1):
            assert torch.equal(a[0, :, h], b[0, :, 0]), (name, h)
    say("  forward and backward of heads 0, 77, 135 equal the one-head call bit for bit")
