"""GPU parity of the split-KV path (fa_decode) against the fp64 oracle.

Each sequence b attends with its Nq query rows to the first seqlens_k[b]
keys of its cache (bottom-right causal alignment, optional window); the
oracle is attn_fwd on exactly those rows and keys.  Cases cover one and
several query rows, GQA groups that fill one and several 32-row blocks,
ragged cache lengths (including 0, 1 and lengths that are not multiples of
the 32-key tile), more splits than tiles, a window, no mask, d = 64 and 128,
and the full decode workload.  Tolerances as the forward: O max|err| <=
2e-2 and mean|err| <= 2e-3, LSE |err| <= 1e-3 (tests/gpu_util.py).
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_lse, check_o, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_28_amd as fa
    fa.lib()  # fail loudly if the library is missing


def _run(inp, num_splits=None):
    import torch
    import exact_io_aware_28_amd as fa
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    lens = torch.from_numpy(np.asarray(inp["seqlens_k"], np.int32)).cuda()
    o, lse = fa.fa_decode(q, k, v, scale=inp["scale"], causal=inp["causal"],
                          window=inp["window"], seqlens_k=lens, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def _reference(inp, b):
    """fp64 oracle for sequence b: its query rows against its used keys."""
    L = int(inp["seqlens_k"][b])
    nq, hq, d = inp["q"].shape[1:]
    if L == 0:
        return np.zeros((nq, hq, d)), np.full((hq, nq), -np.inf)
    o, lse = oracle.attn_fwd(inp["q"][b:b + 1].astype(np.float64),
                             inp["k"][b:b + 1, :L].astype(np.float64),
                             inp["v"][b:b + 1, :L].astype(np.float64),
                             inp["scale"], inp["causal"], inp["window"])
    return o[0], lse[0]


def _check(inp, what, num_splits=None, sequences=None):
    say(f"[decode] {what} splits={num_splits}")
    o, lse = _run(inp, num_splits)
    seqs = list(range(inp["B"])) if sequences is None else list(sequences)
    refs = [_reference(inp, b) for b in seqs]
    o_ref = np.stack([r[0] for r in refs])
    l_ref = np.stack([r[1] for r in refs])
    idx = np.array(seqs)
    check_o(o[idx], o_ref, what)
    check_lse(lse[idx], l_ref, what)


def _inputs(B, Hq, Hkv, Nq, Nk, d, lengths, causal=True, window=0, seed=11):
    return workloads.make_decode_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d,
                                             lengths=lengths, causal=causal, window=window,
                                             seed=seed))


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, lengths, causal, window, splits
    (4, 8, 2, 1, 300, 128, [300, 1, 37, 250], True, 0, None),
    (2, 32, 8, 1, 4096, 128, [4096, 4095], True, 0, None),
    (3, 4, 4, 5, 1000, 64, [1000, 700, 3], True, 0, 7),     # rows that see no key
    (2, 16, 2, 3, 2048, 128, [2048, 1500], True, 512, None),  # window
    (2, 8, 8, 2, 640, 64, [640, 0], False, 0, 3),            # no mask, empty cache
    (1, 32, 4, 9, 777, 128, [777], True, 0, 1),              # 72 rows: three row blocks
    (2, 8, 2, 1, 300, 128, [300, 64], True, 0, 50),          # more splits than tiles
    (3, 8, 1, 4, 520, 64, [520, 31, 33], True, 100, 4),      # MQA, window, ragged ends
    (2, 8, 2, 2, 5000, 128, [5000, 3100], True, 0, 130),    # > 64 splits: chunked merge
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_decode_small(case):
    B, Hq, Hkv, Nq, Nk, d, lengths, causal, window, splits = case
    inp = _inputs(B, Hq, Hkv, Nq, Nk, d, lengths, causal, window, seed=11 + len(lengths))
    _check(inp, f"B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} L={lengths} "
                f"causal={causal} window={window}", splits)


def test_decode_split_count_does_not_change_the_result():
    """1, 2, 5 and the default number of splits agree with each other within
    rounding (the merge through the logsumexps is exact up to fp32)."""
    inp = _inputs(2, 8, 2, 2, 1500, 128, [1500, 999], seed=21)
    outs = [_run(inp, s) for s in (1, 2, 5, None)]
    for o, lse in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 1e-2
        assert np.abs(lse - outs[0][1]).max() <= 1e-4


def test_decode_matches_dense_forward():
    """With every cache full, fa_decode equals fa_fwd with Nq query rows and
    Nk keys (same bottom-right causal alignment)."""
    import torch
    import exact_io_aware_28_amd as fa
    inp = _inputs(2, 16, 4, 4, 1024, 128, [1024, 1024], seed=31)
    o, lse = _run(inp)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    o2, lse2 = fa.fa_fwd(q, k, v, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    assert np.abs(o - to_np(o2)).max() <= 1e-2
    assert np.abs(lse - lse2.cpu().numpy()).max() <= 1e-4


def test_decode_workload_sampled():
    """The full decode workload (16 sequences, 1024..8192 cached keys, GQA
    32/8, d=128) in the launch configuration the bench times, checked on four
    of its sequences."""
    inp = workloads.make_decode_inputs("decode_kv_cache")
    _check(inp, "decode_kv_cache", None, sequences=[0, 5, 10, 15])
