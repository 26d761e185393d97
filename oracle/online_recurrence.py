"""fp64 model of the block-by-block online-softmax recurrence.

TEST INFRASTRUCTURE ONLY.  This is NOT the parity reference (the plain
definition in attention.py is).  It exists to check the pages' exactness claim
on the CPU: carrying the running row maximum m, the running normaliser l and
the unnormalised output accumulator across key blocks, then dividing once at
the end, gives the same O and LSE as the plain definition.

Followed: llms.blog, "FlashAttention: How IO-Aware Tiling and Online Softmax
Solved Transformer Memory Bottlenecks", section "2. Online Softmax Reduction"
(the update of the block maximum, the rescaled normaliser, the rescaled output
accumulator, and the final division by l), and section "1. IO-Aware Tiling"
(query blocks of B_r rows visiting key/value blocks of B_c rows).

Reading taken where the page is silent: the state starts at m = -inf, l = 0,
O = 0; when the running maximum is still -inf (nothing visible yet) the
rescale factor is taken as 1 and the block contributes nothing.
"""

import numpy as np

from .attention import allowed_mask


def online_attention(q, k, v, scale, block_sizes, causal=False, window=0):
    """One head: q [nq,d], k/v [nk,d]; key blocks of the given sizes.

    Returns (O, LSE) computed with the running (m, l, O) state.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, nk = len(q), len(k)
    ok = allowed_mask(nq, nk, causal, window)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    start = 0
    for bc in block_sizes:
        stop = min(nk, start + bc)
        if start >= stop:
            break
        s = scale * (q @ k[start:stop].T)
        s = np.where(ok[:, start:stop], s, -np.inf)
        m_blk = s.max(axis=1)
        m_new = np.maximum(m, m_blk)
        live = ~np.isneginf(m_new)
        shift = np.where(live, m_new, 0.0)
        alpha = np.where(live, np.exp(np.where(live, m - shift, 0.0)), 1.0)
        e = np.exp(s - shift[:, None])
        l = alpha * l + e.sum(axis=1)
        acc = alpha[:, None] * acc + e @ v[start:stop]
        m = m_new
        start = stop
    assert start >= nk, "block sizes must cover every key"
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, acc / l[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return o, lse
