"""Plain fp64 definition of exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity pins for every
function here live in tests/test_oracle.py; no function is "parity unpinned".

Sources (the pages this follows):
  [llms]  llms.blog, "FlashAttention: How IO-Aware Tiling and Online Softmax
          Solved Transformer Memory Bottlenecks"
  [tok]   tokrepo.com, "Flash Attention - Fast Memory-Efficient Exact Attention"
  [klay]  klaylearn.com glossary, "flash-attention"
  [inf]   inferensys.com glossary, "FlashAttention"

Definitions used:
  * S = scale * Q K^T, P = softmax(S) row-wise, O = P V
      ([llms] "Naive Attention Execution Profile"; the scale comes from the
      "scaled dot-product attention" wording in [klay], first question).
  * softmax with the row maximum subtracted
      ([llms] "2. Online Softmax Reduction", the softmax formula).
  * masking (causal, sliding window, packed variable-length batches, GQA/MQA
      head sharing) are the features listed in [tok] "What Flash Attention
      Does" and "Key Features".  The pages fix no convention for them; the
      readings taken here:
        - a masked score is -inf (additive mask in {0, -inf});
        - causal is aligned bottom-right: query i may see key j iff
          j <= i + (Nk - Nq);
        - a window W > 0 lets query i see at most W keys counting itself:
          (i + Nk - Nq) - j < W;  W <= 0 means no window;
        - query head h reads KV head h // (Hq / Hkv) (contiguous groups);
        - in a packed batch a query only sees keys of its own sequence;
        - a row with no visible key has O = 0 and LSE = -inf;
        - a custom mask ([tok] "Key Features" lists custom attention masks)
          is an additive bias B added to the scaled scores before the
          softmax, S = scale * Q K^T + B, with -inf entries hiding a key;
          it is a constant of the problem, so it has no gradient here, and
          it combines with the causal and window masks;
        - dropout (fused with the rest in [inf]'s fused-kernel paragraph)
          acts on the normalised probabilities: O = (P * Z / (1 - p)) V with Z the
          keep-mask of oracle/philox.py; LSE is that of the undropped P.
  * the saved row statistic is the natural-log logsumexp
      LSE_i = m_i + ln(l_i) = ln(sum_j exp(S_ij))
      ([tok] "Architecture Overview" names logsumexp; [llms] "3. Recomputation
      in the Backward Pass" names the pair (m, l), which LSE summarises).
  * backward: the pages only say the gradients are evaluated from recomputed
      scores ([llms] "3. Recomputation in the Backward Pass"); the formulas are
      the textbook chain rule through softmax:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
        dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
      with dK, dV summed over the query heads that share a KV head.

Layouts (token-major, d innermost):
  dense : Q, O [B, Nq, Hq, d]; K, V [B, Nk, Hkv, d]; LSE [B, Hq, Nq]
  packed: Q, O [T, Hq, d];     K, V [T, Hkv, d];     LSE [Hq, T]
          with cu_seqlens the int prefix sums of the B sequence lengths.
"""

import numpy as np

from .philox import keep_mask, keep_scale


def kv_head_of(h, hq, hkv):
    """KV head read by query head h: contiguous groups of Hq/Hkv query heads."""
    return h // (hq // hkv)


def allowed_mask(nq, nk, causal, window):
    """Boolean [nq, nk]: may query i see key j (conventions in module doc)."""
    i = np.arange(nq)[:, None] + (nk - nq)
    j = np.arange(nk)[None, :]
    ok = np.ones((nq, nk), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def _rows_allowed(rows, nq, nk, causal, window):
    """allowed_mask restricted to the given query rows."""
    i = np.asarray(rows)[:, None] + (nk - nq)
    j = np.arange(nk)[None, :]
    ok = np.ones((len(rows), nk), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def _softmax_rows(s):
    """Row softmax with the row max subtracted; returns (P, LSE).

    Fully masked rows (all -inf) give P = 0 and LSE = -inf.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l[:, None] > 0, e / l[:, None], 0.0)
        lse = m_safe + np.log(l)
    # keep NaN rows NaN (NaN inputs propagate)
    p = np.where(np.isnan(l)[:, None], np.nan, p)
    return p, lse


def _dropped(p, keep, p_drop):
    """P * Z / (1 - p_drop): the probabilities that multiply V, with p_drop
    taken as the exact drop probability of the mask (p rounded down to a
    multiple of 2^-16, oracle/philox.py)."""
    if keep is None:
        return p
    return np.where(keep, p * keep_scale(p_drop), 0.0)


def _head_fwd(q, k, v, scale, ok, bias=None, keep=None, p_drop=0.0):
    """One (sequence, head): q [nq,d], k/v [nk,d] fp64 -> O, LSE, P.

    bias: None or [nq, nk], added to the scaled scores; keep: None or the
    boolean dropout keep-mask [nq, nk] (P is returned undropped)."""
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + np.asarray(bias, np.float64)
    s = np.where(ok, s, -np.inf)
    p, lse = _softmax_rows(s)
    return _dropped(p, keep, p_drop) @ v, lse, p


def _keep(dropout_p, seed, b, h, rows, nk):
    if dropout_p == 0.0:
        return None
    return keep_mask(seed, b, h, rows, nk, dropout_p)


def sequence_spans(B, N, cu_seqlens):
    """[(start, length)] of each sequence: dense rows of N, or cu_seqlens."""
    if cu_seqlens is None:
        return [(b * N, N) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[s]), int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)]


def _as_packed(x):
    """View dense [B, N, H, d] as packed [B*N, H, d]; packed stays as is."""
    x = np.asarray(x, dtype=np.float64)
    return x.reshape(-1, x.shape[-2], x.shape[-1]) if x.ndim == 4 else x


def _bias_of(bias, B, hq, nq, nk):
    """The bias as a read-only [B, Hq, Nq, Nk] view (numpy broadcasting)."""
    if bias is None:
        return None
    return np.broadcast_to(bias, (B, hq, nq, nk))


def attn_fwd(q, k, v, scale, causal=False, window=0, cu_seqlens=None, bias=None,
             dropout_p=0.0, seed=0):
    """Exact attention forward.  Returns (O, LSE) in the module's layouts.

    bias: None, or (dense batches only) an array that broadcasts to
    [B, Hq, Nq, Nk], added to the scaled scores.  dropout_p, seed: dropout
    on the probabilities with the Philox keep-mask (oracle/philox.py)."""
    dense = cu_seqlens is None
    if bias is not None and not dense:
        raise ValueError("a bias is defined for dense batches only")
    if dense:
        B, nq, hq, d = q.shape
        nk, hkv = k.shape[1], k.shape[2]
    else:
        hq, hkv = q.shape[1], k.shape[1]
    qp, kp, vp = _as_packed(q), _as_packed(k), _as_packed(v)
    o = np.zeros(qp.shape, dtype=np.float64)
    if dense:
        lse = np.full((B, hq, nq), -np.inf)
        qspans = sequence_spans(B, nq, None)
        kspans = sequence_spans(B, nk, None)
    else:
        lse = np.full((hq, qp.shape[0]), -np.inf)
        qspans = kspans = sequence_spans(None, None, cu_seqlens)
    bb = _bias_of(bias, B, hq, nq, nk) if dense else None
    for s, ((q0, lq), (k0, lk)) in enumerate(zip(qspans, kspans)):
        if lq == 0:
            continue
        ok = allowed_mask(lq, lk, causal, window)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            oh, lh, _ = _head_fwd(qp[q0:q0 + lq, h], kp[k0:k0 + lk, g],
                                  vp[k0:k0 + lk, g], scale, ok,
                                  None if bb is None else bb[s, h],
                                  _keep(dropout_p, seed, s, h, np.arange(lq), lk), dropout_p)
            o[q0:q0 + lq, h] = oh
            if dense:
                lse[s, h] = lh
            else:
                lse[h, q0:q0 + lq] = lh
    return o.reshape(np.shape(q)), lse


def probabilities(q, k, scale, causal=False, window=0):
    """P for one head: q [nq,d], k [nk,d] -> [nq, nk] (used by pins)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    s = np.where(allowed_mask(len(q), len(k), causal, window),
                 scale * (q @ k.T), -np.inf)
    return _softmax_rows(s)[0]


def attn_fwd_rows(q_h, k_g, v_g, rows, scale, causal=False, window=0, bias=None,
                  dropout_p=0.0, seed=0, bh=(0, 0)):
    """O and LSE of selected query rows of one (sequence, head).

    q_h [nq,d], k_g/v_g [nk,d]; rows: indices into q_h; bias: None or this
    head's [nq, nk] bias; dropout_p, seed and bh = (sequence, query head)
    select the dropout mask.  Each row is the plain definition over the
    whole key row, so any subset of rows can be checked at any length.
    """
    q_h = np.asarray(q_h, np.float64)
    k_g = np.asarray(k_g, np.float64)
    v_g = np.asarray(v_g, np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    ok = _rows_allowed(rows, len(q_h), len(k_g), causal, window)
    o, lse, _ = _head_fwd(q_h[rows], k_g, v_g, scale, ok,
                          None if bias is None else np.asarray(bias)[rows],
                          _keep(dropout_p, seed, bh[0], bh[1], rows, len(k_g)), dropout_p)
    return o, lse


def _head_bwd(q, k, v, do, scale, ok, bias=None, keep=None, p_drop=0.0):
    """One (sequence, head) backward from the definition: returns dq, dk, dv.
    With dropout, O = Pd V with Pd = P * Z / (1 - p): dV = Pd^T dO and the
    gradient reaching P is (dO V^T) * Z / (1 - p)."""
    o, _, p = _head_fwd(q, k, v, scale, ok, bias, keep, p_drop)
    dv = _dropped(p, keep, p_drop).T @ do
    dp = _dropped(do @ v.T, keep, p_drop)
    dvec = (do * o).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attn_bwd(q, k, v, do, scale, causal=False, window=0, cu_seqlens=None, bias=None,
             dropout_p=0.0, seed=0):
    """Exact gradients (dQ, dK, dV) of sum(O * dO), same layouts as Q, K, V
    (bias and dropout as in attn_fwd; the bias and the mask are constants)."""
    dense = cu_seqlens is None
    if bias is not None and not dense:
        raise ValueError("a bias is defined for dense batches only")
    if dense:
        B, nq, hq, d = q.shape
        nk, hkv = k.shape[1], k.shape[2]
        qspans = sequence_spans(B, nq, None)
        kspans = sequence_spans(B, nk, None)
    else:
        hq, hkv = q.shape[1], k.shape[1]
        qspans = kspans = sequence_spans(None, None, cu_seqlens)
    qp, kp, vp, dop = _as_packed(q), _as_packed(k), _as_packed(v), _as_packed(do)
    dq = np.zeros(qp.shape)
    dk = np.zeros(kp.shape)
    dv = np.zeros(vp.shape)
    bb = _bias_of(bias, B, hq, nq, nk) if dense else None
    for s, ((q0, lq), (k0, lk)) in enumerate(zip(qspans, kspans)):
        if lq == 0:
            continue
        ok = allowed_mask(lq, lk, causal, window)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            a, b, c = _head_bwd(qp[q0:q0 + lq, h], kp[k0:k0 + lk, g],
                                vp[k0:k0 + lk, g], dop[q0:q0 + lq, h], scale, ok,
                                None if bb is None else bb[s, h],
                                _keep(dropout_p, seed, s, h, np.arange(lq), lk), dropout_p)
            dq[q0:q0 + lq, h] = a
            dk[k0:k0 + lk, g] += b
            dv[k0:k0 + lk, g] += c
    return dq.reshape(np.shape(q)), dk.reshape(np.shape(k)), dv.reshape(np.shape(v))


def attn_bwd_sampled(q, k, v, do, scale, causal, window, b, g, q_rows, k_rows,
                     chunk=2048, bias=None, dropout_p=0.0, seed=0):
    """Gradients of one dense batch entry b and KV head g, at sampled rows.

    Returns (dq [len(q_rows), G, d] for the G query heads of KV head g,
             dk [len(k_rows), d], dv [len(k_rows), d]).

    Same definitions as attn_bwd (bias as there); the full rows of P are rebuilt chunk by
    chunk of query rows (each chunk a full-row softmax, no running state) so
    that long sequences fit in host memory.
    """
    q = np.asarray(q)
    nq, hq, d = q.shape[1], q.shape[2], q.shape[3]
    nk, hkv = k.shape[1], k.shape[2]
    G = hq // hkv
    kb = np.asarray(k[b, :, g], np.float64)
    vb = np.asarray(v[b, :, g], np.float64)
    q_rows = np.asarray(q_rows, np.int64)
    k_rows = np.asarray(k_rows, np.int64)
    dq = np.zeros((len(q_rows), G, d))
    dk = np.zeros((len(k_rows), d))
    dv = np.zeros((len(k_rows), d))
    bb = _bias_of(bias, q.shape[0], hq, nq, nk)
    for gi in range(G):
        h = g * G + gi
        qh = np.asarray(q[b, :, h], np.float64)
        doh = np.asarray(do[b, :, h], np.float64)
        bh = None if bb is None else bb[b, h]
        # dQ rows: each needs only its own full row of P and dP.
        ok = _rows_allowed(q_rows, nq, nk, causal, window)
        keep_r = _keep(dropout_p, seed, b, h, q_rows, nk)
        o_r, _, p_r = _head_fwd(qh[q_rows], kb, vb, scale, ok,
                                None if bh is None else bh[q_rows], keep_r, dropout_p)
        dp_r = _dropped(doh[q_rows] @ vb.T, keep_r, dropout_p)
        dvec_r = (doh[q_rows] * o_r).sum(axis=1)
        dq[:, gi] = scale * ((p_r * (dp_r - dvec_r[:, None])) @ kb)
        # dK/dV rows: need columns k_rows of P and dS over every query row.
        for c0 in range(0, nq, chunk):
            rows = np.arange(c0, min(nq, c0 + chunk))
            okc = _rows_allowed(rows, nq, nk, causal, window)
            keep_c = _keep(dropout_p, seed, b, h, rows, nk)
            o_c, _, p_c = _head_fwd(qh[rows], kb, vb, scale, okc,
                                    None if bh is None else bh[rows], keep_c, dropout_p)
            dvec_c = (doh[rows] * o_c).sum(axis=1)
            kj = None if keep_c is None else keep_c[:, k_rows]
            pj = p_c[:, k_rows]
            dpj = _dropped(doh[rows] @ vb[k_rows].T, kj, dropout_p)
            dsj = pj * (dpj - dvec_c[:, None])
            dv += _dropped(pj, kj, dropout_p).T @ doh[rows]
            dk += scale * (dsj.T @ qh[rows])
    return dq, dk, dv
