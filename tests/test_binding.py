"""CPU tests of the Python binding's argument checks: every malformed
argument is refused with an exception before anything is allocated or
launched.  The host-visible facts (dtype, shape, contiguity, sizes) are
checked for all arguments before the device placement, so these run with
CPU tensors; a well-formed call made of CPU tensors is refused because they
are not device tensors."""

import os

import pytest
import torch

import exact_io_aware_28_amd as fa

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH),
                                reason="library not built")

BF = torch.bfloat16


def dense(B=2, N=64, hq=4, hkv=2, d=64, dtype=BF):
    q = torch.zeros(B, N, hq, d, dtype=dtype)
    k = torch.zeros(B, N, hkv, d, dtype=dtype)
    return q, k, k.clone()


def packed(T=100, hq=4, hkv=2, d=64):
    q = torch.zeros(T, hq, d, dtype=BF)
    k = torch.zeros(T, hkv, d, dtype=BF)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32)
    return q, k, k.clone(), cu


def raises(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


# ------------------------------------------------------------------ forward
def test_forward_shape_and_dtype_checks():
    q, k, v = dense()
    raises(ValueError, "same shape", fa.fa_fwd, q, k, v[:, :, :1].contiguous())
    raises(ValueError, "batch", fa.fa_fwd, q, k[:1].contiguous(), v[:1].contiguous())
    raises(ValueError, "head dimension", fa.fa_fwd, q, k[..., :32].contiguous(),
           v[..., :32].contiguous())
    raises(TypeError, "k must be", fa.fa_fwd, q, k.float(), v)
    raises(TypeError, "must be torch.float16", fa.fa_fwd_f16, q, k, v)
    raises(ValueError, "contiguous", fa.fa_fwd, q.transpose(1, 2), k, v)
    raises(ValueError, "dense q/k/v", fa.fa_fwd, q[0], k[0], v[0])
    raises(TypeError, "torch.Tensor", fa.fa_fwd, [1], k, v)


def test_forward_checks_supplied_outputs():
    q, k, v = dense()
    raises(ValueError, "out must have shape", fa.fa_fwd, q, k, v, out=torch.empty(2, 64, 4, 32,
                                                                               dtype=BF))
    raises(TypeError, "out must be", fa.fa_fwd, q, k, v, out=torch.empty_like(q, dtype=torch.half))
    raises(ValueError, "lse must have shape", fa.fa_fwd, q, k, v,
           lse=torch.empty(2, 64, 4, dtype=torch.float32))
    raises(TypeError, "lse must be", fa.fa_fwd, q, k, v,
           lse=torch.empty(2, 4, 64, dtype=torch.float64))
    raises(ValueError, "out must be contiguous", fa.fa_fwd, q, k, v,
           out=torch.empty(2, 4, 64, 64, dtype=BF).transpose(1, 2))


def test_packed_forward_checks_cu_seqlens():
    q, k, v, cu = packed()
    raises(TypeError, "cu_seqlens must be torch.int32", fa.fa_fwd, q, k, v,
           cu_seqlens=cu.long(), max_seqlen=60)
    raises(ValueError, "1-D", fa.fa_fwd, q, k, v, cu_seqlens=cu[:1].contiguous(), max_seqlen=60)
    raises(ValueError, "1-D", fa.fa_fwd, q, k, v, cu_seqlens=cu.view(1, 3), max_seqlen=60)
    raises(ValueError, "max_seqlen", fa.fa_fwd, q, k, v, cu_seqlens=cu)
    raises(ValueError, "tokens", fa.fa_fwd, q, k[:50].contiguous(), v[:50].contiguous(), cu_seqlens=cu, max_seqlen=60)
    raises(ValueError, "packed q/k/v", fa.fa_fwd, q[None], k[None], v[None], cu_seqlens=cu,
           max_seqlen=60)
    # LSE of a packed batch is [Hq, T]
    raises(ValueError, "lse must have shape", fa.fa_fwd, q, k, v, cu_seqlens=cu, max_seqlen=60,
           lse=torch.empty(2, 4, 60))


def test_well_formed_host_tensors_are_refused_as_not_on_the_device():
    q, k, v = dense()
    raises(ValueError, "q must be a device tensor", fa.fa_fwd, q, k, v)
    q, k, v, cu = packed()
    raises(ValueError, "device tensor", fa.fa_fwd, q, k, v, cu_seqlens=cu, max_seqlen=60)


def test_dropout_forward_uses_the_same_checks():
    q, k, v = dense()
    raises(ValueError, "same shape", fa.fa_fwd_dropout, q, k, v[:, :8].contiguous(), 0.1, 1)
    raises(ValueError, "device tensor", fa.fa_fwd_dropout, q, k, v, 0.1, 1)


# ------------------------------------------------------------------ backward
def bwd_args():
    q, k, v = dense()
    o = torch.zeros_like(q)
    do = torch.zeros_like(q)
    lse = torch.zeros(2, 4, 64)
    return q, k, v, o, do, lse


@pytest.mark.parametrize("fn", ["fa_bwd", "fa_bwd_dropout", "fa_bwd_f16"])
def test_backward_checks(fn):
    q, k, v, o, do, lse = bwd_args()
    if fn == "fa_bwd_f16":
        q, k, v, o, do = (t.half() for t in (q, k, v, o, do))
    extra = (0.1, 5) if fn == "fa_bwd_dropout" else ()
    f = getattr(fa, fn)
    raises(ValueError, "o must have shape", f, q, k, v, o[:, :32].contiguous(), do, lse, *extra)
    raises(ValueError, "dout must have shape", f, q, k, v, o, do[:1].contiguous(), lse, *extra)
    raises(TypeError, "dout must be", f, q, k, v, o, do.float(), lse, *extra)
    raises(ValueError, "lse must have shape", f, q, k, v, o, do, lse[:, :2].contiguous(), *extra)
    raises(ValueError, "dq must have shape", f, q, k, v, o, do, lse, *extra, dq=torch.empty_like(k))
    raises(ValueError, "dk must have shape", f, q, k, v, o, do, lse, *extra, dk=torch.empty_like(q))
    raises(TypeError, "dv must be", f, q, k, v, o, do, lse, *extra,
           dv=torch.empty_like(v, dtype=torch.float32))
    raises(ValueError, "workspace holds", f, q, k, v, o, do, lse, *extra,
           workspace=torch.empty(8, dtype=torch.uint8))
    raises(ValueError, "same shape", f, q, k, v[:, :, :1].contiguous(), o, do, lse, *extra)
    raises(ValueError, "device tensor", f, q, k, v, o, do, lse, *extra)


def test_f16_backward_wants_half_everywhere():
    q, k, v, o, do, lse = bwd_args()
    raises(TypeError, "must be torch.float16", fa.fa_bwd_f16, q, k, v, o, do, lse)
    h = [t.half() for t in (q, k, v, o, do)]
    raises(TypeError, "dout must be torch.float16", fa.fa_bwd_f16, *h[:4], do, lse)
    raises(TypeError, "dq must be torch.float16", fa.fa_bwd_f16, *h, lse,
           dq=torch.empty_like(q))


def test_backward_packed_checks_cu_seqlens():
    q, k, v, cu = packed()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(4, 100)
    raises(TypeError, "cu_seqlens must be torch.int32", fa.fa_bwd, q, k, v, o, do, lse,
           cu_seqlens=cu.long(), max_seqlen=60)
    raises(ValueError, "lse must have shape", fa.fa_bwd, q, k, v, o, do, lse[:, :50].contiguous(),
           cu_seqlens=cu, max_seqlen=60)


# ------------------------------------------------------------------ bias
def test_bias_checks():
    q, k, v, o, do, lse = bwd_args()
    raises(TypeError, "bias must be a float32", fa.fa_fwd_bias, q, k, v, torch.zeros(64, 64,
                                                                                   dtype=BF))
    raises(ValueError, "does not broadcast", fa.fa_fwd_bias, q, k, v, torch.zeros(3, 64, 64))
    raises(ValueError, "cannot broadcast", fa.fa_fwd_bias, q, k, v, torch.zeros(64, 1))
    raises(ValueError, "at most|broadcast to", fa.fa_fwd_bias, q, k, v, torch.zeros(1, 1, 1, 64, 64))
    raises(ValueError, "does not broadcast", fa.fa_bwd_bias, q, k, v, torch.zeros(5, 64), o, do, lse)
    raises(ValueError, "device tensor", fa.fa_fwd_bias, q, k, v, torch.zeros(64, 64))


# ------------------------------------------------------------------ decode
def test_decode_checks():
    q = torch.zeros(3, 1, 8, 128, dtype=BF)
    k = torch.zeros(3, 256, 2, 128, dtype=BF)
    v = k.clone()
    lens = torch.tensor([10, 20, 256], dtype=torch.int32)
    raises(TypeError, "seqlens_k must be torch.int32", fa.fa_decode, q, k, v,
           seqlens_k=lens.long())
    raises(ValueError, "seqlens_k must have shape", fa.fa_decode, q, k, v, seqlens_k=lens[:2].contiguous())
    raises(ValueError, "workspace holds", fa.fa_decode, q, k, v, num_splits=4,
           workspace=torch.empty(16, dtype=torch.uint8))
    raises(ValueError, "out must have shape", fa.fa_decode, q, k, v, out=torch.empty_like(k))
    raises(ValueError, "same shape", fa.fa_decode, q, k, v[:, :100].contiguous())
    raises(ValueError, "device tensor", fa.fa_decode, q, k, v, seqlens_k=lens)
