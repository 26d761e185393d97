"""Python binding of libfa_mi355x (exact IO-aware attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the shared library.  PyTorch supplies device memory and the
stream; nothing here computes attention.  If the library is not built the
import still succeeds but every call raises.

Functions mirror the C ABI in include/fa_mi355x.h:
    fa_fwd(q, k, v, scale, causal, window, cu_seqlens, max_seqlen) -> (o, lse)
    fa_fwd_f16(...)  same, fp16 tensors
    fa_fwd_f32(...)  same, fp32 tensors
    fa_bwd(q, k, v, o, dout, lse, scale, ...) -> (dq, dk, dv)
    fa_fwd_bias(q, k, v, bias, scale, causal, window) -> (o, lse)
    fa_bwd_bias(q, k, v, bias, o, dout, lse, scale, ...) -> (dq, dk, dv)
    fa_bwd_workspace_size(T_q, Hq, d) -> int
    fa_decode(q, k, v, scale, causal, window, seqlens_k, num_splits) -> (o, lse)
    fa_decode_workspace_size(B, Hq, Nq, d, num_splits) -> int
    fa_decode_num_splits(B, Hq, Hkv, Nq, Nk) -> int
    fa_status_string(status) -> str
"""

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_mi355x.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {fa_status_string(status)} ({status})")


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m exact_io_aware_28_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        fwd_args = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, vp]
        L.fa_fwd.argtypes = fwd_args
        L.fa_fwd.restype = i
        L.fa_fwd_f16.argtypes = fwd_args
        L.fa_fwd_f16.restype = i
        L.fa_fwd_f32.argtypes = fwd_args
        L.fa_fwd_f32.restype = i
        L.fa_bwd_workspace_size.argtypes = [i, i, i]
        L.fa_bwd_workspace_size.restype = ctypes.c_size_t
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                             i, i, i, i, i, i, f, i, i, vp, vp]
        L.fa_bwd.restype = i
        i64 = ctypes.c_int64
        L.fa_fwd_bias.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i,
                                  vp, i64, i64, i64, vp]
        L.fa_fwd_bias.restype = i
        L.fa_bwd_bias.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                  i, i, i, i, i, i, f, i, i, vp, i64, i64, i64, vp]
        L.fa_bwd_bias.restype = i
        u64 = ctypes.c_uint64
        L.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, f,
                                     u64, vp]
        L.fa_fwd_dropout.restype = i
        L.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, i, i, i, i, i, i, f, i, i, vp, f, u64,
                                     vp]
        L.fa_bwd_dropout.restype = i
        L.fa_decode_workspace_size.argtypes = [i, i, i, i, i]
        L.fa_decode_workspace_size.restype = ctypes.c_size_t
        L.fa_decode_num_splits.argtypes = [i, i, i, i, i]
        L.fa_decode_num_splits.restype = i
        L.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, i, vp,
                                ctypes.c_size_t, vp]
        L.fa_decode.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def fa_status_string(status):
    return lib().fa_status_string(int(status)).decode()


def fa_bwd_workspace_size(T_q, Hq, d):
    return int(lib().fa_bwd_workspace_size(int(T_q), int(Hq), int(d)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _geometry(q, k, cu_seqlens, max_seqlen):
    """(B, Hq, Hkv, Nq, Nk, d) from the tensor shapes (layouts of the ABI)."""
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense q/k/v must be [B, N, H, d]")
        B, nq, hq, d = q.shape
        nk, hkv = k.shape[1], k.shape[2]
        return B, hq, hkv, nq, nk, d
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q/k/v must be [T, H, d]")
    if max_seqlen is None:
        raise ValueError("packed batches need max_seqlen")
    B = cu_seqlens.numel() - 1
    return B, q.shape[1], k.shape[1], int(max_seqlen), int(max_seqlen), q.shape[2]


def _check(tensors, dtype):
    for name, t in tensors.items():
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _lse_shape(q, B, hq, nq, cu_seqlens):
    return (B, hq, nq) if cu_seqlens is None else (hq, q.shape[0])


def _fwd(fn, dtype, q, k, v, scale, causal, window, cu_seqlens, max_seqlen, out,
         lse, stream):
    import torch
    _check({"q": q, "k": k, "v": v}, dtype)
    B, hq, hkv, nq, nk, d = _geometry(q, k, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(_lse_shape(q, B, hq, nq, cu_seqlens), dtype=torch.float32,
                          device=q.device)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq, nk, d,
            float(scale), int(bool(causal)), int(window), _ptr(cu_seqlens),
            _stream(stream))
    if st != FA_OK:
        raise FaError(st, fn.__name__)
    return out, lse


def fa_fwd(q, k, v, scale=None, causal=False, window=0, cu_seqlens=None,
           max_seqlen=None, out=None, lse=None, stream=None):
    """bf16 forward; returns (o bf16, lse fp32).  See include/fa_mi355x.h."""
    import torch
    return _fwd(lib().fa_fwd, torch.bfloat16, q, k, v, scale, causal, window,
                cu_seqlens, max_seqlen, out, lse, stream)


def fa_fwd_f16(q, k, v, scale=None, causal=False, window=0, cu_seqlens=None,
               max_seqlen=None, out=None, lse=None, stream=None):
    """fp16 forward; returns (o fp16, lse fp32)."""
    import torch
    return _fwd(lib().fa_fwd_f16, torch.float16, q, k, v, scale, causal, window,
                cu_seqlens, max_seqlen, out, lse, stream)


def fa_fwd_f32(q, k, v, scale=None, causal=False, window=0, cu_seqlens=None,
               max_seqlen=None, out=None, lse=None, stream=None):
    """fp32 forward; returns (o fp32, lse fp32)."""
    import torch
    return _fwd(lib().fa_fwd_f32, torch.float32, q, k, v, scale, causal, window,
                cu_seqlens, max_seqlen, out, lse, stream)


def fa_bwd(q, k, v, o, dout, lse, scale=None, causal=False, window=0,
           cu_seqlens=None, max_seqlen=None, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """bf16 backward by recomputation; returns (dq, dk, dv)."""
    import torch
    _check({"q": q, "k": k, "v": v, "o": o, "dout": dout}, torch.bfloat16)
    _check({"lse": lse}, torch.float32)
    B, hq, hkv, nq, nk, d = _geometry(q, k, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = fa_bwd_workspace_size(B * nq, hq, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                      _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                      workspace.numel() * workspace.element_size(),
                      B, hq, hkv, nq, nk, d, float(scale), int(bool(causal)),
                      int(window), _ptr(cu_seqlens), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_fwd_dropout(q, k, v, dropout_p, seed, scale=None, causal=False, window=0,
                   cu_seqlens=None, max_seqlen=None, out=None, lse=None, stream=None):
    """bf16 forward with dropout on the probabilities (Philox keep-mask of
    the public header); returns (o bf16, lse fp32 of the undropped P).
    dropout_p is passed as a C float."""
    import torch
    _check({"q": q, "k": k, "v": v}, torch.bfloat16)
    B, hq, hkv, nq, nk, d = _geometry(q, k, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty(_lse_shape(q, B, hq, nq, cu_seqlens), dtype=torch.float32,
                          device=q.device)
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    st = lib().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv,
                              nq, nk, d, float(scale), int(bool(causal)), int(window),
                              _ptr(cu_seqlens), float(dropout_p), int(seed), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_dropout")
    return out, lse


def fa_bwd_dropout(q, k, v, o, dout, lse, dropout_p, seed, scale=None, causal=False,
                   window=0, cu_seqlens=None, max_seqlen=None, dq=None, dk=None, dv=None,
                   workspace=None, stream=None):
    """bf16 backward of fa_fwd_dropout (same dropout_p and seed); returns
    (dq, dk, dv)."""
    import torch
    _check({"q": q, "k": k, "v": v, "o": o, "dout": dout}, torch.bfloat16)
    _check({"lse": lse}, torch.float32)
    B, hq, hkv, nq, nk, d = _geometry(q, k, cu_seqlens, max_seqlen)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = fa_bwd_workspace_size(B * nq, hq, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                              workspace.numel() * workspace.element_size(),
                              B, hq, hkv, nq, nk, d, float(scale), int(bool(causal)),
                              int(window), _ptr(cu_seqlens), float(dropout_p), int(seed),
                              _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dropout")
    return dq, dk, dv


def _bias_view(bias, B, hq, nq, nk):
    """(tensor, stride_b, stride_h, stride_q): an fp32 device bias that
    broadcasts to [B, Hq, Nq, Nk] as a strided view (no copy unless its key
    dimension is not contiguous)."""
    import torch
    if bias.dtype != torch.float32 or not bias.is_cuda:
        raise TypeError("bias must be a float32 device tensor")
    if bias.dim() > 4:
        raise ValueError("bias must broadcast to [B, Hq, Nq, Nk]")
    if bias.stride(-1) != 1 and bias.shape[-1] != 1:
        bias = bias.contiguous()
    if bias.shape[-1] == 1 and nk != 1:
        raise ValueError("the key dimension of the bias cannot broadcast")
    b4 = bias.reshape((1,) * (4 - bias.dim()) + tuple(bias.shape)) if bias.dim() < 4 else bias
    e = b4.expand(B, hq, nq, nk)
    return e, e.stride(0), e.stride(1), e.stride(2)


def fa_fwd_bias(q, k, v, bias, scale=None, causal=False, window=0, out=None, lse=None,
                stream=None):
    """bf16 forward with an additive fp32 bias that broadcasts to
    [B, Hq, Nq, Nk]; returns (o bf16, lse fp32).  Dense batches only."""
    import torch
    _check({"q": q, "k": k, "v": v}, torch.bfloat16)
    B, hq, hkv, nq, nk, d = _geometry(q, k, None, None)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    bt, sb, sh, sq = _bias_view(bias, B, hq, nq, nk)
    st = lib().fa_fwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq,
                           nk, d, float(scale), int(bool(causal)), int(window), _ptr(bt),
                           sb, sh, sq, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_bias")
    return out, lse


def fa_bwd_bias(q, k, v, bias, o, dout, lse, scale=None, causal=False, window=0,
                dq=None, dk=None, dv=None, workspace=None, stream=None):
    """bf16 backward of fa_fwd_bias (the bias is a constant); returns
    (dq, dk, dv)."""
    import torch
    _check({"q": q, "k": k, "v": v, "o": o, "dout": dout}, torch.bfloat16)
    _check({"lse": lse}, torch.float32)
    B, hq, hkv, nq, nk, d = _geometry(q, k, None, None)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = fa_bwd_workspace_size(B * nq, hq, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    bt, sb, sh, sq = _bias_view(bias, B, hq, nq, nk)
    st = lib().fa_bwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                           _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                           workspace.numel() * workspace.element_size(),
                           B, hq, hkv, nq, nk, d, float(scale), int(bool(causal)),
                           int(window), _ptr(bt), sb, sh, sq, _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_bias")
    return dq, dk, dv


def fa_decode_workspace_size(B, Hq, Nq, d, num_splits):
    return int(lib().fa_decode_workspace_size(int(B), int(Hq), int(Nq), int(d),
                                              int(num_splits)))


def fa_decode_num_splits(B, Hq, Hkv, Nq, Nk):
    return int(lib().fa_decode_num_splits(int(B), int(Hq), int(Hkv), int(Nq), int(Nk)))


def fa_decode(q, k, v, scale=None, causal=False, window=0, seqlens_k=None,
              num_splits=None, out=None, lse=None, workspace=None, stream=None):
    """Split-KV attention of a few query rows per sequence over a K/V cache;
    returns (o bf16 [B, Nq, Hq, d], lse fp32 [B, Hq, Nq])."""
    import torch
    _check({"q": q, "k": k, "v": v}, torch.bfloat16)
    B, hq, hkv, nq, nk, d = _geometry(q, k, None, None)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seqlens_k is not None and seqlens_k.dtype != torch.int32:
        raise TypeError("seqlens_k must be int32")
    if num_splits is None:
        num_splits = fa_decode_num_splits(B, hq, hkv, nq, nk)
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    ws_bytes = fa_decode_workspace_size(B, hq, nq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq,
                         nk, d, float(scale), int(bool(causal)), int(window),
                         _ptr(seqlens_k), int(num_splits), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    if st != FA_OK:
        raise FaError(st, "fa_decode")
    return out, lse
