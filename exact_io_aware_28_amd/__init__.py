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
    fa_decode_noalloc(q, k, v, out, lse, ...) -> (out, lse), no allocation
    fa_decode_noalloc_max_splits(B, Hq, Nq, d) -> int
    fa_quantize_fp8(x, signs, transpose) -> (x8 float8_e4m3fn, scales)
    fa_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, ...) -> (o bf16, lse)
    fa_status_string(status) -> str
"""

import contextlib
import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_mi355x.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
# bytes of the static device array behind fa_decode_noalloc (per GPU)
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {fa_status_string(status)} ({status})")


LIB_DEBUG_SYNC_PATH = os.path.join(_HERE, "libfa_mi355x_debugsync.so")
_override = None


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the wrappers against another build of the same sources (the
    stage-synchronised LIB_DEBUG_SYNC_PATH) inside the block."""
    global _override
    prev = _override
    _override = _load(path)
    try:
        yield _override
    finally:
        _override = prev


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m exact_io_aware_28_amd.build --all` (no fallback exists)")
    L = ctypes.CDLL(path)
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
    L.fa_bwd_f16.argtypes = L.fa_bwd.argtypes
    L.fa_bwd_f16.restype = i
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
    L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, i,
                                    vp]
    L.fa_decode_noalloc.restype = i
    L.fa_decode_noalloc_max_splits.argtypes = [i, i, i, i]
    L.fa_decode_noalloc_max_splits.restype = i
    L.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp]
    L.fa_quantize_fp8.restype = i
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    return L


def fa_status_string(status):
    return lib().fa_status_string(int(status)).decode()


def fa_bwd_workspace_size(T_q, Hq, d):
    return int(lib().fa_bwd_workspace_size(int(T_q), int(Hq), int(d)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _launch_stream(stream):
    """The torch stream the call runs on (the current one by default)."""
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _on(stream):
    """Context for the binding's own allocations: made on the stream that the
    kernels read and write them on, so that the caching allocator never hands
    their memory to other work while those kernels may still use it."""
    import torch
    return torch.cuda.stream(stream)


# ------------------------------------------------------------------ checks
# Every wrapper checks all of its arguments before anything is allocated or
# launched: first what the host can see (types, dtypes, shapes, contiguity,
# sizes), then that every tensor lives on q's device.  A pointer the kernels
# would misread (a host address, int64 offsets, a short output) is refused
# here rather than faulting on the GPU.

def _tensor(name, t, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _optional(name, t, dtype, shape):
    return None if t is None else _tensor(name, t, dtype, shape)


def _workspace(t, nbytes):
    """A caller-supplied scratch buffer: any dtype, contiguous, at least
    `nbytes` long."""
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if _nbytes(t) < nbytes:
        raise ValueError(f"workspace holds {_nbytes(t)} bytes, needs {nbytes}")
    return t


def _same_device(device, named):
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _geometry(q, k, v, cu_seqlens, max_seqlen, dtype):
    """Check q, k, v (and cu_seqlens) against each other and the layouts of
    the C ABI (host-visible facts only); returns (B, Hq, Hkv, Nq, Nk, d)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tensor(name, t, dtype)
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k and v must have the same shape, got {tuple(k.shape)} "
                         f"and {tuple(v.shape)}")
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense q/k/v must be [B, N, H, d]")
        B, nq, hq, d = q.shape
        if k.shape[0] != B:
            raise ValueError(f"k has batch {k.shape[0]}, q has {B}")
        if k.shape[3] != d:
            raise ValueError(f"k has head dimension {k.shape[3]}, q has {d}")
        return B, hq, k.shape[2], nq, k.shape[1], d
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q/k/v must be [T, H, d]")
    if k.shape[0] != q.shape[0]:
        raise ValueError(f"packed k has {k.shape[0]} tokens, q has {q.shape[0]}")
    if k.shape[2] != q.shape[2]:
        raise ValueError(f"k has head dimension {k.shape[2]}, q has {q.shape[2]}")
    _tensor("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with B + 1 >= 2 offsets")
    if max_seqlen is None or int(max_seqlen) < 1:
        raise ValueError("packed batches need max_seqlen >= 1")
    B = cu_seqlens.numel() - 1
    return B, q.shape[1], k.shape[1], int(max_seqlen), int(max_seqlen), q.shape[2]


def _lse_shape(q, B, hq, nq, cu_seqlens):
    return (B, hq, nq) if cu_seqlens is None else (hq, q.shape[0])


def _alloc(t, shape, dtype, stream, device):
    """t if the caller supplied it, else a new tensor made on `stream`."""
    import torch
    if t is not None:
        return t
    with _on(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream_arg(s):
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ forward
def _fwd(fn, dtype, q, k, v, scale, causal, window, cu_seqlens, max_seqlen, out, lse,
         stream, extra=()):
    import torch
    B, hq, hkv, nq, nk, d = _geometry(q, k, v, cu_seqlens, max_seqlen, dtype)
    lse_shape = _lse_shape(q, B, hq, nq, cu_seqlens)
    _optional("out", out, dtype, q.shape)
    _optional("lse", lse, torch.float32, lse_shape)
    _same_device(q.device, [("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens),
                            ("out", out), ("lse", lse)])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = _launch_stream(stream)
    out = _alloc(out, q.shape, dtype, s, q.device)
    lse = _alloc(lse, lse_shape, torch.float32, s, q.device)
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq, nk, d,
            float(scale), int(bool(causal)), int(window), _ptr(cu_seqlens), *extra,
            _stream_arg(s))
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


def fa_fwd_dropout(q, k, v, dropout_p, seed, scale=None, causal=False, window=0,
                   cu_seqlens=None, max_seqlen=None, out=None, lse=None, stream=None):
    """bf16 forward with dropout on the probabilities (Philox keep-mask of
    the public header); returns (o bf16, lse fp32 of the undropped P).
    dropout_p is passed as a C float."""
    import torch
    return _fwd(lib().fa_fwd_dropout, torch.bfloat16, q, k, v, scale, causal, window,
                cu_seqlens, max_seqlen, out, lse, stream,
                extra=(float(dropout_p), int(seed)))


# ------------------------------------------------------------------ backward
def _bwd_prepare(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, dq, dk, dv, workspace,
                 stream, bias=None, dtype=None):
    """Checks and outputs shared by the backward wrappers (dtype: that of
    q, k, v, o, dout and the gradients; bf16 unless given)."""
    import torch
    dt = torch.bfloat16 if dtype is None else dtype
    B, hq, hkv, nq, nk, d = _geometry(q, k, v, cu_seqlens, max_seqlen, dt)
    _tensor("o", o, dt, q.shape)
    _tensor("dout", dout, dt, q.shape)
    _tensor("lse", lse, torch.float32, _lse_shape(q, B, hq, nq, cu_seqlens))
    _optional("dq", dq, dt, q.shape)
    _optional("dk", dk, dt, k.shape)
    _optional("dv", dv, dt, v.shape)
    ws_bytes = fa_bwd_workspace_size(B * nq, hq, d)
    _workspace(workspace, ws_bytes)
    bview = None if bias is None else _bias_view(bias, B, hq, nq, nk)
    _same_device(q.device, [("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout),
                            ("lse", lse), ("cu_seqlens", cu_seqlens), ("dq", dq), ("dk", dk),
                            ("dv", dv), ("workspace", workspace),
                            ("bias", None if bias is None else bias)])
    s = _launch_stream(stream)
    dq = _alloc(dq, q.shape, dt, s, q.device)
    dk = _alloc(dk, k.shape, dt, s, q.device)
    dv = _alloc(dv, v.shape, dt, s, q.device)
    ws = _alloc(workspace, (max(ws_bytes, 1),), torch.uint8, s, q.device)
    return (B, hq, hkv, nq, nk, d), s, dq, dk, dv, ws, bview


def _bwd_call(name, args, geo, scale, causal, window, tail, s):
    B, hq, hkv, nq, nk, d = geo
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = getattr(lib(), name)(*args, B, hq, hkv, nq, nk, d, float(scale), int(bool(causal)),
                              int(window), *tail, _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, name)


def fa_bwd(q, k, v, o, dout, lse, scale=None, causal=False, window=0,
           cu_seqlens=None, max_seqlen=None, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """bf16 backward by recomputation; returns (dq, dk, dv)."""
    geo, s, dq, dk, dv, ws, _ = _bwd_prepare(q, k, v, o, dout, lse, cu_seqlens, max_seqlen,
                                             dq, dk, dv, workspace, stream)
    args = [_ptr(x) for x in (q, k, v, o, dout, lse, dq, dk, dv, ws)] + [_nbytes(ws)]
    _bwd_call("fa_bwd", args, geo, scale, causal, window, [_ptr(cu_seqlens)], s)
    return dq, dk, dv


def fa_bwd_f16(q, k, v, o, dout, lse, scale=None, causal=False, window=0,
               cu_seqlens=None, max_seqlen=None, dq=None, dk=None, dv=None,
               workspace=None, stream=None):
    """fp16 backward of fa_fwd_f16; returns (dq, dk, dv) in fp16."""
    import torch
    geo, s, dq, dk, dv, ws, _ = _bwd_prepare(q, k, v, o, dout, lse, cu_seqlens, max_seqlen,
                                             dq, dk, dv, workspace, stream,
                                             dtype=torch.float16)
    args = [_ptr(x) for x in (q, k, v, o, dout, lse, dq, dk, dv, ws)] + [_nbytes(ws)]
    _bwd_call("fa_bwd_f16", args, geo, scale, causal, window, [_ptr(cu_seqlens)], s)
    return dq, dk, dv


def fa_bwd_dropout(q, k, v, o, dout, lse, dropout_p, seed, scale=None, causal=False,
                   window=0, cu_seqlens=None, max_seqlen=None, dq=None, dk=None, dv=None,
                   workspace=None, stream=None):
    """bf16 backward of fa_fwd_dropout (same dropout_p and seed); returns
    (dq, dk, dv)."""
    geo, s, dq, dk, dv, ws, _ = _bwd_prepare(q, k, v, o, dout, lse, cu_seqlens, max_seqlen,
                                             dq, dk, dv, workspace, stream)
    args = [_ptr(x) for x in (q, k, v, o, dout, lse, dq, dk, dv, ws)] + [_nbytes(ws)]
    _bwd_call("fa_bwd_dropout", args, geo, scale, causal, window,
              [_ptr(cu_seqlens), float(dropout_p), int(seed)], s)
    return dq, dk, dv


# ------------------------------------------------------------------ bias
def _bias_view(bias, B, hq, nq, nk):
    """(tensor, stride_b, stride_h, stride_q): an fp32 bias that broadcasts
    to [B, Hq, Nq, Nk] as a strided view (no copy unless its key dimension is
    not contiguous)."""
    import torch
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32:
        raise TypeError("bias must be a float32 tensor")
    if bias.dim() > 4:
        raise ValueError("bias must broadcast to [B, Hq, Nq, Nk]")
    if bias.shape[-1] == 1 and nk != 1:
        raise ValueError("the key dimension of the bias cannot broadcast")
    b4 = bias.reshape((1,) * (4 - bias.dim()) + tuple(bias.shape)) if bias.dim() < 4 else bias
    try:
        b4.expand(B, hq, nq, nk)
    except RuntimeError as exc:
        raise ValueError(f"bias of shape {tuple(bias.shape)} does not broadcast to "
                         f"{(B, hq, nq, nk)}") from exc
    return b4


def _bias_strides(b4, B, hq, nq, nk):
    if b4.stride(-1) != 1 and nk != 1:  # the kernels read keys at unit stride
        b4 = b4.contiguous()
    e = b4.expand(B, hq, nq, nk)
    return e, e.stride(0), e.stride(1), e.stride(2)


def fa_fwd_bias(q, k, v, bias, scale=None, causal=False, window=0, out=None, lse=None,
                stream=None):
    """bf16 forward with an additive fp32 bias that broadcasts to
    [B, Hq, Nq, Nk]; returns (o bf16, lse fp32).  Dense batches only."""
    import torch
    B, hq, hkv, nq, nk, d = _geometry(q, k, v, None, None, torch.bfloat16)
    b4 = _bias_view(bias, B, hq, nq, nk)
    _optional("out", out, torch.bfloat16, q.shape)
    _optional("lse", lse, torch.float32, (B, hq, nq))
    _same_device(q.device, [("q", q), ("k", k), ("v", v), ("bias", bias), ("out", out),
                            ("lse", lse)])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = _launch_stream(stream)
    bt, sb, sh, sq = _bias_strides(b4, B, hq, nq, nk)
    out = _alloc(out, q.shape, torch.bfloat16, s, q.device)
    lse = _alloc(lse, (B, hq, nq), torch.float32, s, q.device)
    st = lib().fa_fwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq,
                           nk, d, float(scale), int(bool(causal)), int(window), _ptr(bt),
                           sb, sh, sq, _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_bias")
    return out, lse


def fa_bwd_bias(q, k, v, bias, o, dout, lse, scale=None, causal=False, window=0,
                dq=None, dk=None, dv=None, workspace=None, stream=None):
    """bf16 backward of fa_fwd_bias (the bias is a constant); returns
    (dq, dk, dv)."""
    geo, s, dq, dk, dv, ws, b4 = _bwd_prepare(q, k, v, o, dout, lse, None, None, dq, dk, dv,
                                              workspace, stream, bias=bias)
    B, hq, hkv, nq, nk, d = geo
    bt, sb, sh, sq = _bias_strides(b4, B, hq, nq, nk)
    args = [_ptr(x) for x in (q, k, v, o, dout, lse, dq, dk, dv, ws)] + [_nbytes(ws)]
    _bwd_call("fa_bwd_bias", args, geo, scale, causal, window, [_ptr(bt), sb, sh, sq], s)
    return dq, dk, dv


# ------------------------------------------------------------------ decode
def fa_decode_workspace_size(B, Hq, Nq, d, num_splits):
    return int(lib().fa_decode_workspace_size(int(B), int(Hq), int(Nq), int(d),
                                              int(num_splits)))


def fa_decode_num_splits(B, Hq, Hkv, Nq, Nk):
    return int(lib().fa_decode_num_splits(int(B), int(Hq), int(Hkv), int(Nq), int(Nk)))


def _decode_prepare(q, k, v, seqlens_k, num_splits, out, lse, workspace, stream,
                    need_workspace=True):
    import torch
    B, hq, hkv, nq, nk, d = _geometry(q, k, v, None, None, torch.bfloat16)
    if seqlens_k is not None:
        _tensor("seqlens_k", seqlens_k, torch.int32, (B,))
    if num_splits is None:
        num_splits = fa_decode_num_splits(B, hq, hkv, nq, nk)
    num_splits = int(num_splits)
    _optional("out", out, torch.bfloat16, q.shape)
    _optional("lse", lse, torch.float32, (B, hq, nq))
    ws_bytes = fa_decode_workspace_size(B, hq, nq, d, num_splits) if need_workspace else 0
    if need_workspace:
        _workspace(workspace, ws_bytes)
    _same_device(q.device, [("q", q), ("k", k), ("v", v), ("seqlens_k", seqlens_k),
                            ("out", out), ("lse", lse), ("workspace", workspace)])
    s = _launch_stream(stream)
    out = _alloc(out, q.shape, torch.bfloat16, s, q.device)
    lse = _alloc(lse, (B, hq, nq), torch.float32, s, q.device)
    ws = _alloc(workspace, (max(ws_bytes, 1),), torch.uint8, s, q.device) \
        if need_workspace else None
    return (B, hq, hkv, nq, nk, d), num_splits, s, out, lse, ws


def fa_decode(q, k, v, scale=None, causal=False, window=0, seqlens_k=None,
              num_splits=None, out=None, lse=None, workspace=None, stream=None):
    """Split-KV attention of a few query rows per sequence over a K/V cache;
    returns (o bf16 [B, Nq, Hq, d], lse fp32 [B, Hq, Nq])."""
    (B, hq, hkv, nq, nk, d), num_splits, s, out, lse, ws = _decode_prepare(
        q, k, v, seqlens_k, num_splits, out, lse, workspace, stream)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv, nq,
                         nk, d, float(scale), int(bool(causal)), int(window),
                         _ptr(seqlens_k), num_splits, _ptr(ws), _nbytes(ws), _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, "fa_decode")
    return out, lse


def fa_decode_noalloc_max_splits(B, Hq, Nq, d):
    return int(lib().fa_decode_noalloc_max_splits(int(B), int(Hq), int(Nq), int(d)))


def fa_decode_noalloc(q, k, v, out, lse, scale=None, causal=False, window=0, seqlens_k=None,
                      num_splits=0, stream=None):
    """fa_decode for callers that cannot allocate: the caller passes the
    outputs (out bf16 like q, lse fp32 [B, Hq, Nq]) and the split partials go
    to the library's static device scratch, so neither this wrapper nor the
    library allocates.  num_splits = 0 picks the default count that fits.
    Calls that overlap on one GPU race on the scratch."""
    import torch
    if out is None or lse is None:
        raise ValueError("fa_decode_noalloc writes into caller-supplied out and lse")
    B, hq, hkv, nq, nk, d = _geometry(q, k, v, None, None, torch.bfloat16)
    if seqlens_k is not None:
        _tensor("seqlens_k", seqlens_k, torch.int32, (B,))
    _tensor("out", out, torch.bfloat16, q.shape)
    _tensor("lse", lse, torch.float32, (B, hq, nq))
    _same_device(q.device, [("q", q), ("k", k), ("v", v), ("seqlens_k", seqlens_k),
                            ("out", out), ("lse", lse)])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = _launch_stream(stream)
    st = lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, hq, hkv,
                                 nq, nk, d, float(scale), int(bool(causal)), int(window),
                                 _ptr(seqlens_k), int(num_splits), _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, "fa_decode_noalloc")
    return out, lse


# ------------------------------------------------------------------ FP8
FP8_BLOCK = 64  # tokens per scale block


def _fp8(name, t, shape):
    """An E4M3 code tensor (torch.float8_e4m3fn or raw uint8 bytes)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be a float8_e4m3fn (or uint8) tensor")
    return _tensor(name, t, t.dtype, shape)


def fa_quantize_fp8(x, signs=None, transpose=False, out=None, scales=None, stream=None):
    """Block-quantize bf16 x [B, N, H, d] to E4M3 (one fp32 scale per 64
    tokens of one head), optionally rotating each row by x D H / sqrt(d)
    first (signs: device fp32 [d] of +-1).  Returns (x8, scales): x8 is
    float8_e4m3fn [B, N, H, d], or [B, H, d, ldn] (ldn = N rounded up to 64,
    zero padded) with transpose=True, the layout fa_fwd_fp8 takes for V."""
    import torch
    _tensor("x", x, torch.bfloat16)
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, d]")
    B, N, H, d = x.shape
    nb = -(-N // FP8_BLOCK)
    shape = (B, H, d, nb * FP8_BLOCK) if transpose else (B, N, H, d)
    if out is not None:
        _fp8("out", out, shape)
    _optional("scales", scales, torch.float32, (B, H, nb))
    if signs is not None:
        _tensor("signs", signs, torch.float32, (d,))
    _same_device(x.device, [("x", x), ("out", out), ("scales", scales), ("signs", signs)])
    s = _launch_stream(stream)
    out = _alloc(out, shape, torch.float8_e4m3fn, s, x.device)
    scales = _alloc(scales, (B, H, nb), torch.float32, s, x.device)
    st = lib().fa_quantize_fp8(_ptr(x), _ptr(out), _ptr(scales), B, N, H, d, int(bool(transpose)),
                               _ptr(signs), _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, "fa_quantize_fp8")
    return out, scales


def fa_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, scale=None, causal=False, window=0,
               out=None, lse=None, stream=None):
    """FP8 forward over E4M3 codes with block scales (see
    include/fa_mi355x.h): q8 [B, Nq, Hq, d], k8 [B, Nk, Hkv, d], vt8
    [B, Hkv, d, ldv] (ldv = Nk rounded up to 64), scales [B, H, ceil(N/64)].
    Returns (o bf16 [B, Nq, Hq, d], lse fp32 [B, Hq, Nq])."""
    import torch
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        _fp8(name, t, None)
    if q8.dim() != 4 or k8.dim() != 4 or vt8.dim() != 4:
        raise ValueError("q8, k8 must be [B, N, H, d] and vt8 [B, Hkv, d, ldv]")
    B, nq, hq, d = q8.shape
    nk, hkv = k8.shape[1], k8.shape[2]
    if k8.shape[0] != B or k8.shape[3] != d:
        raise ValueError(f"k8 {tuple(k8.shape)} does not match q8 {tuple(q8.shape)}")
    ldv = -(-nk // FP8_BLOCK) * FP8_BLOCK
    _fp8("vt8", vt8, (B, hkv, d, ldv))
    _tensor("q_scale", q_scale, torch.float32, (B, hq, -(-nq // FP8_BLOCK)))
    _tensor("k_scale", k_scale, torch.float32, (B, hkv, -(-nk // FP8_BLOCK)))
    _tensor("v_scale", v_scale, torch.float32, (B, hkv, -(-nk // FP8_BLOCK)))
    _optional("out", out, torch.bfloat16, (B, nq, hq, d))
    _optional("lse", lse, torch.float32, (B, hq, nq))
    _same_device(q8.device, [("q8", q8), ("k8", k8), ("vt8", vt8), ("q_scale", q_scale),
                             ("k_scale", k_scale), ("v_scale", v_scale), ("out", out),
                             ("lse", lse)])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = _launch_stream(stream)
    out = _alloc(out, (B, nq, hq, d), torch.bfloat16, s, q8.device)
    lse = _alloc(lse, (B, hq, nq), torch.float32, s, q8.device)
    st = lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(q_scale), _ptr(k_scale),
                          _ptr(v_scale), _ptr(out), _ptr(lse), B, hq, hkv, nq, nk, d,
                          float(scale), int(bool(causal)), int(window), _stream_arg(s))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse
