"""Thin Python binding of the C ABI in include/flash_attn.h.

Functions carry the C names and only marshal arguments: they check tensor metadata, allocate
output tensors with torch when the caller passes none, and hand raw device pointers plus the
current HIP stream to the library.  Every arithmetic step runs in the library's kernels.
"""
import ctypes
import math

import torch

from . import _lib

_DT = {torch.float32: _lib.FA_DTYPE_F32, torch.bfloat16: _lib.FA_DTYPE_BF16,
       torch.float16: _lib.FA_DTYPE_F16}


class FlashAttnError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {_lib.status_string(code)}")
        self.code = code


def _check(fn, code):
    if code != _lib.FA_OK:
        raise FlashAttnError(fn, code)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _dims(q, k):
    """(B, T, H, HKV, D) of q [B,T,H,D] and k [B,T,HKV,D] (one length for queries and keys)."""
    B, T, Tk, H, HKV, D = _dims_qk(q, k)
    if Tk != T:
        raise ValueError("q and k differ in length; use the *_strided entry points")
    return B, T, H, HKV, D


def _dims_qk(q, k):
    """(B, T, Tk, H, HKV, D) of q [B,T,H,D] and k [B,Tk,HKV,D]."""
    if (not isinstance(q, torch.Tensor) or not isinstance(k, torch.Tensor) or q.dim() != 4
            or k.dim() != 4):
        raise ValueError("expected q [B,T,H,D] and k/v [B,Tk,HKV,D]")
    B, T, H, D = q.shape
    Bk, Tk, HKV, Dk = k.shape
    if (Bk, Dk) != (B, D):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ in batch or head dim")
    return B, T, Tk, H, HKV, D


def _want(t, shape, dtype, name, device=None):
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or not t.is_contiguous() or not t.is_cuda
            or (device is not None and t.device != device)):
        where = f" on {device}" if device is not None else ""
        raise ValueError(f"{name}: expected contiguous {dtype} cuda tensor of shape "
                         f"{tuple(shape)}{where}")


def _dtype_code(dtype):
    if dtype not in _DT:
        raise ValueError(f"unsupported dtype {dtype}: expected float32, bfloat16 or float16")
    return _DT[dtype]


def _want_inputs(q, k, v, **more):
    """q [B,T,H,D], k and v [B,Tk,HKV,D] contiguous, on one device, in one supported dtype;
    each tensor of `more` contiguous with q's shape and dtype on that device."""
    _dtype_code(q.dtype)
    dev = q.device
    _want(q, q.shape, q.dtype, "q", dev)
    _want(k, k.shape, q.dtype, "k", dev)
    _want(v, k.shape, q.dtype, "v", dev)
    for name, t in more.items():
        _want(t, q.shape, q.dtype, name, dev)


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def flash_attn_fwd(q, k, v, causal=True, window=0, scale=None, out=None, lse=None, tiles=(0, 0),
                   stream=None):
    """O [B,T,H,D] (q.dtype) and L [B,H,T] (float32) for q [B,T,H,D], k, v [B,T,HKV,D]."""
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v)
    dt = _DT[q.dtype]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, H, T, device=q.device, dtype=torch.float32) if lse is None else lse
    _want(out, q.shape, q.dtype, "out", q.device)
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    code = _lib.lib().flash_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, T, H,
                                        HKV, D, _scale(scale, D), int(bool(causal)), int(window),
                                        dt, _stream(stream), int(tiles[0]), int(tiles[1]))
    _check("flash_attn_fwd", code)
    return out, lse


def flash_attn_bwd_preprocess(o, do, dvec=None, stream=None):
    if not isinstance(o, torch.Tensor) or o.dim() != 4:
        raise ValueError("o: expected a [B, T, H, D] tensor")
    B, T, H, D = o.shape
    _dtype_code(o.dtype)
    _want(o, o.shape, o.dtype, "o", o.device)
    _want(do, o.shape, o.dtype, "do", o.device)
    dvec = torch.empty(B, H, T, device=o.device, dtype=torch.float32) if dvec is None else dvec
    _want(dvec, (B, H, T), torch.float32, "dvec", o.device)
    code = _lib.lib().flash_attn_bwd_preprocess(_ptr(o), _ptr(do), _ptr(dvec), B, T, H, D,
                                                _DT[o.dtype], _stream(stream))
    _check("flash_attn_bwd_preprocess", code)
    return dvec


def _grads(q, k, dq, dk, dv):
    f = torch.float32
    dq = torch.empty(q.shape, device=q.device, dtype=f) if dq is None else dq
    dk = torch.empty(k.shape, device=q.device, dtype=f) if dk is None else dk
    dv = torch.empty(k.shape, device=q.device, dtype=f) if dv is None else dv
    _want(dq, q.shape, f, "dq", q.device)
    _want(dk, k.shape, f, "dk", q.device)
    _want(dv, k.shape, f, "dv", q.device)
    return dq, dk, dv


def flash_attn_bwd_dkdv(q, k, v, do, lse, dvec, causal=True, window=0, scale=None, dk=None,
                        dv=None, tiles=(0, 0), stream=None):
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v, do=do)
    f = torch.float32
    _want(lse, (B, H, T), f, "lse", q.device)
    _want(dvec, (B, H, T), f, "dvec", q.device)
    dk = torch.empty(k.shape, device=q.device, dtype=f) if dk is None else dk
    dv = torch.empty(k.shape, device=q.device, dtype=f) if dv is None else dv
    _want(dk, k.shape, f, "dk", q.device)
    _want(dv, k.shape, f, "dv", q.device)
    code = _lib.lib().flash_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                                          _ptr(dvec), _ptr(dk), _ptr(dv), B, T, H, HKV, D,
                                          _scale(scale, D), int(bool(causal)), int(window),
                                          _DT[q.dtype], _stream(stream), int(tiles[0]),
                                          int(tiles[1]))
    _check("flash_attn_bwd_dkdv", code)
    return dk, dv


def flash_attn_bwd_dq(q, k, v, do, lse, dvec, causal=True, window=0, scale=None, dq=None,
                      tiles=(0, 0), stream=None):
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v, do=do)
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    _want(dvec, (B, H, T), torch.float32, "dvec", q.device)
    dq = torch.empty(q.shape, device=q.device, dtype=torch.float32) if dq is None else dq
    _want(dq, q.shape, torch.float32, "dq", q.device)
    code = _lib.lib().flash_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse),
                                        _ptr(dvec), _ptr(dq), B, T, H, HKV, D, _scale(scale, D),
                                        int(bool(causal)), int(window), _DT[q.dtype],
                                        _stream(stream), int(tiles[0]), int(tiles[1]))
    _check("flash_attn_bwd_dq", code)
    return dq


def flash_attn_bwd_dq_dvec(q, k, v, o, do, lse, dvec=None, causal=True, window=0, scale=None,
                           dq=None, tiles=(0, 0), stream=None):
    """dQ (float32) and Dvec = rowsum(dO * O) ([B,H,T] float32) in one pass; returns (dq, dvec)."""
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v, o=o, do=do)
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    dq = torch.empty(q.shape, device=q.device, dtype=torch.float32) if dq is None else dq
    dvec = torch.empty(B, H, T, device=q.device, dtype=torch.float32) if dvec is None else dvec
    _want(dq, q.shape, torch.float32, "dq", q.device)
    _want(dvec, (B, H, T), torch.float32, "dvec", q.device)
    code = _lib.lib().flash_attn_bwd_dq_dvec(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                             _ptr(lse), _ptr(dvec), _ptr(dq), B, T, H, HKV, D,
                                             _scale(scale, D), int(bool(causal)), int(window),
                                             _DT[q.dtype], _stream(stream), int(tiles[0]),
                                             int(tiles[1]))
    _check("flash_attn_bwd_dq_dvec", code)
    return dq, dvec


def flash_attn_bwd(q, k, v, o, lse, do, causal=True, window=0, scale=None, dq=None, dk=None,
                   dv=None, tiles=(0, 0), stream=None):
    """dQ, dK, dV (float32) of sum(O * dO); O, L from flash_attn_fwd on the same inputs."""
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v, o=o, do=do)
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    dq, dk, dv = _grads(q, k, dq, dk, dv)
    code = _lib.lib().flash_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                        _ptr(dq), _ptr(dk), _ptr(dv), B, T, H, HKV, D,
                                        _scale(scale, D), int(bool(causal)), int(window),
                                        _DT[q.dtype], _stream(stream), int(tiles[0]),
                                        int(tiles[1]))
    _check("flash_attn_bwd", code)
    return dq, dk, dv


def flash_attn_bwd_noalloc(q, k, v, o, lse, do, causal=True, window=0, scale=None, dq=None,
                           dk=None, dv=None, stream=None):
    """flash_attn_bwd with its Dvec workspace in the library's fixed per-device scratch instead
    of a per-call allocation (B*H*T up to FA_NOALLOC_MAX_DVEC).  Pass dq, dk, dv to keep the
    whole call free of allocations; calls that may overlap on one device race on the scratch."""
    B, T, H, HKV, D = _dims(q, k)
    _want_inputs(q, k, v, o=o, do=do)
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    dq, dk, dv = _grads(q, k, dq, dk, dv)
    code = _lib.lib().flash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                             _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, T, H, HKV,
                                             D, _scale(scale, D), int(bool(causal)), int(window),
                                             _DT[q.dtype], _stream(stream))
    _check("flash_attn_bwd_noalloc", code)
    return dq, dk, dv


def _layout(t, name):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name}: expected a [B, T, heads, D] view with a contiguous last axis")
    sb, st, sh, _ = t.stride()
    return _lib.Layout(sb, st, sh)


def _want_view(t, like, dtype, name):
    """t must be a cuda tensor on like's device with like's shape and strides (elements), in
    dtype."""
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(like.shape)
            or tuple(t.stride()) != tuple(like.stride()) or t.dtype != dtype or not t.is_cuda
            or t.device != like.device):
        raise ValueError(f"{name}: expected a {dtype} cuda view with shape {tuple(like.shape)} "
                         f"and strides {tuple(like.stride())}")


def _empty_like_view(like, dtype):
    return torch.empty_strided(like.shape, like.stride(), dtype=dtype, device=like.device)


def flash_attn_fwd_strided(q, k, v, causal=True, window=0, scale=None, out=None, lse=None,
                           stream=None):
    """flash_attn_fwd on [B, T, heads, D] views with any strides (last axis contiguous), e.g.
    x.transpose(1, 2) of a [B, H, T, D] tensor or of a third of a packed QKV buffer.  k and v
    share strides; O takes q's strides."""
    B, T, Tk, H, HKV, D = _dims_qk(q, k)
    _dtype_code(q.dtype)
    _want_view(q, q, q.dtype, "q")
    _want_view(k, k, q.dtype, "k")
    _want_view(v, k, q.dtype, "v")
    out = _empty_like_view(q, q.dtype) if out is None else out
    _want_view(out, q, q.dtype, "out")
    lse = torch.empty(B, H, T, device=q.device, dtype=torch.float32) if lse is None else lse
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    code = _lib.lib().flash_attn_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                             B, T, Tk, H, HKV, D, _scale(scale, D),
                                             int(bool(causal)), int(window), _DT[q.dtype],
                                             _stream(stream), _layout(q, "q"), _layout(k, "k"))
    _check("flash_attn_fwd_strided", code)
    return out, lse


def flash_attn_bwd_strided(q, k, v, o, lse, do, causal=True, window=0, scale=None, dq=None,
                           dk=None, dv=None, stream=None):
    """flash_attn_bwd on strided views: o, do and dq (float32) take q's strides, dk and dv
    (float32) take k's."""
    B, T, Tk, H, HKV, D = _dims_qk(q, k)
    _dtype_code(q.dtype)
    _want_view(q, q, q.dtype, "q")
    _want_view(k, k, q.dtype, "k")
    _want_view(v, k, q.dtype, "v")
    _want_view(o, q, q.dtype, "o")
    _want_view(do, q, q.dtype, "do")
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    f32 = torch.float32
    dq = _empty_like_view(q, f32) if dq is None else dq
    dk = _empty_like_view(k, f32) if dk is None else dk
    dv = _empty_like_view(k, f32) if dv is None else dv
    _want_view(dq, q, f32, "dq")
    _want_view(dk, k, f32, "dk")
    _want_view(dv, k, f32, "dv")
    code = _lib.lib().flash_attn_bwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                             _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, T, Tk,
                                             H, HKV, D, _scale(scale, D), int(bool(causal)),
                                             int(window), _DT[q.dtype], _stream(stream),
                                             _layout(q, "q"), _layout(k, "k"))
    _check("flash_attn_bwd_strided", code)
    return dq, dk, dv


def flash_attn_bwd_grad16(q, k, v, o, lse, do, causal=True, window=0, scale=None, dq=None,
                          dk=None, dv=None, stream=None):
    """flash_attn_bwd_strided with dq, dk, dv in q's 16-bit dtype (each the float32 result
    rounded to nearest-even); dq takes q's strides, dk and dv k's."""
    B, T, Tk, H, HKV, D = _dims_qk(q, k)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("flash_attn_bwd_grad16 needs bfloat16 or float16 inputs")
    _want_view(q, q, q.dtype, "q")
    _want_view(k, k, q.dtype, "k")
    _want_view(v, k, q.dtype, "v")
    _want_view(o, q, q.dtype, "o")
    _want_view(do, q, q.dtype, "do")
    _want(lse, (B, H, T), torch.float32, "lse", q.device)
    dq = _empty_like_view(q, q.dtype) if dq is None else dq
    dk = _empty_like_view(k, q.dtype) if dk is None else dk
    dv = _empty_like_view(k, q.dtype) if dv is None else dv
    _want_view(dq, q, q.dtype, "dq")
    _want_view(dk, k, q.dtype, "dk")
    _want_view(dv, k, q.dtype, "dv")
    code = _lib.lib().flash_attn_bwd_grad16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, T, Tk,
                                            H, HKV, D, _scale(scale, D), int(bool(causal)),
                                            int(window), _DT[q.dtype], _stream(stream),
                                            _layout(q, "q"), _layout(k, "k"))
    _check("flash_attn_bwd_grad16", code)
    return dq, dk, dv


def flash_attn_qk_norm_rope(qk, factor1, factor2, heads, rotary_dim=None, paired=False,
                            key_offset=False, out_q=None, out_k=None, stream=None):
    """(out_q, out_k) from a packed QK projection qk [tokens, 2*heads, D] (last axis
    contiguous, any token / head strides) and float32 factor tables [tokens, D] ([tokens, 2D]
    when paired): RMS-norm without weight, then y = factor1 * x + factor2 * pair_swap(x)."""
    if (not isinstance(qk, torch.Tensor) or qk.dim() != 3 or qk.stride(2) != 1
            or not qk.is_cuda):
        raise ValueError("qk: expected a cuda [tokens, 2*heads, D] tensor, last axis contiguous")
    _dtype_code(qk.dtype)
    tokens, heads2, D = qk.shape
    if heads2 != 2 * heads:
        raise ValueError("qk: second axis must be 2 * heads")
    rotary_dim = D if rotary_dim is None else rotary_dim
    width = D * (2 if paired else 1)
    for name, f in (("factor1", factor1), ("factor2", factor2)):
        if (not isinstance(f, torch.Tensor) or f.dtype != torch.float32 or not f.is_cuda
                or f.device != qk.device or f.dim() != 2
                or tuple(f.shape) != (tokens, width) or f.stride(1) != 1
                or f.stride() != factor1.stride()):
            raise ValueError(f"{name}: expected float32 cuda [{tokens}, {width}], last axis "
                             "contiguous, both tables with the same strides")
    shape = (2 * tokens, heads // 2, D) if paired else (tokens, heads, D)
    out_q = torch.empty(shape, device=qk.device, dtype=qk.dtype) if out_q is None else out_q
    out_k = torch.empty(shape, device=qk.device, dtype=qk.dtype) if out_k is None else out_k
    _want(out_q, shape, qk.dtype, "out_q", qk.device)
    _want(out_k, shape, qk.dtype, "out_k", qk.device)
    code = _lib.lib().flash_attn_qk_norm_rope(_ptr(qk), qk.stride(0), qk.stride(1),
                                              _ptr(factor1), _ptr(factor2), factor1.stride(0),
                                              _ptr(out_q), _ptr(out_k), tokens, heads, D,
                                              int(rotary_dim), int(bool(paired)),
                                              int(bool(key_offset)), _DT[qk.dtype],
                                              _stream(stream))
    _check("flash_attn_qk_norm_rope", code)
    return out_q, out_k


def flash_attn_block_class(T, bq, bk, causal, window, i, j):
    """(class, off) of block (i, j): class 0 skip, 1 full, 2 masked; off = i*bq - j*bk."""
    off = ctypes.c_int(0)
    cls = _lib.lib().flash_attn_block_class(T, bq, bk, int(bool(causal)), window, i, j,
                                            ctypes.byref(off))
    if cls < 0:
        raise FlashAttnError("flash_attn_block_class", _lib.FA_ERR_INVALID_ARG)
    return cls, off.value


def flash_attn_block_class_qk(Tq, Tk, bq, bk, causal, window, i, j):
    """Class of block (i, j) of a Tq x Tk problem (query rows at the last Tq key positions)."""
    return _lib.lib().flash_attn_block_class_qk(Tq, Tk, bq, bk, int(bool(causal)), window, i, j)


def flash_attn_kv_block_range_qk(Tq, Tk, bq, bk, causal, window, i):
    lo, hi = ctypes.c_int(), ctypes.c_int()
    code = _lib.lib().flash_attn_kv_block_range_qk(Tq, Tk, bq, bk, int(bool(causal)), window, i,
                                                   ctypes.byref(lo), ctypes.byref(hi))
    _check("flash_attn_kv_block_range_qk", code)
    return lo.value, hi.value


def flash_attn_kv_block_range(T, bq, bk, causal, window, i):
    lo, hi = ctypes.c_int(0), ctypes.c_int(0)
    _check("flash_attn_kv_block_range",
           _lib.lib().flash_attn_kv_block_range(T, bq, bk, int(bool(causal)), window, i,
                                                ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def flash_attn_default_tiles(dtype, D, pass_):
    bq, bk = ctypes.c_int(0), ctypes.c_int(0)
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    _check("flash_attn_default_tiles",
           _lib.lib().flash_attn_default_tiles(dt, D, pass_, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def flash_attn_check_layout(strides, B, T, heads, D, dtype):
    """Status code (0 = usable) of the library's check of element strides (batch, row, head)
    for a [B, T, heads, D] view; dtype 0 = f32, 1 = bf16."""
    return _lib.lib().flash_attn_check_layout(_lib.Layout(*strides), B, T, heads, D, dtype)


def flash_attn_mfma_rate_probe(operands, out, grid, iters, stream=None):
    """Launch the library's MFMA throughput probe (grid * 4 * iters * 32 bf16 16x16x32 MFMAs)
    on `operands` (4096 bfloat16 values, cuda) writing grid * 256 floats to `out`."""
    _want(operands, (4096,), torch.bfloat16, "operands")
    _want(out, (grid * 256,), torch.float32, "out", operands.device)
    _check("flash_attn_mfma_rate_probe",
           _lib.lib().flash_attn_mfma_rate_probe(_ptr(operands), _ptr(out), int(grid),
                                                 int(iters), _stream(stream)))
    return out


def flash_attn_version():
    return _lib.lib().flash_attn_version()
