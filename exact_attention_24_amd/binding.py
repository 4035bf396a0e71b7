"""ctypes binding of libfa.so (the C ABI in include/fa.h).

Argument marshalling only: every step of the attention computation runs in
the library's HIP kernels.  torch supplies device memory and the current
stream.  The functions carry the C names (fa_fwd, fa_varlen_fwd, fa_bwd,
fa_varlen_bwd, fa_*_workspace_bytes, fa_check_*); status codes become exceptions the way
the pages' error table does it (ms-swift long-text page, section 4.3): a dtype
mismatch or bad argument raises ValueError, anything else RuntimeError.
There is no fallback: if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_F32, FA_BF16, FA_FP8_E4M3 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_DTYPE_MISMATCH, FA_ERR_UNSUPPORTED, FA_ERR_HIP = range(5)
ABI_VERSION = 7

_I64x4 = ctypes.c_int64 * 4
_I64x3 = ctypes.c_int64 * 3
_I64x2 = ctypes.c_int64 * 2


class FwdParams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("qkv_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", _I64x3), ("k_stride", _I64x3), ("v_stride", _I64x3), ("o_stride", _I64x3),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
        ("dropout_p", ctypes.c_float), ("dropout_offset", ctypes.c_uint32), ("dropout_seed", ctypes.c_uint64),
    ]


class VarlenFwdParams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("qkv_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
        ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", _I64x2), ("k_stride", _I64x2), ("v_stride", _I64x2), ("o_stride", _I64x2),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float),
        ("dropout_p", ctypes.c_float), ("dropout_offset", ctypes.c_uint32), ("dropout_seed", ctypes.c_uint64),
    ]


class BwdParams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("qkv_dtype", ctypes.c_int), ("grad_dtype", ctypes.c_int),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", _I64x3), ("k_stride", _I64x3), ("v_stride", _I64x3), ("o_stride", _I64x3),
        ("do_stride", _I64x3), ("dq_stride", _I64x3), ("dk_stride", _I64x3), ("dv_stride", _I64x3),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("dropout_p", ctypes.c_float), ("dropout_offset", ctypes.c_uint32), ("dropout_seed", ctypes.c_uint64),
    ]


class VarlenBwdParams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("qkv_dtype", ctypes.c_int), ("grad_dtype", ctypes.c_int),
        ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", _I64x2), ("k_stride", _I64x2), ("v_stride", _I64x2), ("o_stride", _I64x2),
        ("do_stride", _I64x2), ("dq_stride", _I64x2), ("dk_stride", _I64x2), ("dv_stride", _I64x2),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("dropout_p", ctypes.c_float), ("dropout_offset", ctypes.c_uint32), ("dropout_seed", ctypes.c_uint64),
    ]


class MergeParams(ctypes.Structure):
    _fields_ = [
        ("o_parts", ctypes.c_void_p), ("lse_parts", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p), ("parts_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
        ("num_parts", ctypes.c_int32), ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("parts_stride", _I64x4), ("o_stride", _I64x3),
    ]


class KvcacheParams(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("cache_seqlens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("qkv_dtype", ctypes.c_int),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("cache_len", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_stride", _I64x3), ("kc_stride", _I64x3), ("vc_stride", _I64x3), ("kn_stride", _I64x3),
        ("vn_stride", _I64x3), ("o_stride", _I64x3),
        ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("page_block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
    ]


EXPORTS = ("fa_abi_version", "fa_last_error", "fa_check_fwd", "fa_check_varlen_fwd", "fa_check_bwd",
           "fa_check_varlen_bwd", "fa_fwd", "fa_varlen_fwd", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_varlen_bwd_workspace_bytes", "fa_varlen_bwd", "fa_check_merge", "fa_merge",
           "fa_check_kvcache", "fa_kvcache_workspace_bytes", "fa_fwd_kvcache", "fa_bwd_noalloc")

_lib = None


def lib():
    """Load libfa.so once (raises if it is not built or has another ABI)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`"
                           " (the attention ops have no other implementation)")
    L = ctypes.CDLL(LIB_PATH)
    L.fa_abi_version.restype = ctypes.c_int
    L.fa_last_error.restype = ctypes.c_char_p
    for name, ptype in (("fa_check_fwd", FwdParams), ("fa_check_varlen_fwd", VarlenFwdParams),
                        ("fa_check_bwd", BwdParams), ("fa_check_varlen_bwd", VarlenBwdParams),
                        ("fa_check_merge", MergeParams), ("fa_check_kvcache", KvcacheParams)):
        getattr(L, name).argtypes = [ctypes.POINTER(ptype)]
        getattr(L, name).restype = ctypes.c_int
    L.fa_fwd.argtypes = [ctypes.POINTER(FwdParams), ctypes.c_void_p]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_varlen_fwd.argtypes = [ctypes.POINTER(VarlenFwdParams), ctypes.c_void_p]
    L.fa_varlen_fwd.restype = ctypes.c_int
    L.fa_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdParams)]
    L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_bwd.argtypes = [ctypes.POINTER(BwdParams), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_noalloc.argtypes = [ctypes.POINTER(BwdParams), ctypes.c_void_p]
    L.fa_bwd_noalloc.restype = ctypes.c_int
    L.fa_varlen_bwd_workspace_bytes.argtypes = [ctypes.POINTER(VarlenBwdParams)]
    L.fa_varlen_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.fa_varlen_bwd.argtypes = [ctypes.POINTER(VarlenBwdParams), ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p]
    L.fa_varlen_bwd.restype = ctypes.c_int
    L.fa_merge.argtypes = [ctypes.POINTER(MergeParams), ctypes.c_void_p]
    L.fa_merge.restype = ctypes.c_int
    L.fa_kvcache_workspace_bytes.argtypes = [ctypes.POINTER(KvcacheParams)]
    L.fa_kvcache_workspace_bytes.restype = ctypes.c_size_t
    L.fa_fwd_kvcache.argtypes = [ctypes.POINTER(KvcacheParams), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.fa_fwd_kvcache.restype = ctypes.c_int
    if L.fa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libfa.so ABI {L.fa_abi_version()} != binding ABI {ABI_VERSION}; rebuild")
    _lib = L
    return L


class FaError(RuntimeError):
    pass


def _raise(status: int):
    if status == FA_OK:
        return
    msg = lib().fa_last_error().decode(errors="replace")
    if status in (FA_ERR_INVALID_ARGUMENT, FA_ERR_DTYPE_MISMATCH):
        raise ValueError(msg)
    raise FaError(f"status {status}: {msg}")


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return FA_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float8_e4m3fn)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _same_gpu(ref, **tensors):
    """Every tensor the kernels read or write must live on ref's GPU: a host
    pointer handed to a kernel would fault the device, not raise.  Checked by
    each launching entry point before anything is allocated or launched (the
    make_*_params builders stay usable on host tensors, for the host-only
    fa_check_* validators)."""
    if not ref.is_cuda:
        raise ValueError(f"tensors must be on a GPU (got {ref.device})")
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise ValueError(f"{name} must be on {ref.device} (got {t.device})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_last_dim(name, t):
    if t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last (head_dim) dimension")


def _set_dropout(p, dropout_p, seed, offset):
    """Dropout fields of a params struct; a nonzero p needs an explicit seed,
    since the backward must regenerate the forward's mask from it."""
    dropout_p = float(dropout_p)
    if dropout_p > 0.0 and seed is None:
        raise ValueError("dropout_p > 0 needs a seed (pass the same seed and offset to the backward)")
    p.dropout_p = dropout_p
    p.dropout_seed = int(seed or 0) & 0xFFFFFFFFFFFFFFFF
    p.dropout_offset = int(offset) & 0xFFFFFFFF


def _default_scale(d, softmax_scale):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def make_fwd_params(q, k, v, o, lse, causal=False, window=0, softmax_scale=None, descale=(1.0, 1.0, 1.0),
                    dropout_p=0.0, seed=None, offset=0):
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{n} must be [batch, seqlen, heads, head_dim] (got {tuple(t.shape)})")
        _check_last_dim(n, t)
    if _code(q) != _code(k) or _code(q) != _code(v):
        raise ValueError("Input and output tensors must have the same dtype (q, k, v differ)")
    b, nq, h, d = q.shape
    nk = k.shape[1]
    if k.shape != (b, nk, h, d) or v.shape != (b, nk, h, d) or o.shape != (b, nq, h, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} o{tuple(o.shape)}")
    if lse is not None and (lse.shape != (b, h, nq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [batch, heads, seqlen_q] tensor")
    p = FwdParams()
    p.q, p.k, p.v, p.o, p.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    p.qkv_dtype, p.o_dtype = _code(q), _code(o)
    p.batch, p.seqlen_q, p.seqlen_k, p.heads, p.head_dim = b, nq, nk, h, d
    p.q_stride = _I64x3(*q.stride()[:3])
    p.k_stride = _I64x3(*k.stride()[:3])
    p.v_stride = _I64x3(*v.stride()[:3])
    p.o_stride = _I64x3(*o.stride()[:3])
    p.softmax_scale = _default_scale(d, softmax_scale)
    p.causal, p.window = int(bool(causal)), int(window)
    p.q_descale, p.k_descale, p.v_descale = (float(x) for x in descale)
    _set_dropout(p, dropout_p, seed, offset)
    return p


def fa_check_fwd(params: FwdParams) -> int:
    return lib().fa_check_fwd(ctypes.byref(params))


def fa_fwd(q, k, v, causal=False, window=0, softmax_scale=None, out=None, lse=None,
           return_lse=True, descale=(1.0, 1.0, 1.0), dropout_p=0.0, seed=None, offset=0):
    """O (and LSE) of exact attention; q [B,Nq,H,d], k/v [B,Nk,H,d] on the GPU.

    bf16 in -> bf16 out, fp32 -> fp32, float8_e4m3fn (with per-tensor
    ``descale`` = (q, k, v)) -> bf16.  ``softmax_scale`` None means 1/sqrt(d).
    ``dropout_p`` > 0 (bf16): dropout of the probabilities from the Philox
    stream of (``seed``, ``offset``); pass the same to ``fa_bwd``.
    """
    odt = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    b, nq, h, d = q.shape
    if out is None:
        out = torch.empty((b, nq, h, d), dtype=odt, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    p = make_fwd_params(q, k, v, out, lse, causal, window, softmax_scale, descale, dropout_p, seed, offset)
    _same_gpu(q, k=k, v=v, out=out, lse=lse)
    _raise(lib().fa_fwd(ctypes.byref(p), _stream()))
    return (out, lse) if return_lse else out


def make_varlen_params(q, k, v, o, lse, cu_seqlens, max_seqlen, causal=False, window=0, softmax_scale=None,
                       descale=(1.0, 1.0, 1.0), dropout_p=0.0, seed=None, offset=0):
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 3:
            raise ValueError(f"{n} must be [total_tokens, heads, head_dim] (got {tuple(t.shape)})")
        _check_last_dim(n, t)
    if _code(q) != _code(k) or _code(q) != _code(v):
        raise ValueError("Input and output tensors must have the same dtype (q, k, v differ)")
    total, h, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or o.shape != q.shape:
        raise ValueError("q, k, v, o must all be [total_tokens, heads, head_dim]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    if lse is not None and (lse.shape != (h, total) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    p = VarlenFwdParams()
    p.q, p.k, p.v, p.o, p.lse, p.cu_seqlens = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens)
    p.qkv_dtype, p.o_dtype = _code(q), _code(o)
    p.num_seqs, p.total_tokens, p.max_seqlen = cu_seqlens.numel() - 1, total, int(max_seqlen)
    p.heads, p.head_dim = h, d
    p.q_stride = _I64x2(*q.stride()[:2])
    p.k_stride = _I64x2(*k.stride()[:2])
    p.v_stride = _I64x2(*v.stride()[:2])
    p.o_stride = _I64x2(*o.stride()[:2])
    p.softmax_scale = _default_scale(d, softmax_scale)
    p.causal, p.window = int(bool(causal)), int(window)
    p.q_descale, p.k_descale, p.v_descale = (float(x) for x in descale)
    _set_dropout(p, dropout_p, seed, offset)
    return p


def fa_check_varlen_fwd(params: VarlenFwdParams) -> int:
    return lib().fa_check_varlen_fwd(ctypes.byref(params))


def fa_varlen_fwd(q, k, v, cu_seqlens, max_seqlen, causal=False, window=0, softmax_scale=None, out=None,
                  lse=None, return_lse=True, descale=(1.0, 1.0, 1.0), dropout_p=0.0, seed=None, offset=0):
    """Packed variable-length forward: q/k/v [total, H, d], int32 cu_seqlens [nseq+1]."""
    odt = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    total, h, d = q.shape
    if out is None:
        out = torch.empty((total, h, d), dtype=odt, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((h, total), dtype=torch.float32, device=q.device)
    p = make_varlen_params(q, k, v, out, lse, cu_seqlens, max_seqlen, causal, window, softmax_scale, descale,
                           dropout_p, seed, offset)
    _same_gpu(q, k=k, v=v, out=out, lse=lse, cu_seqlens=cu_seqlens)
    _raise(lib().fa_varlen_fwd(ctypes.byref(p), _stream()))
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def make_bwd_params(dout, q, k, v, o, lse, dq, dk, dv, causal=False, window=0, softmax_scale=None,
                    deterministic=False, dropout_p=0.0, seed=None, offset=0):
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dim() != 4:
            raise ValueError(f"{n} must be [batch, seqlen, heads, head_dim] (got {tuple(t.shape)})")
        _check_last_dim(n, t)
    codes = {_code(t) for t in (q, k, v, o, dout)}
    if len(codes) != 1:
        raise ValueError("Input and output tensors must have the same dtype (q, k, v, o, dout differ)")
    if dq.dtype != dk.dtype or dq.dtype != dv.dtype:
        raise ValueError("dq, dk, dv must share one dtype")
    b, nq, h, d = q.shape
    nk = k.shape[1]
    if lse.shape != (b, h, nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [batch, heads, seqlen_q] tensor")
    p = BwdParams()
    p.q, p.k, p.v, p.o, p.dout, p.lse = (_ptr(t) for t in (q, k, v, o, dout, lse))
    p.dq, p.dk, p.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    p.qkv_dtype, p.grad_dtype = _code(q), _code(dq)
    p.batch, p.seqlen_q, p.seqlen_k, p.heads, p.head_dim = b, nq, nk, h, d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(p, f"{name}_stride", _I64x3(*t.stride()[:3]))
    p.softmax_scale = _default_scale(d, softmax_scale)
    p.causal, p.window, p.deterministic = int(bool(causal)), int(window), int(bool(deterministic))
    _set_dropout(p, dropout_p, seed, offset)
    return p


def fa_check_bwd(params: BwdParams) -> int:
    return lib().fa_check_bwd(ctypes.byref(params))


def fa_bwd_workspace_bytes(params: BwdParams) -> int:
    return int(lib().fa_bwd_workspace_bytes(ctypes.byref(params)))


def fa_bwd(dout, q, k, v, o, lse, causal=False, window=0, softmax_scale=None, deterministic=False,
           grad_dtype=torch.float32, dq=None, dk=None, dv=None, dropout_p=0.0, seed=None, offset=0):
    """dq, dk, dv of exact attention, recomputing P from the forward's LSE."""
    if dq is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    p = make_bwd_params(dout, q, k, v, o, lse, dq, dk, dv, causal, window, softmax_scale, deterministic,
                        dropout_p, seed, offset)
    _same_gpu(q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    _raise(lib().fa_check_bwd(ctypes.byref(p)))
    nbytes = fa_bwd_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _raise(lib().fa_bwd(ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes), _stream()))
    return dq, dk, dv


def fa_bwd_noalloc(dout, q, k, v, o, lse, dq, dk, dv, causal=False, window=0, softmax_scale=None,
                   deterministic=False, dropout_p=0.0, seed=None, offset=0):
    """fa_bwd with the caller's dq, dk, dv and no allocation at all: the
    library's static device scratch replaces the workspace."""
    p = make_bwd_params(dout, q, k, v, o, lse, dq, dk, dv, causal, window, softmax_scale, deterministic,
                        dropout_p, seed, offset)
    _same_gpu(q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    _raise(lib().fa_bwd_noalloc(ctypes.byref(p), _stream()))
    return dq, dk, dv


def make_varlen_bwd_params(dout, q, k, v, o, lse, dq, dk, dv, cu_seqlens, max_seqlen, causal=False, window=0,
                           softmax_scale=None, deterministic=False, dropout_p=0.0, seed=None, offset=0):
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.dim() != 3:
            raise ValueError(f"{n} must be [total_tokens, heads, head_dim] (got {tuple(t.shape)})")
        _check_last_dim(n, t)
    codes = {_code(t) for t in (q, k, v, o, dout)}
    if len(codes) != 1:
        raise ValueError("Input and output tensors must have the same dtype (q, k, v, o, dout differ)")
    if dq.dtype != dk.dtype or dq.dtype != dv.dtype:
        raise ValueError("dq, dk, dv must share one dtype")
    total, h, d = q.shape
    for t in (k, v, o, dout, dq, dk, dv):
        if t.shape != q.shape:
            raise ValueError("q, k, v, o, dout, dq, dk, dv must all be [total_tokens, heads, head_dim]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    if lse.shape != (h, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    p = VarlenBwdParams()
    p.q, p.k, p.v, p.o, p.dout, p.lse = (_ptr(t) for t in (q, k, v, o, dout, lse))
    p.dq, p.dk, p.dv, p.cu_seqlens = _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens)
    p.qkv_dtype, p.grad_dtype = _code(q), _code(dq)
    p.num_seqs, p.total_tokens, p.max_seqlen = cu_seqlens.numel() - 1, total, int(max_seqlen)
    p.heads, p.head_dim = h, d
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        setattr(p, f"{name}_stride", _I64x2(*t.stride()[:2]))
    p.softmax_scale = _default_scale(d, softmax_scale)
    p.causal, p.window, p.deterministic = int(bool(causal)), int(window), int(bool(deterministic))
    _set_dropout(p, dropout_p, seed, offset)
    return p


def fa_check_varlen_bwd(params: VarlenBwdParams) -> int:
    return lib().fa_check_varlen_bwd(ctypes.byref(params))


def fa_varlen_bwd_workspace_bytes(params: VarlenBwdParams) -> int:
    return int(lib().fa_varlen_bwd_workspace_bytes(ctypes.byref(params)))


def fa_varlen_bwd(dout, q, k, v, o, lse, cu_seqlens, max_seqlen, causal=False, window=0, softmax_scale=None,
                  deterministic=False, grad_dtype=torch.float32, dq=None, dk=None, dv=None, dropout_p=0.0, seed=None,
                  offset=0):
    """dq, dk, dv of the packed variable-length forward (q/k/v [total, H, d], lse [H, total])."""
    if dq is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    p = make_varlen_bwd_params(dout, q, k, v, o, lse, dq, dk, dv, cu_seqlens, max_seqlen, causal, window,
                               softmax_scale, deterministic, dropout_p, seed, offset)
    _same_gpu(q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, cu_seqlens=cu_seqlens)
    _raise(lib().fa_check_varlen_bwd(ctypes.byref(p)))
    nbytes = fa_varlen_bwd_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _raise(lib().fa_varlen_bwd(ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes),
                               _stream()))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# merge of partial results
# ---------------------------------------------------------------------------
def make_merge_params(o_parts, lse_parts, o, lse):
    if o_parts.dim() != 5:
        raise ValueError(f"o_parts must be [parts, batch, seqlen, heads, head_dim] (got {tuple(o_parts.shape)})")
    _check_last_dim("o_parts", o_parts)
    _check_last_dim("o", o)
    n_p, b, n, h, d = o_parts.shape
    if o.shape != (b, n, h, d):
        raise ValueError("o must be [batch, seqlen, heads, head_dim] of o_parts")
    if lse_parts.shape != (n_p, b, h, n) or lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous float32 [parts, batch, heads, seqlen] tensor")
    if lse is not None and (lse.shape != (b, h, n) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [batch, heads, seqlen] tensor")
    p = MergeParams()
    p.o_parts, p.lse_parts, p.o, p.lse = _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse)
    p.parts_dtype, p.o_dtype = _code(o_parts), _code(o)
    p.num_parts, p.batch, p.seqlen, p.heads, p.head_dim = n_p, b, n, h, d
    p.parts_stride = _I64x4(*o_parts.stride()[:4])
    p.o_stride = _I64x3(*o.stride()[:3])
    return p


def fa_check_merge(params: MergeParams) -> int:
    return lib().fa_check_merge(ctypes.byref(params))


def fa_merge(o_parts, lse_parts, out=None, lse=None, out_dtype=None, return_lse=True):
    """Combine partial results over disjoint key subsets: o_parts [P, B, N, H, d]
    (fp32 or bf16), lse_parts [P, B, H, N] -> O [B, N, H, d], LSE [B, H, N]."""
    n_p, b, n, h, d = o_parts.shape
    if out is None:
        out = torch.empty((b, n, h, d), dtype=out_dtype or o_parts.dtype, device=o_parts.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=o_parts.device)
    p = make_merge_params(o_parts, lse_parts, out, lse)
    _same_gpu(o_parts, lse_parts=lse_parts, out=out, lse=lse)
    _raise(lib().fa_merge(ctypes.byref(p), _stream()))
    return (out, lse) if return_lse else out


# ---------------------------------------------------------------------------
# KV-cache decode
# ---------------------------------------------------------------------------
def make_kvcache_params(q, k_cache, v_cache, k_new, v_new, cache_seqlens, o, lse, causal=False, window=0,
                        softmax_scale=None, num_splits=0, block_table=None):
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{n} must be [batch, seqlen, heads, head_dim] (got {tuple(t.shape)})")
        _check_last_dim(n, t)
    if (k_new is None) != (v_new is None):
        raise ValueError("k and v must be given together")
    tensors = [q, k_cache, v_cache] + ([k_new, v_new] if k_new is not None else [])
    if len({_code(t) for t in tensors}) != 1:
        raise ValueError("Input and output tensors must have the same dtype (q, caches, new k/v differ)")
    b, nq, h, d = q.shape
    if block_table is None:
        lmax = k_cache.shape[1]
        if k_cache.shape != (b, lmax, h, d) or v_cache.shape != (b, lmax, h, d):
            raise ValueError("k_cache, v_cache must be [batch, cache_len, heads, head_dim] matching q")
    else:
        nb, page = k_cache.shape[:2]
        if k_cache.shape != (nb, page, h, d) or v_cache.shape != (nb, page, h, d):
            raise ValueError("paged k_cache, v_cache must be [num_blocks, page_block_size, heads, head_dim]")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != b \
                or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [batch, max_blocks_per_seq] tensor")
        lmax = block_table.shape[1] * page
    if k_new is not None and (k_new.shape != q.shape or v_new.shape != q.shape):
        raise ValueError("k, v must have q's shape [batch, seqlen_q, heads, head_dim]")
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    if cache_seqlens.dtype != torch.int32 or cache_seqlens.shape != (b,) or not cache_seqlens.is_contiguous():
        raise ValueError("cache_seqlens must be a contiguous int32 [batch] tensor")
    if lse is not None and (lse.shape != (b, h, nq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [batch, heads, seqlen_q] tensor")
    p = KvcacheParams()
    p.q, p.k_cache, p.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    p.k_new, p.v_new = _ptr(k_new), _ptr(v_new)
    p.cache_seqlens, p.o, p.lse = _ptr(cache_seqlens), _ptr(o), _ptr(lse)
    p.qkv_dtype = _code(q)
    p.batch, p.seqlen_q, p.cache_len, p.heads, p.head_dim = b, nq, lmax, h, d
    p.q_stride = _I64x3(*q.stride()[:3])
    p.kc_stride = _I64x3(*k_cache.stride()[:3])
    p.vc_stride = _I64x3(*v_cache.stride()[:3])
    if k_new is not None:
        p.kn_stride = _I64x3(*k_new.stride()[:3])
        p.vn_stride = _I64x3(*v_new.stride()[:3])
    p.o_stride = _I64x3(*o.stride()[:3])
    p.softmax_scale = _default_scale(d, softmax_scale)
    p.causal, p.window, p.num_splits = int(bool(causal)), int(window), int(num_splits)
    if block_table is not None:
        p.block_table = _ptr(block_table)
        p.page_block_size, p.max_blocks_per_seq = k_cache.shape[1], block_table.shape[1]
    return p


def fa_check_kvcache(params: KvcacheParams) -> int:
    return lib().fa_check_kvcache(ctypes.byref(params))


def fa_kvcache_workspace_bytes(params: KvcacheParams) -> int:
    return int(lib().fa_kvcache_workspace_bytes(ctypes.byref(params)))


def fa_fwd_kvcache(q, k_cache, v_cache, k=None, v=None, cache_seqlens=0, causal=False, window=0,
                   softmax_scale=None, num_splits=0, out=None, lse=None, return_lse=True, block_table=None):
    """One decoding step against a KV cache (the caches are updated in place
    when k, v are given).  cache_seqlens: an int for every batch entry, or an
    int32 [batch] tensor on the device.  block_table (int32 [batch,
    max_blocks]) makes k_cache, v_cache paged: [num_blocks, page, H, d]."""
    b, nq, h, d = q.shape
    cap = k_cache.shape[1] if block_table is None else block_table.shape[1] * k_cache.shape[1]
    if isinstance(cache_seqlens, int):
        if cache_seqlens < 0 or cache_seqlens + (nq if k is not None else 0) > cap:
            raise ValueError(f"cache_seqlens={cache_seqlens} does not fit cache_len={cap}")
        cache_seqlens = torch.full((b,), cache_seqlens, dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    p = make_kvcache_params(q, k_cache, v_cache, k, v, cache_seqlens, out, lse, causal, window, softmax_scale,
                            num_splits, block_table)
    _same_gpu(q, k_cache=k_cache, v_cache=v_cache, k=k, v=v, cache_seqlens=cache_seqlens, out=out, lse=lse,
              block_table=block_table)
    _raise(lib().fa_check_kvcache(ctypes.byref(p)))
    nbytes = fa_kvcache_workspace_bytes(p)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _raise(lib().fa_fwd_kvcache(ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes), _stream()))
    return (out, lse) if return_lse else out
