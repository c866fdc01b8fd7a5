"""Thin Python binding of libfa.so (include/fa.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, then their device pointers and the current HIP stream go to the C ABI.
Every step of the computation runs in the library's HIP kernels; there is no
fallback path.  PyTorch supplies device memory and streams.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_F16, FA_BF16 = 0, 1
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(6)
SYMBOLS = ("fa_fwd", "fa_fwd_gqa", "fa_fwd_varlen", "fa_splitkv_workspace_bytes", "fa_fwd_splitkv",
           "fa_fwd_splitkv_gqa", "fa_fwd_splitkv_paged", "fa_fwd_splitkv_varlen", "fa_splitkv_combine", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_bwd_gqa", "fa_bwd_gqa_noalloc", "fa_bwd_varlen", "fa_fwd_fp8", "fa_quantize_fp8", "fa_status_str")
_DTYPES = {torch.float16: FA_F16, torch.bfloat16: FA_BF16}
_lib = None


class FaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def lib():
    """Load libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run exact_attention_22_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.fa_fwd.restype = i
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        L.fa_fwd_gqa.restype = i
        L.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        L.fa_fwd_splitkv_gqa.restype = i
        L.fa_fwd_splitkv_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
        L.fa_fwd_varlen.restype = i
        L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
        L.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
        L.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_fwd_splitkv.restype = i
        L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.fa_fwd_splitkv_paged.restype = i
        L.fa_fwd_splitkv_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
        L.fa_fwd_splitkv_varlen.restype = i
        L.fa_fwd_splitkv_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        L.fa_splitkv_combine.restype = i
        L.fa_splitkv_combine.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i]
        L.fa_bwd.restype = i
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, i, f, i, vp]
        L.fa_bwd_gqa.restype = i
        L.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, i, i, f, i,
                                 vp]
        L.fa_bwd_gqa_noalloc.restype = i
        L.fa_bwd_gqa_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
        L.fa_bwd_varlen.restype = i
        L.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    i, i, i, i, i, i, i, i, i, f, i, vp]
        L.fa_fwd_fp8.restype = i
        L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        L.fa_quantize_fp8.restype = i
        L.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
        L.fa_status_str.restype = ctypes.c_char_p
        L.fa_status_str.argtypes = [i]
        _lib = L
    return _lib


def status_str(status):
    return lib().fa_status_str(status).decode()


def _check(status):
    if status != FA_OK:
        msg = status_str(status)
        if status == FA_ERR_HIP:
            raise FaError(status, msg)
        raise ValueError(f"{msg} (status {status})")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_tensor(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _qkv(q, k, v, grouped=False):
    """Pointers and sizes of [B, H, Nq, d] queries and [B, H_kv, Nk, d] keys/values
    (H_kv = H unless grouped)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk, H_kv = k.shape[2], k.shape[1]
    if not grouped and H_kv != H:
        raise ValueError("k and v must have q's H heads (fwd_gqa / fwd_splitkv_gqa take fewer)")
    if tuple(k.shape) != (B, H_kv, Nk, d) or tuple(v.shape) != (B, H_kv, Nk, d):
        raise ValueError("k and v must be [B, H_kv, Nk, d] with q's B and d")
    ptrs = [_dev_tensor(t, n, q.dtype) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    if grouped:
        return ptrs, (B, H, H_kv, Nq, Nk, d)
    return ptrs, (B, H, Nq, Nk, d)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """O, LSE of softmax(scale * Q K^T (+ causal mask)) V.  scale defaults to 1/sqrt(d)."""
    (qp, kp, vp), (B, H, Nq, Nk, d) = _qkv(q, k, v)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out must be [B, H, Nq, d] and lse [B, H, Nq]")
    op = _dev_tensor(out, "out", q.dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    _check(lib().fa_fwd(qp, kp, vp, op, lp, B, H, Nq, Nk, d, int(bool(causal)), _scale(scale, d),
                        _DTYPES[q.dtype], _stream(stream)))
    return out, lse


def fwd_gqa(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """fwd with K/V heads shared by groups of query heads: k, v [B, H_kv, Nk, d]."""
    (qp, kp, vp), (B, H, H_kv, Nq, Nk, d) = _qkv(q, k, v, grouped=True)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out must be [B, H, Nq, d] and lse [B, H, Nq]")
    op = _dev_tensor(out, "out", q.dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    _check(lib().fa_fwd_gqa(qp, kp, vp, op, lp, B, H, H_kv, Nq, Nk, d, int(bool(causal)), _scale(scale, d),
                            _DTYPES[q.dtype], _stream(stream)))
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=False,
               scale=None, out=None, lse=None, stream=None):
    """Packed variable-length sequences with grouped K/V heads.

    q [total_q, H, d], k and v [total_k, H_kv, d] (H_kv divides H), cu_seqlens_q
    and cu_seqlens_k int32 [B + 1] device tensors of cumulative offsets.  Returns
    O [total_q, H, d] and LSE [H, total_q] (fp32).  scale defaults to 1/sqrt(d).
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [total_q, H, d] and k, v [total_k, H_kv, d]")
    total_q, H, d = q.shape
    total_k, H_kv = k.shape[0], k.shape[1]
    if tuple(k.shape) != (total_k, H_kv, d) or tuple(v.shape) != (total_k, H_kv, d):
        raise ValueError("k and v must be [total_k, H_kv, d] with q's d")
    if cu_seqlens_q.dim() != 1 or tuple(cu_seqlens_k.shape) != tuple(cu_seqlens_q.shape):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.shape[0] - 1
    qp, kp, vp = (_dev_tensor(t, n, q.dtype) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    cqp = _dev_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    ckp = _dev_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    # rows of a sequence whose offsets break the contract are left unwritten by the
    # library; outputs allocated here start as O = 0, LSE = -inf (no visible key)
    out = torch.zeros_like(q) if out is None else out
    lse = torch.full((H, total_q), -math.inf, dtype=torch.float32, device=q.device) if lse is None else lse
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (H, total_q):
        raise ValueError("out must be [total_q, H, d] and lse [H, total_q]")
    op = _dev_tensor(out, "out", q.dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    _check(lib().fa_fwd_varlen(qp, kp, vp, op, lp, cqp, ckp, B, H, H_kv, total_q, total_k,
                               int(max_seqlen_q), int(max_seqlen_k), d, int(bool(causal)),
                               _scale(scale, d), _DTYPES[q.dtype], _stream(stream)))
    return out, lse


def workspace_bytes(B, H, Nq, d, num_splits):
    return int(lib().fa_splitkv_workspace_bytes(B, H, Nq, d, num_splits))


def fwd_splitkv(q, k, v, num_splits, causal=False, scale=None, o_part=None, lse_part=None, stream=None):
    """Per-split normalised partials: o_part [S,B,H,Nq,d] fp32, lse_part [S,B,H,Nq] fp32."""
    (qp, kp, vp), (B, H, Nq, Nk, d) = _qkv(q, k, v)
    S = int(num_splits)
    if o_part is None:
        o_part = torch.empty((S, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((S, B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (S, B, H, Nq, d) or tuple(lse_part.shape) != (S, B, H, Nq):
        raise ValueError("o_part must be [S, B, H, Nq, d] and lse_part [S, B, H, Nq]")
    opp = _dev_tensor(o_part, "o_part", torch.float32)
    lpp = _dev_tensor(lse_part, "lse_part", torch.float32)
    _check(lib().fa_fwd_splitkv(qp, kp, vp, opp, lpp, B, H, Nq, Nk, d, int(bool(causal)),
                                _scale(scale, d), S, _DTYPES[q.dtype], _stream(stream)))
    return o_part, lse_part


def fwd_splitkv_gqa(q, k, v, num_splits, causal=False, scale=None, o_part=None, lse_part=None, stream=None):
    """fwd_splitkv with grouped K/V heads: k, v [B, H_kv, Nk, d]."""
    (qp, kp, vp), (B, H, H_kv, Nq, Nk, d) = _qkv(q, k, v, grouped=True)
    S = int(num_splits)
    if o_part is None:
        o_part = torch.empty((S, B, H, Nq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((S, B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (S, B, H, Nq, d) or tuple(lse_part.shape) != (S, B, H, Nq):
        raise ValueError("o_part must be [S, B, H, Nq, d] and lse_part [S, B, H, Nq]")
    opp = _dev_tensor(o_part, "o_part", torch.float32)
    lpp = _dev_tensor(lse_part, "lse_part", torch.float32)
    _check(lib().fa_fwd_splitkv_gqa(qp, kp, vp, opp, lpp, B, H, H_kv, Nq, Nk, d, int(bool(causal)),
                                    _scale(scale, d), S, _DTYPES[q.dtype], _stream(stream)))
    return o_part, lse_part


def fwd_splitkv_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits, scale=None, o_part=None,
                      lse_part=None, stream=None):
    """Split-KV partials of one query row per sequence over a paged K/V cache.

    q [B, H, d]; k_cache, v_cache [num_pages, page_size, H_kv, d]; block_table
    int32 [B, max_pages] and seqlens_k int32 [B] on the device.  Returns o_part
    [S, B, H, 1, d] and lse_part [S, B, H, 1] (fp32) for splitkv_combine.
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, H, d] and the caches [num_pages, page_size, H_kv, d]")
    B, H, d = q.shape
    num_pages, page_size, H_kv = k_cache.shape[:3]
    if tuple(k_cache.shape) != (num_pages, page_size, H_kv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, H_kv, d] with q's d")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seqlens_k.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens_k [B]")
    max_pages = block_table.shape[1]
    qp, kp, vp = (_dev_tensor(t, n, q.dtype) for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")))
    btp = _dev_tensor(block_table, "block_table", torch.int32)
    slp = _dev_tensor(seqlens_k, "seqlens_k", torch.int32)
    S = int(num_splits)
    # a sequence whose length breaks the contract leaves its partials unwritten;
    # partials allocated here start as empty splits (O = 0, LSE = -inf)
    if o_part is None:
        o_part = torch.zeros((S, B, H, 1, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.full((S, B, H, 1), -math.inf, dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (S, B, H, 1, d) or tuple(lse_part.shape) != (S, B, H, 1):
        raise ValueError("o_part must be [S, B, H, 1, d] and lse_part [S, B, H, 1]")
    opp = _dev_tensor(o_part, "o_part", torch.float32)
    lpp = _dev_tensor(lse_part, "lse_part", torch.float32)
    _check(lib().fa_fwd_splitkv_paged(qp, kp, vp, btp, slp, opp, lpp, B, H, H_kv, d, page_size, max_pages,
                                      num_pages, _scale(scale, d), S, _DTYPES[q.dtype], _stream(stream)))
    return o_part, lse_part


def decode_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits=16, scale=None, stream=None,
                 o_part=None, lse_part=None):
    """fwd_splitkv_paged followed by the combine: O [B, H, 1, d], LSE [B, H, 1]."""
    o_part, lse_part = fwd_splitkv_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits, scale,
                                         o_part, lse_part, stream)
    return splitkv_combine(o_part, lse_part, q.dtype, stream=stream)


def fwd_splitkv_varlen(q, k, v, cu_seqlens_k, max_seqlen_k, num_splits, scale=None, o_part=None, lse_part=None,
                       stream=None):
    """Split-KV partials of one query row per packed sequence.

    q [B, H, d]; k, v [total_k, H_kv, d] with sequence b in rows
    [cu_seqlens_k[b], cu_seqlens_k[b+1]) (int32 [B + 1] on the device).  Returns
    o_part [S, B, H, 1, d] and lse_part [S, B, H, 1] (fp32) for splitkv_combine.
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [B, H, d] and k, v [total_k, H_kv, d]")
    B, H, d = q.shape
    total_k, H_kv = k.shape[:2]
    if tuple(k.shape) != (total_k, H_kv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [total_k, H_kv, d] with q's d")
    if tuple(cu_seqlens_k.shape) != (B + 1,):
        raise ValueError("cu_seqlens_k must be [B + 1]")
    qp, kp, vp = (_dev_tensor(t, n, q.dtype) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    cup = _dev_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    S = int(num_splits)
    # a sequence whose offsets break the contract leaves its partials unwritten;
    # partials allocated here start as empty splits (O = 0, LSE = -inf)
    if o_part is None:
        o_part = torch.zeros((S, B, H, 1, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.full((S, B, H, 1), -math.inf, dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (S, B, H, 1, d) or tuple(lse_part.shape) != (S, B, H, 1):
        raise ValueError("o_part must be [S, B, H, 1, d] and lse_part [S, B, H, 1]")
    opp = _dev_tensor(o_part, "o_part", torch.float32)
    lpp = _dev_tensor(lse_part, "lse_part", torch.float32)
    _check(lib().fa_fwd_splitkv_varlen(qp, kp, vp, cup, opp, lpp, B, H, H_kv, total_k, int(max_seqlen_k), d,
                                       _scale(scale, d), S, _DTYPES[q.dtype], _stream(stream)))
    return o_part, lse_part


def decode_varlen(q, k, v, cu_seqlens_k, max_seqlen_k, num_splits=16, scale=None, stream=None, o_part=None,
                  lse_part=None):
    """fwd_splitkv_varlen followed by the combine: O [B, H, 1, d], LSE [B, H, 1]."""
    o_part, lse_part = fwd_splitkv_varlen(q, k, v, cu_seqlens_k, max_seqlen_k, num_splits, scale, o_part,
                                          lse_part, stream)
    return splitkv_combine(o_part, lse_part, q.dtype, stream=stream)


def splitkv_combine(o_part, lse_part, dtype, out=None, lse=None, stream=None):
    """Merge split partials into O (dtype) and LSE (fp32)."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float16 or bfloat16, got {dtype}")
    if o_part.dim() != 5 or tuple(lse_part.shape) != tuple(o_part.shape[:4]):
        raise ValueError("o_part must be [S, B, H, Nq, d] and lse_part [S, B, H, Nq]")
    S, B, H, Nq, d = o_part.shape
    opp = _dev_tensor(o_part, "o_part", torch.float32)
    lpp = _dev_tensor(lse_part, "lse_part", torch.float32)
    out = torch.empty((B, H, Nq, d), dtype=dtype, device=o_part.device) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=o_part.device) if lse is None else lse
    if tuple(out.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out must be [B, H, Nq, d] and lse [B, H, Nq]")
    op = _dev_tensor(out, "out", dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    _check(lib().fa_splitkv_combine(opp, lpp, op, lp, B, H, Nq, d, S, _DTYPES[dtype], _stream(stream)))
    return out, lse


def bwd_workspace_bytes(B, H, Nq):
    return int(lib().fa_bwd_workspace_bytes(B, H, Nq))


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
        stream=None):
    """dQ, dK, dV for the upstream gradient dout, from the forward's inputs, o and lse.

    k and v may carry fewer heads than q (grouped K/V heads, [B, H_kv, Nk, d]): then
    fa_bwd_gqa runs, and dk and dv have k's shape and sum over each head's group."""
    grouped = k.dim() == 4 and q.dim() == 4 and k.shape[1] != q.shape[1]
    return _bwd(grouped, q, k, v, o, lse, dout, causal, scale, dq, dk, dv, workspace, stream)


def bwd_gqa(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
            stream=None):
    """bwd through fa_bwd_gqa whatever the head counts: k, v [B, H_kv, Nk, d]."""
    return _bwd(True, q, k, v, o, lse, dout, causal, scale, dq, dk, dv, workspace, stream)


def _bwd(grouped, q, k, v, o, lse, dout, causal, scale, dq, dk, dv, workspace, stream):
    if grouped:
        (qp, kp, vp), (B, H, H_kv, Nq, Nk, d) = _qkv(q, k, v, grouped=True)
    else:
        (qp, kp, vp), (B, H, Nq, Nk, d) = _qkv(q, k, v)
        H_kv = H
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o and dout must be [B, H, Nq, d] and lse [B, H, Nq]")
    opp = _dev_tensor(o, "o", q.dtype)
    gp = _dev_tensor(dout, "dout", q.dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(v.shape):
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    nbytes = bwd_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    wp = _dev_tensor(workspace, "workspace")
    ptrs = [_dev_tensor(t, n, q.dtype) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    nws = workspace.numel() * workspace.element_size()
    if grouped:
        _check(lib().fa_bwd_gqa(qp, kp, vp, opp, gp, lp, *ptrs, wp, nws, B, H, H_kv, Nq, Nk, d,
                                int(bool(causal)), _scale(scale, d), _DTYPES[q.dtype], _stream(stream)))
    else:
        _check(lib().fa_bwd(qp, kp, vp, opp, gp, lp, *ptrs, wp, nws, B, H, Nq, Nk, d, int(bool(causal)),
                            _scale(scale, d), _DTYPES[q.dtype], _stream(stream)))
    return dq, dk, dv


BWD_NOALLOC_MAX_ROWS = 1 << 20     # B * H * Nq limit of bwd_gqa_noalloc (FA_BWD_NOALLOC_MAX_ROWS)


def bwd_gqa_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, scale=None, stream=None):
    """fa_bwd_gqa_noalloc: bwd_gqa without a workspace (the library's fixed device
    scratch holds it), for callers that cannot allocate.  The caller passes the
    outputs dq, dk, dv; nothing is allocated here either.  B * H * Nq must not
    exceed BWD_NOALLOC_MAX_ROWS.  Calls overlapping in time on one GPU race."""
    (qp, kp, vp), (B, H, H_kv, Nq, Nk, d) = _qkv(q, k, v, grouped=True)
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o and dout must be [B, H, Nq, d] and lse [B, H, Nq]")
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(v.shape):
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    opp, gp = _dev_tensor(o, "o", q.dtype), _dev_tensor(dout, "dout", q.dtype)
    lp = _dev_tensor(lse, "lse", torch.float32)
    ptrs = [_dev_tensor(t, n, q.dtype) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _check(lib().fa_bwd_gqa_noalloc(qp, kp, vp, opp, gp, lp, *ptrs, B, H, H_kv, Nq, Nk, d, int(bool(causal)),
                                    _scale(scale, d), _DTYPES[q.dtype], _stream(stream)))
    return dq, dk, dv


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=False,
               scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of fwd_varlen: q, o, dout [total_q, H, d], k, v [total_k, H_kv, d],
    lse [H, total_q] as fwd_varlen returned it.  Returns dq, dk, dv shaped like q,
    k, v (dk, dv summed over each K/V head's group)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [total_q, H, d] and k, v [total_k, H_kv, d]")
    total_q, H, d = q.shape
    total_k, H_kv = k.shape[0], k.shape[1]
    if tuple(k.shape) != (total_k, H_kv, d) or tuple(v.shape) != (total_k, H_kv, d):
        raise ValueError("k and v must be [total_k, H_kv, d] with q's d")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (H, total_q):
        raise ValueError("o and dout must be [total_q, H, d] and lse [H, total_q]")
    if cu_seqlens_q.dim() != 1 or tuple(cu_seqlens_k.shape) != tuple(cu_seqlens_q.shape):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.shape[0] - 1
    qp, kp, vp, opp, gp = (_dev_tensor(t, n, q.dtype) for t, n in
                           ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")))
    lp = _dev_tensor(lse, "lse", torch.float32)
    cqp = _dev_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    ckp = _dev_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    # rows of a sequence whose offsets break the contract are left unwritten by the
    # library; gradients allocated here start at zero
    dq = torch.zeros_like(q) if dq is None else dq
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(v) if dv is None else dv
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(v.shape):
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    if workspace is None:
        workspace = torch.empty(bwd_workspace_bytes(1, H, total_q) // 4, dtype=torch.float32, device=q.device)
    wp = _dev_tensor(workspace, "workspace")
    ptrs = [_dev_tensor(t, n, q.dtype) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _check(lib().fa_bwd_varlen(qp, kp, vp, opp, gp, lp, *ptrs, cqp, ckp, wp,
                               workspace.numel() * workspace.element_size(), B, H, H_kv, total_q, total_k,
                               int(max_seqlen_q), int(max_seqlen_k), d, int(bool(causal)), _scale(scale, d),
                               _DTYPES[q.dtype], _stream(stream)))
    return dq, dk, dv


def decode(q, k, v, num_splits=16, causal=False, scale=None, stream=None, o_part=None, lse_part=None):
    """Split-KV forward followed by the combine, both on the same stream; k and v
    may carry fewer heads than q (grouped K/V heads)."""
    split = fwd_splitkv_gqa if k.dim() == 4 and q.dim() == 4 and k.shape[1] != q.shape[1] else fwd_splitkv
    o_part, lse_part = split(q, k, v, num_splits, causal, scale, o_part, lse_part, stream)
    return splitkv_combine(o_part, lse_part, q.dtype, stream=stream)


FP8_BLOCK = 128   # rows per Q scale and per K scale of fwd_fp8


def _codes(t, name):
    """uint8 (or float8_e4m3fn, viewed as bytes) GPU tensor -> pointer."""
    if isinstance(t, torch.Tensor) and t.dtype == getattr(torch, "float8_e4m3fn", None):
        t = t.view(torch.uint8)
    return _dev_tensor(t, name, torch.uint8)


def quantize_fp8(x, block_rows, out=None, descale=None, stream=None):
    """Per-block e4m3 quantization of x [G, N, d] (fp16/bf16): returns codes
    (uint8 [G, N, d]) and descale (fp32 [G, ceil(N / block_rows)])."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"x must be float16 or bfloat16, got {x.dtype}")
    if x.dim() != 3:
        raise ValueError("x must be [G, N, d]")
    G, N, d = x.shape
    nb = -(-N // int(block_rows))
    out = torch.empty((G, N, d), dtype=torch.uint8, device=x.device) if out is None else out
    descale = torch.empty((G, nb), dtype=torch.float32, device=x.device) if descale is None else descale
    if tuple(out.shape) != (G, N, d) or tuple(descale.shape) != (G, nb):
        raise ValueError("out must be [G, N, d] and descale [G, ceil(N / block_rows)]")
    _check(lib().fa_quantize_fp8(_dev_tensor(x, "x", x.dtype), _codes(out, "out"),
                                 _dev_tensor(descale, "descale", torch.float32), G, N, d, int(block_rows),
                                 _DTYPES[x.dtype], _stream(stream)))
    return out, descale


def fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal=False, scale=None, out=None, lse=None,
            stream=None):
    """FP8 forward: e4m3 codes q8 [B, H, Nq, 128], k8 and v8 [B, H_kv, Nk, 128];
    descales q [B, H, ceil(Nq/128)], k [B, H_kv, ceil(Nk/128)], v [B, H_kv] (fp32).
    Returns O (bf16 [B, H, Nq, 128]) and LSE (fp32 [B, H, Nq])."""
    if q8.dim() != 4 or k8.dim() != 4 or v8.dim() != 4:
        raise ValueError("q8, k8, v8 must be [B, H, N, d]")
    B, H, Nq, d = q8.shape
    H_kv, Nk = k8.shape[1], k8.shape[2]
    if tuple(k8.shape) != (B, H_kv, Nk, d) or tuple(v8.shape) != (B, H_kv, Nk, d):
        raise ValueError("k8 and v8 must be [B, H_kv, Nk, d] with q8's B and d")
    nq, nk = -(-Nq // FP8_BLOCK), -(-Nk // FP8_BLOCK)
    if (tuple(q_descale.shape) != (B, H, nq) or tuple(k_descale.shape) != (B, H_kv, nk)
            or tuple(v_descale.shape) != (B, H_kv)):
        raise ValueError("descales must be q [B, H, ceil(Nq/128)], k [B, H_kv, ceil(Nk/128)], v [B, H_kv]")
    ptrs = [_codes(t, n) for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8"))]
    dps = [_dev_tensor(t, n, torch.float32) for t, n in ((q_descale, "q_descale"), (k_descale, "k_descale"),
                                                         (v_descale, "v_descale"))]
    out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q8.device) if lse is None else lse
    if tuple(out.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("out must be [B, H, Nq, d] and lse [B, H, Nq]")
    op = _dev_tensor(out, "out", torch.bfloat16)
    lp = _dev_tensor(lse, "lse", torch.float32)
    _check(lib().fa_fwd_fp8(*ptrs, *dps, op, lp, B, H, H_kv, Nq, Nk, d, int(bool(causal)), _scale(scale, d),
                            _stream(stream)))
    return out, lse
