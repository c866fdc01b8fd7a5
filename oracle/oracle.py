"""Python access to the fp64 CPU oracle (oracle/attention.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg -- never by the product path.

Every function follows the plain definition of attention documented at the top
of attention.c (safe softmax of the scaled, masked scores; LSE = m + ln l; an
empty row gives O = 0, LSE = -inf), evaluated in double precision.
"""
import ctypes
import math
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")
_DTYPE_CODE = {torch.float16: 0, torch.bfloat16: 1}

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _bits(t):
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor as a contiguous uint16 array."""
    if t.dtype not in _DTYPE_CODE:
        raise TypeError(f"oracle takes fp16/bf16 tensors, got {t.dtype}")
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


class Oracle:
    """One loaded copy of the oracle library (a path lets tests load variants)."""

    def __init__(self, path=DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is not built; run oracle/build.py")
        lib = ctypes.CDLL(path)
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [
            _u16p, _u16p, _u16p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_int64,
            _f64p, _f64p, ctypes.c_int]
        lib.oracle_attention_varlen.restype = ctypes.c_int
        lib.oracle_attention_varlen.argtypes = [
            _u16p, _u16p, _u16p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p,
            ctypes.c_int, ctypes.c_float, _i64p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int]
        lib.oracle_attention_bwd.restype = ctypes.c_int
        lib.oracle_attention_bwd.argtypes = [
            _u16p, _u16p, _u16p, _u16p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            _i64p, ctypes.c_int64, _i64p, ctypes.c_int64, _f64p, _f64p, _f64p, ctypes.c_int]
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_combine.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       _f64p, _f64p]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        self.lib = lib
        self.path = path

    # -- decoders ---------------------------------------------------------
    def decode(self, bits, dtype):
        f = self.lib.oracle_decode_bf16 if dtype == torch.bfloat16 else self.lib.oracle_decode_f16
        return np.array([f(int(b)) for b in np.asarray(bits, dtype=np.uint16).ravel()])

    # -- attention --------------------------------------------------------
    def attention(self, q, k, v, causal, scale, rows=None, key_range=None, nthreads=None):
        """fp64 attention of [B,H,Nq,d] queries against [B,H,Nk,d] keys/values.

        rows: optional flat row indices (b*H + h)*Nq + i; then o is [len(rows), d]
        and lse is [len(rows)], otherwise o is [B,H,Nq,d] and lse [B,H,Nq].
        key_range: optional (begin, end) restricting the keys (split-KV partials).
        """
        if q.dtype != k.dtype or q.dtype != v.dtype:
            raise TypeError("q, k, v must share a dtype")
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
            raise ValueError("k and v must be [B, H, Nk, d] matching q")
        qb, kb, vb = _bits(q), _bits(k), _bits(v)
        kr = (0, Nk) if key_range is None else key_range
        if rows is None:
            nrows = B * H * Nq
            rows_arr = None
            o = np.empty((nrows, d), dtype=np.float64)
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nrows = rows_arr.size
            o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(
            _ptr(qb, _u16p), _ptr(kb, _u16p), _ptr(vb, _u16p), _DTYPE_CODE[q.dtype],
            B, H, Nq, Nk, d, int(bool(causal)), float(scale), int(kr[0]), int(kr[1]),
            _ptr(rows_arr, _i64p) if rows_arr is not None else None, nrows,
            _ptr(o, _f64p), _ptr(lse, _f64p), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_attention_rows failed ({rc})")
        if rows is None:
            return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)
        return o, lse

    # -- backward -------------------------------------------------------------
    def attention_bwd(self, q, k, v, dout, causal, scale, q_rows=None, k_rows=None, nthreads=None):
        """fp64 gradients dQ, dK, dV of attention for the upstream gradient dout
        (Ringi, "Lecture 25", section 3.3, with the scale carried through).

        q, dout [B,H,Nq,d]; k, v [B,H,Nk,d].  q_rows (flat (b*H+h)*Nq + i) and
        k_rows (flat (b*H+h)*Nk + j) select rows; then dq is [len(q_rows), d] and
        dk, dv [len(k_rows), d], otherwise full [B,H,N,d] arrays.
        """
        if not (q.dtype == k.dtype == v.dtype == dout.dtype):
            raise TypeError("q, k, v, dout must share a dtype")
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d) or tuple(dout.shape) != tuple(q.shape):
            raise ValueError("k, v must be [B,H,Nk,d] and dout [B,H,Nq,d]")
        bits = [_bits(t) for t in (q, k, v, dout)]
        qr = None if q_rows is None else np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64))
        kr = None if k_rows is None else np.ascontiguousarray(np.asarray(k_rows, dtype=np.int64))
        n_q = B * H * Nq if qr is None else qr.size
        n_k = B * H * Nk if kr is None else kr.size
        dq = np.empty((max(n_q, 1), d), dtype=np.float64)
        dk = np.empty((max(n_k, 1), d), dtype=np.float64)
        dv = np.empty((max(n_k, 1), d), dtype=np.float64)
        rc = self.lib.oracle_attention_bwd(
            *(_ptr(b, _u16p) for b in bits), _DTYPE_CODE[q.dtype], B, H, Nq, Nk, d, int(bool(causal)),
            float(scale), _ptr(qr, _i64p) if qr is not None else None, n_q,
            _ptr(kr, _i64p) if kr is not None else None, n_k,
            _ptr(dq, _f64p), _ptr(dk, _f64p), _ptr(dv, _f64p), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
        dq, dk, dv = dq[:n_q], dk[:n_k], dv[:n_k]
        if qr is None:
            dq = dq.reshape(B, H, Nq, d)
        if kr is None:
            dk, dv = dk.reshape(B, H, Nk, d), dv.reshape(B, H, Nk, d)
        return dq, dk, dv

    # -- grouped K/V heads in the [B, H, N, d] layout ----------------------
    @staticmethod
    def expand_kv_heads(t, H):
        """[B, H_kv, N, d] -> [B, H, N, d]: K/V head g serves the H // H_kv
        consecutive query heads g*G .. g*G + G-1 (KingOfEgg, "Flash Attention (4)",
        section 5: K/V indexed by head group)."""
        H_kv = t.shape[1]
        if H % H_kv != 0:
            raise ValueError("H_kv must divide H")
        return t.repeat_interleave(H // H_kv, dim=1).contiguous()

    def attention_gqa(self, q, k, v, causal, scale, rows=None, key_range=None, nthreads=None):
        """attention() with k, v [B, H_kv, Nk, d]: query head h reads K/V head h // (H // H_kv)."""
        H = q.shape[1]
        return self.attention(q, self.expand_kv_heads(k, H), self.expand_kv_heads(v, H), causal, scale,
                              rows=rows, key_range=key_range, nthreads=nthreads)

    # -- packed variable-length sequences, grouped K/V heads -------------
    def attention_bwd_gqa(self, q, k, v, dout, causal, scale, q_rows=None, k_rows=None, nthreads=None):
        """attention_bwd() with k, v [B, H_kv, Nk, d] shared by groups of query heads.

        A K/V head enters the loss through each of its G = H // H_kv query heads, so
        by the chain rule its dK (dV) is the sum of the per-query-head dK (dV) that
        attention_bwd gives on the expanded heads (KingOfEgg, "Flash Attention (4)",
        section 5: K/V indexed by head group).  k_rows are flat (b*H_kv + hk)*Nk + j;
        dq and q_rows are as in attention_bwd.
        """
        B, H, Nq, d = q.shape
        H_kv, Nk = k.shape[1], k.shape[2]
        if H % H_kv != 0:
            raise ValueError("H_kv must divide H")
        G = H // H_kv
        ke, ve = self.expand_kv_heads(k, H), self.expand_kv_heads(v, H)
        if k_rows is None:
            dq, dk, dv = self.attention_bwd(q, ke, ve, dout, causal, scale, q_rows=q_rows, nthreads=nthreads)
            return dq, dk.reshape(B, H_kv, G, Nk, d).sum(axis=2), dv.reshape(B, H_kv, G, Nk, d).sum(axis=2)
        kr = np.asarray(k_rows, dtype=np.int64)
        bh, j = kr // Nk, kr % Nk
        b, hk = bh // H_kv, bh % H_kv
        # the G expanded rows of each selected K/V row, group member fastest
        er = (((b * H + hk * G)[:, None] + np.arange(G)[None, :]) * Nk + j[:, None]).reshape(-1)
        dq, dk, dv = self.attention_bwd(q, ke, ve, dout, causal, scale, q_rows=q_rows, k_rows=er,
                                        nthreads=nthreads)
        return dq, dk.reshape(-1, G, d).sum(axis=1), dv.reshape(-1, G, d).sum(axis=1)

    def attention_bwd_varlen(self, q, k, v, dout, cu_seqlens_q, cu_seqlens_k, causal, scale, nthreads=None):
        """Gradients for packed variable-length sequences: q, dout [total_q, H, d];
        k, v [total_k, H_kv, d]; sequence b owns query rows cu_q[b]..cu_q[b+1] and key
        rows cu_k[b]..cu_k[b+1] and sees nothing else (KingOfEgg, "Flash Attention
        (4)", section 5: per-sequence offsets; causal bottom-right within a sequence).
        Sequences never interact, so each is attention_bwd_gqa on its own rows; a
        query with no key gets dq = 0 and a key no query sees dk = dv = 0.  Returns
        fp64 dq [total_q, H, d], dk, dv [total_k, H_kv, d]."""
        total_q, H, d = q.shape
        total_k, H_kv = k.shape[0], k.shape[1]
        cq, ck = np.asarray(cu_seqlens_q, dtype=np.int64), np.asarray(cu_seqlens_k, dtype=np.int64)
        dq = np.zeros((total_q, H, d))
        dk = np.zeros((total_k, H_kv, d))
        dv = np.zeros((total_k, H_kv, d))
        for b in range(len(cq) - 1):
            q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
            if q1 == q0 or k1 == k0:
                continue
            head_major = lambda t, a, z: t[a:z].permute(1, 0, 2).unsqueeze(0).contiguous()
            gq, gk, gv = self.attention_bwd_gqa(head_major(q, q0, q1), head_major(k, k0, k1), head_major(v, k0, k1),
                                                head_major(dout, q0, q1), causal, scale, nthreads=nthreads)
            dq[q0:q1] = gq[0].transpose(1, 0, 2)
            dk[k0:k1] = gk[0].transpose(1, 0, 2)
            dv[k0:k1] = gv[0].transpose(1, 0, 2)
        return dq, dk, dv

    def attention_varlen(self, q, k, v, cu_seqlens_q, cu_seqlens_k, causal, scale, rows=None,
                         nthreads=None):
        """fp64 attention of packed sequences: q [total_q, H, d] against k, v
        [total_k, H_kv, d], sequence b spanning tokens [cu[b], cu[b+1]) of each;
        query head h reads K/V head h // (H // H_kv).

        rows: optional flat indices token*H + h; then o is [len(rows), d] and lse
        [len(rows)], otherwise o is [total_q, H, d] and lse [H, total_q].
        """
        if q.dtype != k.dtype or q.dtype != v.dtype:
            raise TypeError("q, k, v must share a dtype")
        total_q, H, d = q.shape
        total_k, H_kv = k.shape[0], k.shape[1]
        if tuple(k.shape) != (total_k, H_kv, d) or tuple(v.shape) != (total_k, H_kv, d):
            raise ValueError("k and v must be [total_k, H_kv, d] matching q")
        cq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
        ck = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int32))
        B = cq.size - 1
        if ck.size != B + 1 or B < 1 or cq[-1] != total_q or ck[-1] != total_k:
            raise ValueError("cu_seqlens must hold B+1 offsets ending at total_q / total_k")
        qb, kb, vb = _bits(q), _bits(k), _bits(v)
        if rows is None:
            rows_arr = None
            nrows = total_q * H
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nrows = rows_arr.size
        o = np.empty((nrows, d), dtype=np.float64)
        lse = np.empty((nrows,), dtype=np.float64)
        rc = self.lib.oracle_attention_varlen(
            _ptr(qb, _u16p), _ptr(kb, _u16p), _ptr(vb, _u16p), _DTYPE_CODE[q.dtype],
            B, H, H_kv, d, _ptr(cq, _i32p), _ptr(ck, _i32p), int(bool(causal)), float(scale),
            _ptr(rows_arr, _i64p) if rows_arr is not None else None, nrows,
            _ptr(o, _f64p), _ptr(lse, _f64p), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError(f"oracle_attention_varlen failed ({rc})")
        if rows is None:
            return o.reshape(total_q, H, d), lse.reshape(total_q, H).T.copy()
        return o, lse

    # -- paged K/V cache ---------------------------------------------------
    @staticmethod
    def gather_pages(cache, block_table, seqlens):
        """The keys of a paged cache in sequence order, token-major: for sequence
        b and t = 0 .. len_b - 1, row t % page_size of physical page
        block_table[b][t // page_size] (the page-table indirection the pages pose
        for a cache split into non-contiguous pages: Ringi, "Lecture 25", section
        8.3, the PagedAttention question).  cache [num_pages, page_size, H_kv, d]
        -> [sum(len_b), H_kv, d]."""
        page_size = cache.shape[1]
        table = np.asarray(block_table, dtype=np.int64)
        rows = []
        for b in range(table.shape[0]):
            for t in range(int(seqlens[b])):
                rows.append(cache[int(table[b, t // page_size]), t % page_size])
        if not rows:
            return cache.new_empty((0,) + tuple(cache.shape[2:]))
        return torch.stack(rows).contiguous()

    def attention_paged(self, q, k_cache, v_cache, block_table, seqlens, scale, nthreads=None):
        """fp64 single-row decode over a paged cache: q [B, H, d] (one query row
        per sequence and head) against the len_b keys of sequence b gathered
        through its block table; query head h reads K/V head h // (H // H_kv).
        Returns o [B, H, d] and lse [B, H] (o = 0, lse = -inf for an empty
        sequence)."""
        B, H, d = q.shape
        lens = [int(n) for n in seqlens]
        k = self.gather_pages(k_cache, block_table, lens)
        v = self.gather_pages(v_cache, block_table, lens)
        if k.shape[0] == 0:
            return np.zeros((B, H, d)), np.full((B, H), -np.inf)
        cu_q = np.arange(B + 1, dtype=np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        o, lse = self.attention_varlen(q.contiguous(), k, v, cu_q, cu_k, False, scale, nthreads=nthreads)
        return o, lse.T.copy()

    def split_partials_paged(self, q, k_cache, v_cache, block_table, seqlens, scale, num_splits,
                             nthreads=None):
        """Per-split normalised partials of attention_paged: sequence b's keys are
        cut into num_splits chunks of ceil(len_b / num_splits) keys (the split rule
        of split_ranges applied per sequence).  Returns o_part [S, B, H, 1, d] and
        lse_part [S, B, H, 1]."""
        B, H, d = q.shape
        S = num_splits
        o_part = np.zeros((S, B, H, 1, d))
        lse_part = np.full((S, B, H, 1), -np.inf)
        for b in range(B):
            n = int(seqlens[b])
            if n == 0:
                continue
            kb = self.gather_pages(k_cache, block_table[b:b + 1], [n]).permute(1, 0, 2).unsqueeze(0).contiguous()
            vb = self.gather_pages(v_cache, block_table[b:b + 1], [n]).permute(1, 0, 2).unsqueeze(0).contiguous()
            ob, lb = self.split_partials(q[b:b + 1, :, None, :].contiguous(), kb, vb, False, scale, S,
                                         nthreads=nthreads)
            o_part[:, b] = ob[:, 0]
            lse_part[:, b] = lb[:, 0]
        return o_part, lse_part

    def split_partials_varlen(self, q, k, v, cu_seqlens_k, scale, num_splits, nthreads=None):
        """Per-split normalised partials of one query row per packed sequence (the
        varlen interface, Ringi, "Lecture 25", section 7, with split-KV for decode,
        LLM Infra Atlas, "FA2: parallelism", section 2): q [B, H, d]; sequence b's
        keys are rows [cu[b], cu[b+1]) of k, v [total_k, H_kv, d], cut into
        num_splits chunks of ceil(len_b / num_splits) keys (split_ranges applied
        per sequence, as for the paged cache).  Returns o_part [S, B, H, 1, d] and
        lse_part [S, B, H, 1]."""
        B, H, d = q.shape
        S = num_splits
        cu = [int(x) for x in cu_seqlens_k]
        if len(cu) != B + 1:
            raise ValueError("cu_seqlens_k must hold B + 1 offsets")
        o_part = np.zeros((S, B, H, 1, d))
        lse_part = np.full((S, B, H, 1), -np.inf)
        for b in range(B):
            lo, hi = cu[b], cu[b + 1]
            if hi == lo:
                continue
            kb = k[lo:hi].permute(1, 0, 2).unsqueeze(0).contiguous()
            vb = v[lo:hi].permute(1, 0, 2).unsqueeze(0).contiguous()
            ob, lb = self.split_partials(q[b:b + 1, :, None, :].contiguous(), kb, vb, False, scale, S,
                                         nthreads=nthreads)
            o_part[:, b] = ob[:, 0]
            lse_part[:, b] = lb[:, 0]
        return o_part, lse_part

    # -- split-KV ---------------------------------------------------------
    @staticmethod
    def split_ranges(Nk, num_splits):
        """Contiguous key chunks of ceil(Nk / S) keys; trailing splits may be empty."""
        chunk = -(-Nk // num_splits)
        return [(min(Nk, s * chunk), min(Nk, (s + 1) * chunk)) for s in range(num_splits)]

    def split_partials(self, q, k, v, causal, scale, num_splits, rows=None, nthreads=None):
        """Per-split normalised (O_s, LSE_s): attention restricted to each key chunk
        (k, v may carry fewer heads than q: grouped K/V heads)."""
        outs, lses = [], []
        attn = self.attention_gqa if k.shape[1] != q.shape[1] else self.attention
        for kr in self.split_ranges(k.shape[2], num_splits):
            o, l = attn(q, k, v, causal, scale, rows=rows, key_range=kr, nthreads=nthreads)
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)

    def combine(self, o_part, lse_part):
        """LSE-weighted merge of [S, ..., d] partials into [..., d] and [...]."""
        o_part = np.ascontiguousarray(np.asarray(o_part, dtype=np.float64))
        lse_part = np.ascontiguousarray(np.asarray(lse_part, dtype=np.float64))
        S, d = o_part.shape[0], o_part.shape[-1]
        rest = lse_part.shape[1:]
        R = int(np.prod(rest)) if rest else 1
        if o_part.shape[:-1] != lse_part.shape:
            raise ValueError("o_part must be lse_part's shape plus a trailing d")
        o = np.empty((R, d), dtype=np.float64)
        lse = np.empty((R,), dtype=np.float64)
        rc = self.lib.oracle_combine(_ptr(o_part, _f64p), _ptr(lse_part, _f64p), S, R, d,
                                     _ptr(o, _f64p), _ptr(lse, _f64p))
        if rc != 0:
            raise RuntimeError(f"oracle_combine failed ({rc})")
        return o.reshape(*rest, d), lse.reshape(rest)


_default = None


def get():
    """The oracle built from oracle/attention.c (loaded once)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


__all__ = ["Oracle", "get", "default_threads"]
