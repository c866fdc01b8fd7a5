"""Seeded synthetic workloads for the attention forward.

This module holds no attention arithmetic: it only names the workloads and draws
their Q/K/V from a seeded normal generator.  Both sides of every parity check (the
HIP library and the fp64 oracle) receive the exact same 16-bit patterns from here.

Workloads (Q, K, V iid N(0, 1), layout [B, H, N, d], scale = 1/sqrt(d)):
  tiny            B=1  H=1  Nq=Nk=128   d=64  fp16  non-causal
  prefill_d64     B=16 H=16 Nq=Nk=1024  d=64  fp16  non-causal
  causal_d128     B=4  H=16 Nq=Nk=2048  d=128 fp16  causal
  long_causal     B=1  H=32 Nq=Nk=8192  d=128 bf16  causal, values scaled by 0.5
  decode          B=8  H=32 Nq=1 Nk=32768 d=128 fp16 non-causal, 16 KV splits
  decode_gqa      as decode with the 32 query heads sharing H_kv=8 K/V heads
                  (K, V [B, 8, Nk, d])
  varlen_gqa      16 packed sequences, lengths log-uniform in [64, 8192] (seeded),
                  H=32 query heads sharing H_kv=8 K/V heads, d=128 bf16 causal,
                  Nq = Nk per sequence; layout [total, heads, d]
  decode_paged    as decode_gqa with K/V in a paged cache of 16-row pages
                  [num_pages, 16, H_kv, d], pages assigned by a seeded
                  permutation (a fragmented cache); q [B, H, d]
  decode_varlen   one query row per sequence over 16 packed sequences of keys,
                  lengths log-uniform in [512, 32768] (seeded), H=32 query heads
                  on H_kv=8 K/V heads, d=128 fp16, 16 splits per sequence;
                  q [B, H, d], K, V [total_k, H_kv, d]
These follow the shapes the pages benchmark (randn fp16, d in {64, 128},
N from 1K to 16K) -- no dataset is involved.
"""
from dataclasses import dataclass, replace
import math

import torch

F16 = torch.float16
BF16 = torch.bfloat16


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: torch.dtype
    causal: bool
    mult: float = 1.0        # the long-context workload draws N(0,1) * 0.5
    splits: int = 0          # > 0: decode through split-KV + combine
    seed: int = 42
    H_kv: int = 0            # K/V heads when grouped (0: H)
    seqlens: tuple = ()      # non-empty: packed layout with these lengths (queries = keys; with
                             # splits > 0, one query row per sequence and these key lengths)
    page_size: int = 0       # > 0: decode from a paged K/V cache with pages of this many rows

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def log_uniform_lengths(n, lo, hi, seed):
    """n sequence lengths drawn log-uniformly from [lo, hi] by a seeded generator."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(n, generator=g, dtype=torch.float64).tolist()
    return tuple(int(round(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u)


_VARLEN_LENS = log_uniform_lengths(16, 64, 8192, 47)
_DECODE_VARLEN_LENS = log_uniform_lengths(16, 512, 32768, 51)

WORKLOADS = [
    Workload("tiny", 1, 1, 128, 128, 64, F16, False, seed=42),
    Workload("prefill_d64", 16, 16, 1024, 1024, 64, F16, False, seed=43),
    Workload("causal_d128", 4, 16, 2048, 2048, 128, F16, True, seed=44),
    Workload("long_causal", 1, 32, 8192, 8192, 128, BF16, True, mult=0.5, seed=45),
    Workload("decode", 8, 32, 1, 32768, 128, F16, False, splits=16, seed=46),
    Workload("decode_gqa", 8, 32, 1, 32768, 128, F16, False, splits=16, seed=48, H_kv=8),
    Workload("decode_paged", 8, 32, 1, 32768, 128, F16, False, splits=16, seed=49, H_kv=8, page_size=16),
    Workload("varlen_gqa", len(_VARLEN_LENS), 32, max(_VARLEN_LENS), max(_VARLEN_LENS), 128, BF16, True,
             seed=47, H_kv=8, seqlens=_VARLEN_LENS),
    Workload("decode_varlen", len(_DECODE_VARLEN_LENS), 32, 1, max(_DECODE_VARLEN_LENS), 128, F16, False,
             splits=16, seed=50, H_kv=8, seqlens=_DECODE_VARLEN_LENS),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def make_qkv(w: Workload, device="cpu"):
    """Draw Q [B,H,Nq,d], then K and V [B,H_kv,Nk,d] as float32 N(0,1) (times
    w.mult), cast to w.dtype.

    The generator runs on `device`, so the bits depend on it; callers that need
    the same data on the CPU copy the tensors rather than drawing again.
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    out = []
    hk = w.H_kv or w.H
    for n, heads in ((w.Nq, w.H), (w.Nk, hk), (w.Nk, hk)):
        x = torch.randn((w.B, heads, n, w.d), generator=g, dtype=torch.float32, device=device)
        if w.mult != 1.0:
            x.mul_(w.mult)
        out.append(x.to(w.dtype))
        del x
    return tuple(out)


def cu_seqlens(lengths):
    """Cumulative offsets [0, l0, l0 + l1, ...] of packed sequences (int32)."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_varlen(w: Workload, device="cpu"):
    """Packed Q [total, H, d] and K, V [total, H_kv, d] drawn as in make_qkv, plus
    the cumulative offsets of w.seqlens (the same for queries and keys)."""
    total = sum(w.seqlens)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    out = []
    for heads in (w.H, w.H_kv, w.H_kv):
        x = torch.randn((total, heads, w.d), generator=g, dtype=torch.float32, device=device)
        if w.mult != 1.0:
            x.mul_(w.mult)
        out.append(x.to(w.dtype))
        del x
    cu = cu_seqlens(w.seqlens).to(device)
    return (*out, cu, cu.clone())


def make_varlen_decode(w: Workload, device="cpu", seqlens=None, spare_rows=0, fill=float("nan")):
    """One query row per sequence over packed keys.

    Returns q [B, H, d]; k, v [total_k, H_kv, d] with sequence b in rows
    [cu[b], cu[b+1]) (lengths w.seqlens unless given) followed by `spare_rows`
    rows of `fill` (NaN by default: a kernel that reads past the last sequence
    produces NaN); cu_seqlens_k int32 [B + 1].  Q, then the keys, then the values
    are drawn as in make_qkv.
    """
    lens = [int(n) for n in (seqlens if seqlens is not None else w.seqlens)]
    B, hk, total = len(lens), w.H_kv or w.H, sum(lens)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    out = []
    for shape in ((B, w.H, w.d), (total, hk, w.d), (total, hk, w.d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        if w.mult != 1.0:
            x.mul_(w.mult)
        out.append(x.to(w.dtype))
        del x
    q, k_tok, v_tok = out
    kv = []
    for tok in (k_tok, v_tok):
        if spare_rows:
            pad = torch.full((spare_rows, hk, w.d), fill, dtype=w.dtype, device=device)
            tok = torch.cat([tok, pad])
        kv.append(tok)
    return q, kv[0], kv[1], cu_seqlens(lens).to(device)


def make_partials(S, B, H, Nq, d, seed=7, device="cpu", empty_every=0):
    """Seeded fp32 partial results for exercising a split combine on its own.

    o_part [S,B,H,Nq,d] ~ N(0,1); lse_part [S,B,H,Nq] ~ 4*N(0,1).  With
    empty_every = k > 0, every k-th split of every row is marked empty (-inf).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    o = torch.randn((S, B, H, Nq, d), generator=g, dtype=torch.float32, device=device)
    lse = 4.0 * torch.randn((S, B, H, Nq), generator=g, dtype=torch.float32, device=device)
    if empty_every > 0:
        R = B * H * Nq
        s_idx = torch.arange(S, device=device)[:, None]
        r_idx = torch.arange(R, device=device)[None, :]
        empty = ((s_idx + r_idx) % empty_every == 0).reshape(S, B, H, Nq)
        lse[empty] = -math.inf
    return o, lse


def make_paged(w: Workload, device="cpu", seqlens=None, spare_pages=0, fill=float("nan")):
    """A paged K/V cache for a single-row decode workload.

    Returns q [B, H, d]; k_cache, v_cache [num_pages, page_size, H_kv, d] holding
    key t of sequence b at row t % page_size of page block_table[b][t //
    page_size]; block_table int32 [B, max_pages] (-1 past a sequence's pages);
    seqlens int32 [B] (default Nk for every sequence).  Q, then every sequence's
    K and V (token-major) are drawn as in make_qkv; physical pages are handed out
    in the order of a seeded permutation, so consecutive logical pages are
    scattered.  Rows past a sequence's end and `spare_pages` unused pages hold
    `fill` (NaN by default: a kernel that reads them produces NaN).
    """
    lens = [int(n) for n in (seqlens if seqlens is not None else [w.Nk] * w.B)]
    B, ps, hk = len(lens), w.page_size, w.H_kv or w.H
    npg = [-(-n // ps) for n in lens]
    max_pages = max(1, max(npg))
    num_pages = max(1, sum(npg) + spare_pages)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    total = sum(lens)
    drawn = []
    for shape in ((B, w.H, w.d), (total, hk, w.d), (total, hk, w.d)):
        x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
        if w.mult != 1.0:
            x.mul_(w.mult)
        drawn.append(x.to(w.dtype))
        del x
    q, k_tok, v_tok = drawn
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(w.seed + 1000))
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    page_of_tok, row_of_tok = [], []
    nxt = 0
    for b, n in enumerate(lens):
        pages = perm[nxt:nxt + npg[b]]
        nxt += npg[b]
        table[b, :npg[b]] = pages.to(torch.int32)
        t = torch.arange(n)
        page_of_tok.append(pages[t // ps])
        row_of_tok.append(t % ps)
    caches = []
    for tok in (k_tok, v_tok):
        cache = torch.full((num_pages, ps, hk, w.d), fill, dtype=w.dtype, device=device)
        if total:
            pi = torch.cat(page_of_tok).to(device)
            ri = torch.cat(row_of_tok).to(device)
            cache[pi, ri] = tok
        caches.append(cache)
    del k_tok, v_tok
    return q, caches[0], caches[1], table.to(device), torch.tensor(lens, dtype=torch.int32, device=device)
