"""GPU parity of fa_bwd_varlen (backward over packed variable-length sequences
with grouped K/V heads) through the C ABI against the fp64 oracle.

The library's fa_fwd_varlen supplies o and lse, as in use.  Every element of dq,
dk and dv is compared, on batches with ragged lengths, empty sequences on either
side, Nq != Nk, GQA and MQA groups, and a mix of long and short sequences.  The
reference adds to the oracle's exact gradients the exact effect of forming
D = rowsum(dO o O) from the rounded O the forward stored, per sequence
(parity.varlen_bwd_refs): very short sequences make dP - D cancel.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import cu_seqlens
from tests import parity

pytestmark = pytest.mark.gpu
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rnd(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def say(msg):
    print(f"[case] {msg}", flush=True)


def packed(q_lens, k_lens, H, H_kv, d, dt, seed):
    cq, ck = cu_seqlens(q_lens), cu_seqlens(k_lens)
    tq, tk = int(cq[-1]), int(ck[-1])
    q, g = rnd((tq, H, d), dt, seed), rnd((tq, H, d), dt, seed + 3)
    k, v = rnd((tk, H_kv, d), dt, seed + 1), rnd((tk, H_kv, d), dt, seed + 2)
    return q, k, v, g, cq, ck


def lens(cu):
    return cu[1:] - cu[:-1]


def run(dev, q, k, v, g, cq, ck, causal, scale=None, max_q=None, max_k=None):
    mq = int(lens(cq).max()) if max_q is None else max_q
    mk = max(int(lens(ck).max()), 1) if max_k is None else max_k
    qd, kd, vd, gd, cqd, ckd = (t.to(dev) for t in (q, k, v, g, cq, ck))
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, mq, mk, causal=causal, scale=scale)
    grads = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, mq, mk, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return grads


SMALL = [  # q lens, k lens, H, H_kv, d, causal, dtype
    ([300, 1, 0, 129], [300, 77, 5, 129], 4, 4, 128, True, BF16),
    ([300, 1, 0, 129], [300, 77, 5, 129], 4, 2, 128, False, F16),
    ([64, 65, 200], [64, 65, 200], 8, 2, 64, True, F16),
    ([500, 7], [130, 7], 4, 1, 64, True, BF16),            # Nq > Nk: leading rows see no key
    ([33, 257], [400, 1000], 6, 3, 128, True, F16),          # Nq < Nk: bottom-right diagonal
    ([90, 40], [0, 40], 2, 1, 128, True, F16),               # a sequence with no keys
    ([0, 70, 2], [150, 70, 2], 4, 2, 64, True, BF16),        # keys no query sees
    ([1500, 64, 900, 1, 333], [1500, 64, 900, 1, 333], 8, 2, 128, True, BF16),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"H{c[2]}kv{c[3]}d{c[4]}c{int(c[5])}-{('bf16' if c[6] == BF16 else 'f16')}-{len(c[0])}seq")
def test_bwd_varlen_small(dev, oracle_lib, case):
    q_lens, k_lens, H, H_kv, d, causal, dt = case
    q, k, v, g, cq, ck = packed(q_lens, k_lens, H, H_kv, d, dt, 51)
    say(f"fa_bwd_varlen {case}")
    grads = run(dev, q, k, v, g, cq, ck, causal)
    ref = parity.varlen_bwd_refs(oracle_lib, q, k, v, g, cq, ck, causal, 1 / math.sqrt(d), dt)
    parity.check_grads(grads, ref, dt, f"bwd varlen {case}")


def test_bwd_varlen_scales(dev, oracle_lib):
    q, k, v, g, cq, ck = packed([150, 70], [150, 90], 4, 2, 64, F16, 61)
    for scale in (0.0, -0.4, 1.7):
        say(f"fa_bwd_varlen scale={scale}")
        grads = run(dev, q, k, v, g, cq, ck, True, scale=scale)
        ref = parity.varlen_bwd_refs(oracle_lib, q, k, v, g, cq, ck, True, scale, F16)
        parity.check_grads(grads, ref, F16, f"bwd varlen scale {scale}")


def test_bwd_varlen_matches_dense_kernel(dev):
    """Equal lengths: the packed backward gives bit-identical gradients to fa_bwd_gqa
    on the [B, H, N, d] transpose of the same data."""
    B, H, H_kv, N, d = 2, 4, 2, 300, 128
    q, k, v, g, cq, ck = packed([N] * B, [N] * B, H, H_kv, d, BF16, 71)
    say("fa_bwd_varlen vs fa_bwd_gqa")
    dq, dk, dv = run(dev, q, k, v, g, cq, ck, True)

    def dense(t):
        return t.reshape(B, N, t.shape[1], d).permute(0, 2, 1, 3).contiguous().to(dev)

    qd, kd, vd, gd = dense(q), dense(k), dense(v), dense(g)
    o, lse = fa.fwd_gqa(qd, kd, vd, causal=True)
    ref = fa.bwd_gqa(qd, kd, vd, o, lse, gd, causal=True)
    torch.cuda.synchronize()
    for x, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert torch.equal(dense(x).view(torch.int16), r.view(torch.int16)), f"{n} differs from the dense kernels"


def test_bwd_varlen_skips_malformed_sequences(dev, oracle_lib):
    """A sequence longer than max_seqlen breaks the contract: its rows of dq, dk and
    dv keep their previous contents, the other sequences' gradients are right."""
    q_lens = [100, 300, 50]
    q, k, v, g, cq, ck = packed(q_lens, q_lens, 2, 1, 64, F16, 81)
    say("fa_bwd_varlen malformed sequence")
    qd, kd, vd, gd, cqd, ckd = (t.to(dev) for t in (q, k, v, g, cq, ck))
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, 300, 300, causal=True)
    dq, dk, dv = (torch.full(t.shape, 7.0, dtype=F16, device=dev) for t in (q, k, v))
    fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, 100, 100, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    s1, e1 = int(cq[1]), int(cq[2])
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert torch.all(t[s1:e1] == 7.0), f"skipped rows of {n} were written"
    rq, rk, rv = parity.varlen_bwd_refs(oracle_lib, q, k, v, g, cq, ck, True, 1 / math.sqrt(64), F16)
    keep = np.r_[0:s1, e1:q.shape[0]]
    parity.check_grads((dq[keep], dk[keep], dv[keep]), (rq[keep], rk[keep], rv[keep]), F16,
                       "bwd varlen other sequences")
    # gradients allocated by the binding start at zero
    g2 = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, 100, 100, causal=True)
    torch.cuda.synchronize()
    for t, r, n in zip(g2, (dq, dk, dv), ("dq", "dk", "dv")):
        assert torch.all(t[s1:e1] == 0), f"binding-allocated {n} not cleared"
        assert torch.equal(t[keep], r[keep]), f"binding-allocated {n} differs"
