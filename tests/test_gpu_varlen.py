"""GPU parity of fa_fwd_varlen (packed variable-length sequences with grouped
K/V heads) through the C ABI against the fp64 oracle.

Small packed batches (ragged lengths, empty sequences, sequences without keys,
Nq != Nk, GQA and MQA head groups) are compared on every output element; the
varlen_gqa workload is compared at full size on sampled rows, through the same
call the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import BY_NAME, cu_seqlens, make_varlen
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
    q = rnd((int(cq[-1]), H, d), dt, seed)
    k = rnd((int(ck[-1]), H_kv, d), dt, seed + 1)
    v = rnd((int(ck[-1]), H_kv, d), dt, seed + 2)
    return q, k, v, cq, ck


def run(dev, q, k, v, cq, ck, causal, scale=None):
    max_q = int((cq[1:] - cq[:-1]).max())
    max_k = int((ck[1:] - ck[:-1]).max())
    o, lse = fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cq.to(dev), ck.to(dev), max_q, max(max_k, 1),
                           causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [  # q lens, k lens, H, H_kv, d, causal, dtype
    ([300, 1, 0, 129], [300, 77, 5, 129], 4, 4, 128, True, BF16),
    ([300, 1, 0, 129], [300, 77, 5, 129], 4, 2, 128, False, F16),
    ([64, 65, 200], [64, 65, 200], 8, 2, 64, True, F16),
    ([500, 7], [130, 7], 4, 1, 64, True, BF16),            # Nq > Nk: leading rows see no key
    ([33, 257], [400, 1000], 6, 3, 128, True, F16),          # Nq < Nk: bottom-right diagonal
    ([90, 40], [0, 40], 2, 1, 128, True, F16),               # a sequence with no keys
    ([1000], [1000], 2, 2, 128, True, BF16),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"H{c[2]}kv{c[3]}d{c[4]}c{int(c[5])}-{('bf16' if c[6] == BF16 else 'f16')}-{len(c[0])}seq")
def test_varlen_small(dev, oracle_lib, case):
    q_lens, k_lens, H, H_kv, d, causal, dt = case
    q, k, v, cq, ck = packed(q_lens, k_lens, H, H_kv, d, dt, 11)
    say(f"fa_fwd_varlen {case}")
    o, lse = run(dev, q, k, v, cq, ck, causal)
    ro, rl = oracle_lib.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), causal, 1 / math.sqrt(d))
    parity.check(o, lse.T, ro, rl.T, dt, f"varlen {case}")     # LSE as [total, H], like O


def test_varlen_scales(dev, oracle_lib):
    q, k, v, cq, ck = packed([150, 70], [150, 90], 4, 2, 64, F16, 21)
    for scale in (0.0, -0.4, 1.7):
        say(f"fa_fwd_varlen scale={scale}")
        o, lse = run(dev, q, k, v, cq, ck, True, scale=scale)
        ro, rl = oracle_lib.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), True, scale)
        parity.check(o, lse.T, ro, rl.T, F16, f"varlen scale {scale}")


def test_varlen_matches_dense_kernel(dev):
    """Equal lengths and H_kv = H: the packed entry point gives bit-identical
    results to fa_fwd on the [B, H, N, d] transpose of the same data."""
    B, H, N, d = 3, 4, 300, 128
    q, k, v, cq, ck = packed([N] * B, [N] * B, H, H, d, BF16, 31)
    say("fa_fwd_varlen vs fa_fwd")
    o, lse = run(dev, q, k, v, cq, ck, True)

    def dense(t):
        return t.reshape(B, N, H, d).permute(0, 2, 1, 3).contiguous().to(dev)

    od, ld = fa.fwd(dense(q), dense(k), dense(v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(B, N, H, d).permute(0, 2, 1, 3), od), "O differs from the dense kernel"
    assert torch.equal(lse.reshape(H, B, N).permute(1, 0, 2), ld), "LSE differs from the dense kernel"


def test_varlen_skips_malformed_sequences(dev, oracle_lib):
    """A sequence whose offsets break the contract (here longer than max_seqlen_q)
    is skipped: its output rows keep their previous contents, the others are right."""
    q_lens = [100, 300, 50]
    q, k, v, cq, ck = packed(q_lens, q_lens, 2, 1, 64, F16, 41)
    say("fa_fwd_varlen malformed sequence")
    out = torch.full(q.shape, 7.0, dtype=F16, device=dev)
    lse = torch.full((2, q.shape[0]), 7.0, dtype=torch.float32, device=dev)
    fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cq.to(dev), ck.to(dev), 100, 100, causal=True,
                  out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle_lib.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), True, 1 / math.sqrt(64))
    s1, e1 = int(cq[1]), int(cq[2])
    assert torch.all(out[s1:e1] == 7.0) and torch.all(lse[:, s1:e1] == 7.0), "skipped rows were written"
    keep = np.r_[0:s1, e1:q.shape[0]]
    parity.check(out[keep], lse[:, keep].T, ro[keep], rl[:, keep].T, F16, "varlen other sequences")
    # outputs allocated by the binding start as O = 0, LSE = -inf, so a skipped
    # sequence reads as one that sees no key instead of uninitialised memory
    o2, l2 = fa.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), cq.to(dev), ck.to(dev), 100, 100, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o2[s1:e1] == 0) and torch.all(torch.isneginf(l2[:, s1:e1])), "binding outputs not cleared"
    assert torch.equal(o2[keep], out[keep]) and torch.equal(l2[:, keep], lse[:, keep])


def test_varlen_gqa_workload(dev, oracle_lib):
    """Full-size varlen_gqa (the benchmark's call), sampled rows vs the oracle."""
    w = BY_NAME["varlen_gqa"]
    q, k, v, cq, ck = make_varlen(w)
    say(f"varlen_gqa total={q.shape[0]} H={w.H} H_kv={w.H_kv}")
    o, lse = run(dev, q, k, v, cq, ck, w.causal)
    total = q.shape[0]
    rng = np.random.default_rng(5)
    cqn = cq.numpy()
    firsts = np.concatenate([[cqn[b] * w.H + h for h in (0, w.H - 1)] for b in range(w.B) if cqn[b + 1] > cqn[b]])
    lasts = np.concatenate([[(cqn[b + 1] - 1) * w.H + h for h in (0, w.H - 1)] for b in range(w.B) if cqn[b + 1] > cqn[b]])
    rows = np.unique(np.concatenate([firsts, lasts, rng.integers(0, total * w.H, 384)]))
    ro, rl = oracle_lib.attention_varlen(q, k, v, cqn, ck.numpy(), w.causal, w.scale, rows=rows)
    idx = torch.from_numpy(rows).to(dev)      # token * H + head
    parity.check(o.reshape(-1, w.d)[idx], lse.T.reshape(-1)[idx], ro, rl, w.dtype, "varlen_gqa sampled")
