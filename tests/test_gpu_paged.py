"""GPU parity of the paged-KV split-KV decode (fa_fwd_splitkv_paged, then
fa_splitkv_combine) through the C ABI against the fp64 oracle.

Caches are built by inputs.make_paged: pages handed out in a seeded random
order, rows past each sequence's end and spare pages filled with NaN, so any
read outside a sequence's keys shows up as NaN.  Small cases compare every
partial and every output row; the decode_paged workload (the benchmark's
calls) is compared on every output row at full size.
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import BY_NAME, make_paged
from tests import parity

pytestmark = pytest.mark.gpu
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(f"[case] {msg}", flush=True)


CASES = [  # B, H, H_kv, d, page_size, lengths, splits, dtype
    (3, 8, 2, 128, 16, (1000, 1, 333), 4, F16),
    (2, 4, 4, 64, 1, (77, 130), 3, BF16),               # one row per page, no grouping
    (4, 32, 8, 128, 64, (0, 4096, 65, 2049), 16, BF16),  # an empty sequence
    (1, 16, 2, 64, 256, (3000,), 7, F16),
    (2, 8, 1, 128, 32, (5, 17), 8, F16),                 # MQA; fewer keys than splits
    (2, 64, 8, 128, 16, (700, 1500), 5, BF16),           # 8 query heads per workgroup
    (2, 8, 4, 128, 1, (300, 1201), 6, F16),              # 4 K/V heads per workgroup, 2 query heads each
    (3, 16, 4, 128, 16, (0, 1, 999), 4, BF16),           # 4 K/V heads per workgroup; an empty sequence
]


def _ids(c):
    return f"B{c[0]}H{c[1]}kv{c[2]}d{c[3]}ps{c[4]}S{c[6]}-{str(c[7])[-4:]}"


@pytest.mark.parametrize("ci,case", list(enumerate(CASES)), ids=lambda x: _ids(x) if isinstance(x, tuple) else str(x))
def test_paged_decode(dev, oracle_lib, ci, case):
    B, H, H_kv, d, ps, lens, S, dt = case
    w = BY_NAME["decode_paged"].with_(B=B, H=H, H_kv=H_kv, d=d, page_size=ps, dtype=dt, seed=60 + ci)
    q, kc, vc, bt, sl = make_paged(w, seqlens=lens, spare_pages=5)
    say(f"fa_fwd_splitkv_paged + combine {case}")
    op, lp = fa.fwd_splitkv_paged(q.to(dev), kc.to(dev), vc.to(dev), bt.to(dev), sl.to(dev), S)
    o, lse = fa.splitkv_combine(op, lp, dt)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    rop, rlp = oracle_lib.split_partials_paged(q, kc, vc, bt.numpy(), list(lens), scale, S)
    parity.check(op, lp, rop, rlp, dt, f"paged partials {case}")
    ro, rl = oracle_lib.attention_paged(q, kc, vc, bt.numpy(), list(lens), scale)
    parity.check(o.reshape(B, H, d), lse.reshape(B, H), ro, rl, dt, f"paged decode {case}")


@pytest.mark.parametrize("H,H_kv", [(8, 2), (16, 4)], ids=["kv2", "kv4"])
def test_paged_bad_entries(dev, oracle_lib, H, H_kv):
    """A page entry outside [0, num_pages) drops its keys; a length beyond the
    table leaves that sequence's partials unwritten (H_kv = 4: the kernel that
    takes four K/V heads per workgroup)."""
    B, d, ps, S = 3, 128, 16, 4
    lens = [100, 80, 50]
    w = BY_NAME["decode_paged"].with_(B=B, H=H, H_kv=H_kv, d=d, page_size=ps, seed=70)
    q, kc, vc, bt, sl = make_paged(w, seqlens=lens)
    num_pages, max_pages = kc.shape[0], bt.shape[1]
    bt_bad, sl_bad = bt.clone(), sl.clone()
    bt_bad[0, 6] = num_pages + 3          # sequence 0: keys 96..99 dropped
    bt_bad[1, 0] = -7                     # sequence 1: keys 0..15 dropped
    sl_bad[2] = max_pages * ps + 1        # sequence 2: skipped
    say("fa_fwd_splitkv_paged with out-of-range entries")
    op = torch.full((S, B, H, 1, d), 7.0, device=dev)
    lp = torch.full((S, B, H, 1), 7.0, device=dev)
    fa.fwd_splitkv_paged(q.to(dev), kc.to(dev), vc.to(dev), bt_bad.to(dev), sl_bad.to(dev), S, o_part=op,
                         lse_part=lp)
    torch.cuda.synchronize()
    assert bool((op[:, 2] == 7.0).all()) and bool((lp[:, 2] == 7.0).all()), "skipped sequence was written"
    o, lse = fa.splitkv_combine(op[:, :2].contiguous(), lp[:, :2].contiguous(), w.dtype)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    # the expected result: sequence 0 without its last page, sequence 1 without its first
    r0o, r0l = oracle_lib.attention_paged(q[:1].contiguous(), kc, vc, bt[:1].numpy(), [96], scale)
    bt1 = bt[1:2, 1:].contiguous().numpy()
    r1o, r1l = oracle_lib.attention_paged(q[1:2].contiguous(), kc, vc, bt1, [64], scale)
    parity.check(o.reshape(2, H, d), lse.reshape(2, H), np.concatenate([r0o, r1o]), np.concatenate([r0l, r1l]),
                 w.dtype, "paged decode with dropped pages")
    # partials allocated by the binding start as empty splits: the skipped
    # sequence combines to O = 0, LSE = -inf instead of uninitialised memory
    o3, l3 = fa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), bt_bad.to(dev), sl_bad.to(dev), num_splits=S)
    torch.cuda.synchronize()
    assert torch.all(o3[2] == 0) and torch.all(torch.isneginf(l3[2])), "skipped sequence not empty"
    assert torch.equal(o3[:2], o.reshape(o3[:2].shape)) and torch.equal(l3[:2], lse.reshape(l3[:2].shape))


def test_decode_paged_workload(dev, oracle_lib):
    """The decode_paged workload at full size (8 sequences of 32768 keys in
    16-row pages, 32 query heads on 8 K/V heads), every output row."""
    w = BY_NAME["decode_paged"]
    q, kc, vc, bt, sl = make_paged(w)
    say(f"decode_paged B={w.B} H={w.H} H_kv={w.H_kv} Nk={w.Nk} page={w.page_size} S={w.splits}")
    o, lse = fa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), bt.to(dev), sl.to(dev), num_splits=w.splits,
                             scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_lib.attention_paged(q, kc, vc, bt.numpy(), sl.tolist(), w.scale)
    parity.check(o.reshape(w.B, w.H, w.d), lse.reshape(w.B, w.H), ro, rl, w.dtype, "decode_paged full")
