"""Output canaries: every entry point writes only inside its output tensors.

Each output is a view into a larger buffer filled with a sentinel; after the
call the sentinel regions before and after the view must be intact, and a
second call into fresh tensors must give the same bits (deterministic).
Shapes have ragged tails (sizes that are not multiples of the tiles).
"""
import math

import numpy as np
import pytest
import torch

from exact_attention_22_amd import fa
from exact_attention_22_amd.inputs import BY_NAME, make_paged, make_varlen_decode
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu
F16, BF16 = torch.float16, torch.bfloat16
PAD = 4096                     # elements of sentinel on each side (keeps 16-byte alignment)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rnd(shape, dtype, seed, dev):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(dev)


def say(msg):
    print(f"[case] {msg}", flush=True)


class Padded:
    """A view of `shape` inside a buffer with PAD sentinel elements on each side."""

    def __init__(self, shape, dtype, dev, fill=None):
        n = int(np.prod(shape))
        if fill is None:
            fill = 0xA5 if dtype == torch.uint8 else 12345.0
        self.fill = fill
        self.buf = torch.full((n + 2 * PAD,), fill, dtype=dtype, device=dev)
        self.n = n
        self.view = self.buf[PAD:PAD + n].view(shape)

    def intact(self):
        return bool(torch.all(self.buf[:PAD] == self.fill)) and bool(torch.all(self.buf[PAD + self.n:] == self.fill))


def same_bits(a, b):
    if a.dtype.is_floating_point:
        w = {2: torch.int16, 4: torch.int32}[a.element_size()]
        return torch.equal(a.view(w), b.view(w))
    return torch.equal(a, b)


def check(outs, again, what):
    torch.cuda.synchronize()
    for i, p in enumerate(outs):
        assert p.intact(), f"{what}: output {i} wrote outside its tensor"
    for i, (p, r) in enumerate(zip(outs, again)):
        assert same_bits(p.view, r), f"{what}: output {i} differs between two calls"
    print(f"[canary] {what} ok", flush=True)


def test_canary_splitkv_and_combine(dev):
    B, H, Nq, Nk, d, S = 2, 3, 5, 1001, 128, 7
    q, k, v = rnd((B, H, Nq, d), F16, 1, dev), rnd((B, H, Nk, d), F16, 2, dev), rnd((B, H, Nk, d), F16, 3, dev)
    say("canary fa_fwd_splitkv / fa_splitkv_combine")
    op, lp = Padded((S, B, H, Nq, d), torch.float32, dev), Padded((S, B, H, Nq), torch.float32, dev)
    fa.fwd_splitkv(q, k, v, S, causal=True, o_part=op.view, lse_part=lp.view)
    check([op, lp], fa.fwd_splitkv(q, k, v, S, causal=True), "splitkv partials")
    o, l = Padded((B, H, Nq, d), F16, dev), Padded((B, H, Nq), torch.float32, dev)
    fa.splitkv_combine(op.view, lp.view, F16, out=o.view, lse=l.view)
    check([o, l], fa.splitkv_combine(op.view, lp.view, F16), "combine")
    # single-row decode path (Nq = 1) with grouped heads
    qg = rnd((B, 8, 1, d), BF16, 4, dev)
    kg, vg = rnd((B, 2, Nk, d), BF16, 5, dev), rnd((B, 2, Nk, d), BF16, 6, dev)
    op2, lp2 = Padded((S, B, 8, 1, d), torch.float32, dev), Padded((S, B, 8, 1), torch.float32, dev)
    fa.fwd_splitkv_gqa(qg, kg, vg, S, o_part=op2.view, lse_part=lp2.view)
    check([op2, lp2], fa.fwd_splitkv_gqa(qg, kg, vg, S), "splitkv gqa decode partials")


@pytest.mark.parametrize("H,H_kv", [(8, 2), (16, 4)], ids=["kv2", "kv4"])
def test_canary_paged(dev, H, H_kv):
    w = BY_NAME["decode_paged"].with_(B=3, H=H, H_kv=H_kv, page_size=16, seed=90)
    q, kc, vc, bt, sl = (t.to(dev) for t in make_paged(w, seqlens=[300, 1, 77], spare_pages=3))
    S = 5
    say(f"canary fa_fwd_splitkv_paged H={H} H_kv={H_kv}")
    op, lp = Padded((S, 3, H, 1, w.d), torch.float32, dev), Padded((S, 3, H, 1), torch.float32, dev)
    fa.fwd_splitkv_paged(q, kc, vc, bt, sl, S, o_part=op.view, lse_part=lp.view)
    check([op, lp], fa.fwd_splitkv_paged(q, kc, vc, bt, sl, S), "paged partials")


def test_canary_packed_decode(dev):
    w = BY_NAME["decode_varlen"].with_(H=8, H_kv=2, seed=91)
    q, k, v, cu = (t.to(dev) for t in make_varlen_decode(w, seqlens=[300, 1, 0, 77], spare_rows=3))
    S = 5
    say("canary fa_fwd_splitkv_varlen")
    op, lp = Padded((S, 4, 8, 1, w.d), torch.float32, dev), Padded((S, 4, 8, 1), torch.float32, dev)
    fa.fwd_splitkv_varlen(q, k, v, cu, 300, S, o_part=op.view, lse_part=lp.view)
    check([op, lp], fa.fwd_splitkv_varlen(q, k, v, cu, 300, S), "packed decode partials")


def test_canary_fwd_gqa_and_varlen(dev):
    B, H, H_kv, N, d = 1, 4, 2, 333, 64
    q, k, v = rnd((B, H, N, d), BF16, 7, dev), rnd((B, H_kv, N, d), BF16, 8, dev), rnd((B, H_kv, N, d), BF16, 9, dev)
    say("canary fa_fwd_gqa")
    o, l = Padded((B, H, N, d), BF16, dev), Padded((B, H, N), torch.float32, dev)
    fa.fwd_gqa(q, k, v, causal=True, out=o.view, lse=l.view)
    check([o, l], fa.fwd_gqa(q, k, v, causal=True), "fwd gqa")
    lens = [130, 1, 0, 257]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    T = sum(lens)
    qv, kv_, vv = rnd((T, H, 128), F16, 10, dev), rnd((T, H_kv, 128), F16, 11, dev), rnd((T, H_kv, 128), F16, 12, dev)
    say("canary fa_fwd_varlen")
    o2, l2 = Padded((T, H, 128), F16, dev), Padded((H, T), torch.float32, dev)
    fa.fwd_varlen(qv, kv_, vv, cu, cu, max(lens), max(lens), causal=True, out=o2.view, lse=l2.view)
    check([o2, l2], fa.fwd_varlen(qv, kv_, vv, cu, cu, max(lens), max(lens), causal=True), "fwd varlen")


def test_canary_bwd(dev):
    B, H, N, d = 1, 2, 257, 128
    q, k, v, g = (rnd((B, H, N, d), F16, s, dev) for s in (13, 14, 15, 16))
    o, lse = fa.fwd(q, k, v, causal=True)
    say("canary fa_bwd")
    grads = [Padded((B, H, N, d), F16, dev) for _ in range(3)]
    ws = Padded((fa.bwd_workspace_bytes(B, H, N) // 4,), torch.float32, dev)
    fa.bwd(q, k, v, o, lse, g, causal=True, dq=grads[0].view, dk=grads[1].view, dv=grads[2].view,
           workspace=ws.view)
    torch.cuda.synchronize()
    assert ws.intact(), "bwd workspace written outside its bounds"
    check(grads, fa.bwd(q, k, v, o, lse, g, causal=True), "bwd")
    # packed sequences with grouped heads
    lens = [100, 1, 200]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    T, H, H_kv = sum(lens), 4, 2
    qv, gv = rnd((T, H, d), BF16, 17, dev), rnd((T, H, d), BF16, 18, dev)
    kv_, vv = rnd((T, H_kv, d), BF16, 19, dev), rnd((T, H_kv, d), BF16, 20, dev)
    ov, lv = fa.fwd_varlen(qv, kv_, vv, cu, cu, 200, 200, causal=True)
    say("canary fa_bwd_varlen")
    pg = [Padded(tuple(t.shape), BF16, dev) for t in (qv, kv_, vv)]
    fa.bwd_varlen(qv, kv_, vv, ov, lv, gv, cu, cu, 200, 200, causal=True, dq=pg[0].view, dk=pg[1].view,
                  dv=pg[2].view)
    check(pg, fa.bwd_varlen(qv, kv_, vv, ov, lv, gv, cu, cu, 200, 200, causal=True), "bwd varlen")


def test_canary_fp8(dev):
    B, H, N, d = 1, 2, 300, 128
    x = rnd((B * H, N, d), BF16, 21, dev)
    say("canary fa_quantize_fp8")
    c, s = Padded((B * H, N, d), torch.uint8, dev), Padded((B * H, 3), torch.float32, dev)
    fa.quantize_fp8(x, 128, out=c.view, descale=s.view)
    check([c, s], fa.quantize_fp8(x, 128), "quantize fp8")
    q8 = c.view.reshape(B, H, N, d)
    qd = s.view.reshape(B, H, 3)
    vcodes, vd = fa.quantize_fp8(x, N)
    say("canary fa_fwd_fp8")
    o, l = Padded((B, H, N, d), BF16, dev), Padded((B, H, N), torch.float32, dev)
    args = (q8, q8, vcodes.reshape(B, H, N, d), qd, qd, vd.reshape(B, H))
    fa.fwd_fp8(*args, causal=True, scale=1 / math.sqrt(d), out=o.view, lse=l.view)
    check([o, l], fa.fwd_fp8(*args, causal=True, scale=1 / math.sqrt(d)), "fwd fp8")
    assert ofp8.E4M3_MAX == 448.0
