"""Pins that tie the fp64 oracle to facts outside itself.

Each pin takes an `Oracle` and raises AssertionError when the oracle disagrees
with what the pages and the mathematics fix.  The same pins run against the real
oracle (must pass) and against deliberately broken copies (at least one must
fail), so a plausible mistake anywhere in the oracle is caught.

Sources for the facts used here:
  Ringi, "Lecture 25", section 2.1 (safe softmax), section 2.2 (merge identity),
  section 1.1 (three-step attention);  AIInfraGuide 6.2 "FlashAttention V2
  explained", section 5.1 (causal mask, -inf before softmax) and its forward
  pseudocode (L = m + log l);  LLM Infra Atlas "FA2: parallelism", section 4
  (causal bound offset by seqlen_k - seqlen_q);  KingOfEgg "Flash Attention (4)",
  section 3.5 (empty row: inv_sum = 1 so O = 0);  Ringi, "Lecture 25", section 8.3
  (the PagedAttention question: a K/V cache in non-contiguous pages reached
  through a page table).
"""
import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = (torch.float16, torch.bfloat16)


def _close(a, b, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b) and np.array_equal(a[inf_a], b[inf_b]), f"{what}: infinities differ"
    assert not np.isnan(a).any() and not np.isnan(b).any(), f"{what}: NaN"
    fin = ~inf_a
    err = np.max(np.abs(a[fin] - b[fin]), initial=0.0)
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol:.1e}"


def _rand(shape, dtype, seed, lo=None, hi=None, step=None):
    g = torch.Generator().manual_seed(seed)
    if step is None:
        return torch.randn(shape, generator=g).to(dtype)
    n = torch.randint(int(lo / step), int(hi / step) + 1, shape, generator=g)
    return (n.double() * step).to(dtype)     # exactly representable grid values


def _visible(Nq, Nk, causal):
    """[Nq, Nk] boolean visibility: key j < Nk, and j <= i + Nk - Nq when causal."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    vis = np.ones((Nq, Nk), dtype=bool)
    if causal:
        vis &= j <= i + (Nk - Nq)
    return vis


def library_reference(q, k, v, causal, scale):
    """Attention from numpy matmul + scipy's logsumexp/softmax (fp64)."""
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    sigma = float(np.float32(scale))
    s = sigma * (qd @ np.swapaxes(kd, -1, -2))
    vis = _visible(q.shape[2], k.shape[2], causal)
    s = np.where(vis, s, -np.inf)
    empty = ~vis.any(axis=1)                                   # [Nq]
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = scipy.special.logsumexp(s, axis=-1)
        p = scipy.special.softmax(np.where(empty[:, None], 0.0, s), axis=-1)
    o = p @ vd
    o[..., empty, :] = 0.0
    lse[..., empty] = -np.inf
    return o, lse


CASES = [  # B, H, Nq, Nk, d, causal
    (1, 2, 7, 13, 8, False), (1, 2, 7, 13, 8, True), (2, 1, 16, 16, 4, True),
    (1, 1, 1, 5, 16, False), (1, 2, 33, 16, 8, True), (1, 1, 3, 40, 8, True),
    (2, 2, 20, 20, 64, False), (1, 1, 9, 9, 128, True),
]
SCALES = (None, 0.37, -0.5, 2.0)


def pin_library_reference(orc):
    """Every case and scale matches numpy/scipy attention to 1e-12."""
    n = 0
    for ci, (B, H, Nq, Nk, d, causal) in enumerate(CASES):
        for dt in DTYPES:
            for sc in SCALES:
                scale = 1 / math.sqrt(d) if sc is None else sc
                q = _rand((B, H, Nq, d), dt, 100 + n)
                k = _rand((B, H, Nk, d), dt, 200 + n)
                v = _rand((B, H, Nk, d), dt, 300 + n)
                n += 1
                o, lse = orc.attention(q, k, v, causal, scale, nthreads=2)
                ro, rl = library_reference(q, k, v, causal, scale)
                _close(o, ro, 1e-12, f"O case {ci} {dt} scale {scale}")
                _close(lse, rl, 1e-11, f"LSE case {ci} {dt} scale {scale}")


def pin_torch_sdpa(orc):
    """O matches torch's fp64 scaled_dot_product_attention with an explicit mask."""
    for ci, (B, H, Nq, Nk, d, causal) in enumerate(CASES):
        vis = _visible(Nq, Nk, causal)
        rows = vis.any(axis=1)
        if not rows.any():
            continue
        q = _rand((B, H, Nq, d), torch.float16, 400 + ci)
        k = _rand((B, H, Nk, d), torch.float16, 500 + ci)
        v = _rand((B, H, Nk, d), torch.float16, 600 + ci)
        scale = float(np.float32(1 / math.sqrt(d)))
        o, _ = orc.attention(q, k, v, causal, scale, nthreads=2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.double(), k.double(), v.double(), attn_mask=torch.from_numpy(vis), scale=scale)
        _close(o[:, :, rows], ref.numpy()[:, :, rows], 1e-12, f"SDPA case {ci}")


def pin_identical_keys(orc):
    """All keys equal: O_i is the mean of the visible values, LSE_i = s_i + ln|V_i|."""
    for causal in (False, True):
        for dt in DTYPES:
            B, H, Nq, Nk, d = 1, 2, 12, 17, 8
            q = _rand((B, H, Nq, d), dt, 11)
            k = _rand((B, H, 1, d), dt, 12).expand(B, H, Nk, d).contiguous()
            v = _rand((B, H, Nk, d), dt, 13)
            scale = 0.5
            o, lse = orc.attention(q, k, v, causal, scale, nthreads=1)
            vis = _visible(Nq, Nk, causal)
            vd = v.double().numpy()
            cnt = vis.sum(axis=1)
            exp_o = np.einsum("ij,bhjd->bhid", vis.astype(np.float64), vd) / np.maximum(cnt, 1)[:, None]
            s = scale * np.einsum("bhid,bhd->bhi", q.double().numpy(), k.double().numpy()[:, :, 0])
            with np.errstate(divide="ignore"):
                exp_l = np.where(cnt > 0, s + np.log(cnt), -np.inf)
            exp_o[:, :, cnt == 0] = 0.0
            _close(o, exp_o, 1e-12, f"identical keys O causal={causal}")
            _close(lse, exp_l, 1e-12, f"identical keys LSE causal={causal}")


def pin_first_causal_row(orc):
    """Nq == Nk causal: row 0 sees only key 0, so O_0 = v_0 and LSE_0 = sigma q_0.k_0;
    the last row sees every key, so it equals the non-causal last row."""
    for dt in DTYPES:
        B, H, N, d = 2, 2, 24, 16
        q, k, v = (_rand((B, H, N, d), dt, s) for s in (21, 22, 23))
        o, lse = orc.attention(q, k, v, True, 0.25, nthreads=1)
        on, ln = orc.attention(q, k, v, False, 0.25, nthreads=1)
        _close(o[:, :, 0], v.double().numpy()[:, :, 0], 0.0, "first causal row O")
        s0 = 0.25 * (q.double().numpy()[:, :, 0] * k.double().numpy()[:, :, 0]).sum(-1)
        _close(lse[:, :, 0], s0, 1e-13, "first causal row LSE")
        _close(o[:, :, -1], on[:, :, -1], 1e-13, "last causal row O")
        _close(lse[:, :, -1], ln[:, :, -1], 1e-13, "last causal row LSE")


def pin_scale_zero(orc):
    """scale = 0: uniform weights, O_i = mean of visible v, LSE_i = ln |V_i|."""
    for causal in (False, True):
        B, H, Nq, Nk, d = 1, 1, 10, 6, 8
        q, k, v = (_rand((B, H, n, d), torch.bfloat16, s) for n, s in ((Nq, 31), (Nk, 32), (Nk, 33)))
        o, lse = orc.attention(q, k, v, causal, 0.0, nthreads=1)
        vis = _visible(Nq, Nk, causal)
        cnt = vis.sum(axis=1)
        exp_o = (vis.astype(np.float64) @ v.double().numpy()[0, 0]) / np.maximum(cnt, 1)[:, None]
        with np.errstate(divide="ignore"):
            exp_l = np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf)
        _close(o[0, 0], exp_o, 1e-13, f"scale 0 O causal={causal}")
        _close(lse[0, 0], exp_l, 1e-13, f"scale 0 LSE causal={causal}")


def pin_key_shift(orc):
    """Adding u to every key shifts s_ij by sigma q_i.u for all j: O is unchanged and
    LSE_i moves by sigma q_i.u (softmax(S + c_i) = softmax(S))."""
    for causal in (False, True):
        for dt in DTYPES:
            B, H, Nq, Nk, d = 1, 2, 9, 14, 8
            q = _rand((B, H, Nq, d), dt, 41, -2, 2, 0.125)
            k = _rand((B, H, Nk, d), dt, 42, -3, 3, 0.125)
            u = _rand((1, 1, 1, d), dt, 43, -1, 1, 0.125)
            v = _rand((B, H, Nk, d), dt, 44)
            k2 = (k.double() + u.double()).to(dt)
            assert torch.equal(k2.double(), k.double() + u.double()), "shift not exact"
            o1, l1 = orc.attention(q, k, v, causal, 0.3, nthreads=1)
            o2, l2 = orc.attention(q, k2, v, causal, 0.3, nthreads=1)
            shift = float(np.float32(0.3)) * (q.double().numpy() @ u.double().numpy()[0, 0, 0])
            _close(o2, o1, 1e-12, "key shift O")
            _close(l2, l1 + shift, 1e-12, "key shift LSE")


def pin_value_shift(orc):
    """Adding w to every value row adds w to every non-empty output row."""
    for causal in (False, True):
        B, H, Nq, Nk, d = 1, 1, 8, 11, 16
        q = _rand((B, H, Nq, d), torch.float16, 51)
        k = _rand((B, H, Nk, d), torch.float16, 52)
        v = _rand((B, H, Nk, d), torch.float16, 53, -2, 2, 0.125)
        w = _rand((1, 1, 1, d), torch.float16, 54, -1, 1, 0.125)
        v2 = (v.double() + w.double()).to(torch.float16)
        o1, _ = orc.attention(q, k, v, causal, 0.7, nthreads=1)
        o2, _ = orc.attention(q, k, v2, causal, 0.7, nthreads=1)
        _close(o2, o1 + w.double().numpy()[0, 0], 1e-12, "value shift")


def pin_key_permutation(orc):
    """Non-causal attention is invariant to a joint permutation of keys and values."""
    B, H, Nq, Nk, d = 2, 1, 5, 19, 8
    q, k, v = (_rand((B, H, n, d), torch.float16, s) for n, s in ((Nq, 61), (Nk, 62), (Nk, 63)))
    perm = torch.randperm(Nk, generator=torch.Generator().manual_seed(64))
    o1, l1 = orc.attention(q, k, v, False, 0.4, nthreads=1)
    o2, l2 = orc.attention(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, 0.4, nthreads=1)
    _close(o2, o1, 1e-13, "permutation O")
    _close(l2, l1, 1e-13, "permutation LSE")


def pin_empty_rows(orc):
    """Causal with Nq > Nk: rows i < Nq - Nk see no key (O = 0, LSE = -inf)."""
    B, H, Nq, Nk, d = 1, 1, 20, 8, 8
    q, k, v = (_rand((B, H, n, d), torch.float16, s) for n, s in ((Nq, 71), (Nk, 72), (Nk, 73)))
    o, lse = orc.attention(q, k, v, True, 0.5, nthreads=1)
    assert np.all(o[0, 0, :12] == 0.0) and np.all(lse[0, 0, :12] == -np.inf), "empty rows"
    assert np.all(np.isfinite(lse[0, 0, 12:])), "non-empty rows must be finite"
    # row 12 sees exactly key 0
    _close(o[0, 0, 12], v.double().numpy()[0, 0, 0], 0.0, "first non-empty row")


def pin_dominant_score(orc):
    """When one score leads the rest by > 100 nats, O_i = v_argmax and LSE_i = max s
    (to double rounding) -- also forces scores far beyond exp's range."""
    B, H, Nq, Nk, d = 1, 1, 3, 9, 4
    q = torch.zeros((B, H, Nq, d))
    q[0, 0, :, 0] = torch.tensor([1.0, -1.0, 2.0])
    k = torch.zeros((B, H, Nk, d))
    k[0, 0, :, 0] = torch.arange(Nk) / 4.0
    v = _rand((B, H, Nk, d), torch.float16, 81)
    q, k = q.half(), k.half()
    o, lse = orc.attention(q, k, v, False, 512.0, nthreads=1)
    vd = v.double().numpy()[0, 0]
    exp_o = np.stack([vd[Nk - 1], vd[0], vd[Nk - 1]])
    exp_l = np.array([512.0 * (Nk - 1) / 4.0, 0.0, 512.0 * 2 * (Nk - 1) / 4.0])
    _close(o[0, 0], exp_o, 1e-15, "dominant score O")
    _close(lse[0, 0], exp_l, 1e-12, "dominant score LSE")


def pin_decoders(orc):
    """All 65536 patterns of each format decode as numpy/torch convert them."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in DTYPES:
        mine = orc.decode(bits, dt)
        ref = torch.from_numpy(bits.view(np.int16)).view(dt).double().numpy()
        nan_m, nan_r = np.isnan(mine), np.isnan(ref)
        assert np.array_equal(nan_m, nan_r), f"{dt}: NaN patterns differ"
        assert np.array_equal(mine[~nan_m], ref[~nan_r]), f"{dt}: decoded values differ"


def pin_split_combine(orc):
    """Merging per-split partials reproduces unsplit attention (merge identity)."""
    for causal in (False, True):
        B, H, Nq, Nk, d = 1, 2, 6, 37, 8
        q, k, v = (_rand((B, H, n, d), torch.float16, s) for n, s in ((Nq, 91), (Nk, 92), (Nk, 93)))
        o, lse = orc.attention(q, k, v, causal, 0.6, nthreads=1)
        for S in (1, 2, 16, 17, 37):
            op, lp = orc.split_partials(q, k, v, causal, 0.6, S, nthreads=1)
            oc, lc = orc.combine(op, lp)
            _close(oc, o, 1e-12, f"combine O S={S} causal={causal}")
            _close(lc, lse, 1e-12, f"combine LSE S={S} causal={causal}")


def pin_combine_closed_form(orc):
    """Two splits with l ratio 1:3 (LSE 0 and ln 3): O = (O_1 + 3 O_2)/4, LSE = ln 4;
    an all-empty row gives O = 0, LSE = -inf; one split is the identity."""
    op = np.array([[[1.0, 0.0], [5.0, 6.0]], [[0.0, 1.0], [7.0, 8.0]]])   # [S=2, R=2, d=2]
    lp = np.array([[0.0, -np.inf], [math.log(3.0), -np.inf]])
    o, lse = orc.combine(op, lp)
    _close(o, np.array([[0.25, 0.75], [0.0, 0.0]]), 1e-15, "combine closed form O")
    _close(lse, np.array([math.log(4.0), -np.inf]), 1e-15, "combine closed form LSE")
    o1, l1 = orc.combine(op[:1, :1], lp[:1, :1])
    _close(o1, op[0, :1], 0.0, "combine identity O")
    _close(l1, lp[0, :1], 0.0, "combine identity LSE")


def _eval(expr):
    if isinstance(expr, (int, float)):
        return float(expr)
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log, "inf": math.inf}))


def pin_worked_examples(orc):
    """Hand-derived examples in tests/golden/worked_examples.json."""
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        doc = json.load(f)
    for ex in doc["examples"]:
        dt = {"f16": torch.float16, "bf16": torch.bfloat16}[ex["dtype"]]
        if ex["kind"] == "attention":
            q, k, v = (torch.tensor(ex[n], dtype=torch.float64)[None, None].to(dt) for n in ("q", "k", "v"))
            o, lse = orc.attention(q, k, v, ex["causal"], ex["scale"], nthreads=1)
            exp_o = np.array([[_eval(x) for x in row] for row in ex["O"]])
            exp_l = np.array([_eval(x) for x in ex["LSE"]])
            _close(o[0, 0], exp_o, 1e-14, ex["name"])
            _close(lse[0, 0], exp_l, 1e-14, ex["name"])
        else:
            o, lse = orc.combine(np.array(ex["o_part"], dtype=np.float64),
                                 np.array([[_eval(x) for x in s] for s in ex["lse_part"]]))
            _close(o, np.array([[_eval(x) for x in r] for r in ex["O"]]), 1e-14, ex["name"])
            _close(lse, np.array([_eval(x) for x in ex["LSE"]]), 1e-14, ex["name"])


# -- packed variable-length sequences with grouped K/V heads ---------------
# KingOfEgg "Flash Attention (4)", section 5 (K/V indexed by head group, entry
# with cu_seqlens); Ringi "Lecture 25", section 7 (packing without padding).

def _packed(lens, heads, d, dt, seed):
    """Random packed [sum(lens), heads, d] tensor and its cumulative offsets."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return _rand((int(cu[-1]), heads, d), dt, seed), cu


VARLEN_CASES = [  # (q lens, k lens, H, d, causal)
    ([5, 0, 9, 1], [7, 3, 9, 4], 2, 8, True),
    ([5, 0, 9, 1], [7, 3, 9, 4], 2, 8, False),
    ([12, 3], [4, 3], 3, 16, True),            # Nq > Nk: leading rows of sequence 0 see no key
    ([6, 2, 7], [0, 5, 7], 1, 8, True),        # a sequence with no keys
    ([1, 1, 1], [13, 2, 1], 2, 64, False),
]


def pin_varlen_per_sequence(orc):
    """With H_kv = H each sequence of a packed batch equals the [B,H,N,d] oracle
    (itself pinned above) on that sequence alone, rows and heads transposed."""
    n = 0
    for ql, kl, H, d, causal in VARLEN_CASES:
        for dt in DTYPES:
            q, cq = _packed(ql, H, d, dt, 700 + n)
            k, ck = _packed(kl, H, d, dt, 800 + n)
            v, _ = _packed(kl, H, d, dt, 900 + n)
            n += 1
            o, lse = orc.attention_varlen(q, k, v, cq, ck, causal, 0.3, nthreads=2)
            assert o.shape == (int(cq[-1]), H, d) and lse.shape == (H, int(cq[-1])), "varlen shapes"
            for b in range(len(ql)):
                if ql[b] == 0:
                    continue
                sq = q[cq[b]:cq[b + 1]].permute(1, 0, 2)[None].contiguous()
                if kl[b] == 0:
                    _close(o[cq[b]:cq[b + 1]], np.zeros((ql[b], H, d)), 0.0, "no-key sequence O")
                    assert np.all(lse[:, cq[b]:cq[b + 1]] == -np.inf), "no-key sequence LSE"
                    continue
                sk = k[ck[b]:ck[b + 1]].permute(1, 0, 2)[None].contiguous()
                sv = v[ck[b]:ck[b + 1]].permute(1, 0, 2)[None].contiguous()
                ro, rl = orc.attention(sq, sk, sv, causal, 0.3, nthreads=1)
                _close(o[cq[b]:cq[b + 1]], ro[0].transpose(1, 0, 2), 1e-15, f"varlen seq {b} O")
                _close(lse[:, cq[b]:cq[b + 1]], rl[0], 1e-15, f"varlen seq {b} LSE")


def pin_varlen_grouped_heads(orc):
    """Grouped K/V heads (H_kv < H, MQA at H_kv = 1) equal full multi-head attention
    with each K/V head repeated for the H / H_kv consecutive query heads of its group."""
    for H, H_kv in ((4, 2), (6, 3), (4, 1), (8, 4)):
        for causal in (False, True):
            ql, kl, d, dt = [9, 4, 0, 6], [9, 11, 2, 3], 8, torch.bfloat16
            q, cq = _packed(ql, H, d, dt, 1000 + H * 10 + H_kv)
            k, ck = _packed(kl, H_kv, d, dt, 1100 + H * 10 + H_kv)
            v, _ = _packed(kl, H_kv, d, dt, 1200 + H * 10 + H_kv)
            o, lse = orc.attention_varlen(q, k, v, cq, ck, causal, 0.45, nthreads=2)
            G = H // H_kv
            k_full = k.repeat_interleave(G, dim=1).contiguous()
            v_full = v.repeat_interleave(G, dim=1).contiguous()
            ro, rl = orc.attention_varlen(q, k_full, v_full, cq, ck, causal, 0.45, nthreads=2)
            _close(o, ro, 0.0, f"grouped heads O H={H} H_kv={H_kv}")
            _close(lse, rl, 0.0, f"grouped heads LSE H={H} H_kv={H_kv}")


def pin_varlen_rows(orc):
    """Selected rows (token*H + h) equal the same rows of the full result."""
    ql, kl, H, d = [7, 5], [3, 9], 4, 16
    q, cq = _packed(ql, H, d, torch.float16, 1301)
    k, ck = _packed(kl, 2, d, torch.float16, 1302)
    v, _ = _packed(kl, 2, d, torch.float16, 1303)
    o, lse = orc.attention_varlen(q, k, v, cq, ck, True, 0.5, nthreads=1)
    rows = np.array([0, 5, 13, 27, 47])
    ro, rl = orc.attention_varlen(q, k, v, cq, ck, True, 0.5, rows=rows, nthreads=1)
    _close(ro, o.reshape(-1, d)[rows], 0.0, "varlen selected rows O")
    _close(rl, lse.T.reshape(-1)[rows], 0.0, "varlen selected rows LSE")


def pin_dense_grouped_heads(orc):
    """Grouped K/V heads in the [B, H, N, d] layout equal the packed-sequence oracle
    (whose head grouping is pinned above) on the same data with uniform lengths."""
    for H, H_kv in ((8, 2), (4, 1), (6, 3)):
        for causal in (False, True):
            B, Nq, Nk, d, dt = 2, 9, 13, 16, torch.float16
            q = _rand((B, H, Nq, d), dt, 1400 + H)
            k = _rand((B, H_kv, Nk, d), dt, 1500 + H)
            v = _rand((B, H_kv, Nk, d), dt, 1600 + H)
            o, lse = orc.attention_gqa(q, k, v, causal, 0.35, nthreads=2)

            def pack(t):
                return t.permute(0, 2, 1, 3).reshape(-1, t.shape[1], d).contiguous()
            cq = np.arange(B + 1, dtype=np.int32) * Nq
            ck = np.arange(B + 1, dtype=np.int32) * Nk
            ro, rl = orc.attention_varlen(pack(q), pack(k), pack(v), cq, ck, causal, 0.35, nthreads=2)
            _close(o, ro.reshape(B, Nq, H, d).transpose(0, 2, 1, 3), 0.0, f"dense GQA O H={H} H_kv={H_kv}")
            _close(lse, rl.reshape(H, B, Nq).transpose(1, 0, 2), 0.0, f"dense GQA LSE H={H} H_kv={H_kv}")


# -- backward (Ringi, "Lecture 25", section 3.3) ------------------------------

def _torch_grads(q, k, v, dout, causal, scale):
    """fp64 autograd of softmax(scale Q K^T + mask) V, rows without keys giving 0."""
    qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
    vis = torch.from_numpy(_visible(q.shape[2], k.shape[2], causal))
    s = float(np.float32(scale)) * (qd @ kd.transpose(-1, -2))
    s = s.masked_fill(~vis, -math.inf)
    empty = ~vis.any(dim=1)
    p = torch.softmax(s.masked_fill(empty[:, None], 0.0), dim=-1).masked_fill(empty[:, None], 0.0)
    o = p @ vd
    o.backward(dout.double())
    return qd.grad.numpy(), kd.grad.numpy(), vd.grad.numpy()


BWD_CASES = [  # B, H, Nq, Nk, d, causal, scale
    (1, 2, 7, 13, 8, False, 0.3), (1, 2, 13, 7, 8, True, 0.3), (2, 1, 16, 16, 16, True, -0.45),
    (1, 1, 1, 9, 8, False, 1.7), (1, 1, 20, 6, 8, True, 0.5), (1, 2, 12, 12, 64, True, 0.125),
]


def pin_bwd_autograd(orc):
    """dQ, dK, dV equal torch autograd of the plain forward in fp64."""
    for ci, (B, H, Nq, Nk, d, causal, scale) in enumerate(BWD_CASES):
        for dt in DTYPES:
            q, k, v, g = (_rand((B, H, n, d), dt, 1700 + 10 * ci + s) for s, n in enumerate((Nq, Nk, Nk, Nq)))
            dq, dk, dv = orc.attention_bwd(q, k, v, g, causal, scale, nthreads=2)
            rq, rk, rv = _torch_grads(q, k, v, g, causal, scale)
            _close(dq, rq, 1e-12, f"bwd dQ case {ci} {dt}")
            _close(dk, rk, 1e-12, f"bwd dK case {ci} {dt}")
            _close(dv, rv, 1e-12, f"bwd dV case {ci} {dt}")


def pin_bwd_gqa_autograd(orc):
    """Grouped K/V heads: dK, dV of a shared head equal fp64 autograd through the
    head expansion (a gather inside the graph, so autograd itself sums the group),
    full and on selected rows."""
    for ci, (B, H, H_kv, Nq, Nk, d, causal, scale) in enumerate([
            (1, 4, 2, 9, 11, 8, True, 0.4), (2, 3, 1, 6, 6, 16, False, -0.7), (1, 4, 1, 5, 12, 8, True, 1.1)]):
        dt = DTYPES[ci % len(DTYPES)]
        q, g = (_rand((B, H, Nq, d), dt, 1800 + 10 * ci + s) for s in (0, 1))
        k, v = (_rand((B, H_kv, Nk, d), dt, 1802 + 10 * ci + s) for s in (0, 1))
        qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
        head = torch.arange(H) // (H // H_kv)
        vis = torch.from_numpy(_visible(Nq, Nk, causal))
        sc = float(np.float32(scale)) * (qd @ kd[:, head].transpose(-1, -2))
        empty = ~vis.any(dim=1)
        p = torch.softmax(sc.masked_fill(~vis, -math.inf).masked_fill(empty[:, None], 0.0), dim=-1)
        (p.masked_fill(empty[:, None], 0.0) @ vd[:, head]).backward(g.double())
        dq, dk, dv = orc.attention_bwd_gqa(q, k, v, g, causal, scale, nthreads=2)
        _close(dq, qd.grad.numpy(), 1e-12, f"bwd gqa dQ case {ci}")
        _close(dk, kd.grad.numpy(), 1e-12, f"bwd gqa dK case {ci}")
        _close(dv, vd.grad.numpy(), 1e-12, f"bwd gqa dV case {ci}")
        rows = np.array([0, Nk - 1, B * H_kv * Nk - 1, (B * H_kv - 1) * Nk])
        _, sk, sv = orc.attention_bwd_gqa(q, k, v, g, causal, scale, k_rows=rows, nthreads=2)
        _close(sk, kd.grad.numpy().reshape(-1, d)[rows], 1e-12, f"bwd gqa dK rows case {ci}")
        _close(sv, vd.grad.numpy().reshape(-1, d)[rows], 1e-12, f"bwd gqa dV rows case {ci}")


def pin_bwd_varlen_autograd(orc):
    """Packed sequences: gradients equal fp64 autograd of one attention over all
    packed tokens whose mask allows only same-sequence pairs (bottom-right causal
    within a sequence), grouped K/V heads included; empty sequences on either side."""
    for ci, (q_lens, k_lens, H, H_kv, d, causal, scale) in enumerate([
            ([5, 0, 9, 3], [7, 4, 9, 0], 4, 2, 8, True, 0.45),
            ([6, 11], [6, 11], 2, 1, 16, False, -0.6), ([1, 8, 4], [9, 2, 4], 3, 3, 8, True, 0.9)]):
        dt = DTYPES[ci % len(DTYPES)]
        cq, ck = np.concatenate([[0], np.cumsum(q_lens)]), np.concatenate([[0], np.cumsum(k_lens)])
        tq, tk = int(cq[-1]), int(ck[-1])
        q, g = (_rand((tq, H, d), dt, 1900 + 10 * ci + s) for s in (0, 1))
        k, v = (_rand((tk, H_kv, d), dt, 1902 + 10 * ci + s) for s in (0, 1))
        seq_q, seq_k = np.repeat(np.arange(len(q_lens)), q_lens), np.repeat(np.arange(len(k_lens)), k_lens)
        pos_q, pos_k = np.arange(tq) - cq[seq_q], np.arange(tk) - ck[seq_k]
        vis = seq_q[:, None] == seq_k[None, :]
        if causal:
            shift = (np.asarray(k_lens) - np.asarray(q_lens))[seq_q]
            vis &= pos_k[None, :] <= (pos_q + shift)[:, None]
        vis = torch.from_numpy(vis)
        qd, kd, vd = (t.double().requires_grad_(True) for t in (q, k, v))
        head = torch.arange(H) // (H // H_kv)
        sc = float(np.float32(scale)) * torch.einsum("ihd,jhd->hij", qd, kd[:, head])
        empty = ~vis.any(dim=1)
        p = torch.softmax(sc.masked_fill(~vis, -math.inf).masked_fill(empty[:, None], 0.0), dim=-1)
        o = torch.einsum("hij,jhd->ihd", p.masked_fill(empty[:, None], 0.0), vd[:, head])
        o.backward(g.double())
        dq, dk, dv = orc.attention_bwd_varlen(q, k, v, g, cq, ck, causal, scale, nthreads=2)
        _close(dq, qd.grad.numpy(), 1e-12, f"bwd varlen dQ case {ci}")
        _close(dk, kd.grad.numpy(), 1e-12, f"bwd varlen dK case {ci}")
        _close(dv, vd.grad.numpy(), 1e-12, f"bwd varlen dV case {ci}")


def pin_bwd_finite_differences(orc):
    """Central differences of L = sum(O o dO) (O from torch's fp64 attention) match
    the gradients to within the O(h^2) truncation error."""
    B, H, Nq, Nk, d = 1, 1, 3, 4, 4
    for causal in (False, True):
        q, k, v, g = (_rand((B, H, n, d), torch.float16, 1800 + s, -1, 1, 0.125)
                      for s, n in enumerate((Nq, Nk, Nk, Nq)))
        vis = torch.from_numpy(_visible(Nq, Nk, causal))
        sc = 0.7

        def loss(qd, kd, vd):
            o = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=vis, scale=float(np.float32(sc)))
            return float((o * g.double()).sum())
        dq, dk, dv = orc.attention_bwd(q, k, v, g, causal, sc, nthreads=1)
        base = [q.double(), k.double(), v.double()]
        h = 1e-5
        for which, grad in enumerate((dq, dk, dv)):
            fd = np.zeros_like(grad)
            for idx in np.ndindex(*grad.shape):
                plus = [t.clone() for t in base]
                minus = [t.clone() for t in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
            _close(grad, fd, 1e-8, f"finite differences input {which} causal={causal}")


def pin_bwd_scale_zero(orc):
    """scale = 0: uniform weights, so dQ = dK = 0 and dV_j = sum over rows i that see
    key j of dO_i / |V_i|."""
    for causal in (False, True):
        B, H, Nq, Nk, d = 1, 1, 10, 7, 8
        q, k, v, g = (_rand((B, H, n, d), torch.bfloat16, 1900 + s) for s, n in enumerate((Nq, Nk, Nk, Nq)))
        dq, dk, dv = orc.attention_bwd(q, k, v, g, causal, 0.0, nthreads=1)
        vis = _visible(Nq, Nk, causal).astype(np.float64)
        cnt = vis.sum(axis=1)
        w = vis / np.maximum(cnt, 1)[:, None]
        _close(dq, np.zeros_like(dq), 0.0, "scale 0 dQ")
        _close(dk, np.zeros_like(dk), 0.0, "scale 0 dK")
        _close(dv[0, 0], w.T @ g.double().numpy()[0, 0], 1e-14, f"scale 0 dV causal={causal}")


def pin_bwd_key_gradient_sums_to_zero(orc):
    """Every row of dS sums to 0 (P o (dP - rowsum(dP o P))), so sum_j dK_j = 0: the
    loss does not change when one vector is added to every key."""
    for causal in (False, True):
        B, H, Nq, Nk, d = 2, 2, 11, 9, 16
        q, k, v, g = (_rand((B, H, n, d), torch.float16, 2000 + s) for s, n in enumerate((Nq, Nk, Nk, Nq)))
        _, dk, _ = orc.attention_bwd(q, k, v, g, causal, 0.4, nthreads=1)
        _close(dk.sum(axis=2), np.zeros((B, H, d)), 1e-12, f"sum of dK causal={causal}")


def pin_bwd_rows(orc):
    """Selected query and key rows equal the same rows of the full result."""
    B, H, Nq, Nk, d = 2, 2, 9, 12, 8
    q, k, v, g = (_rand((B, H, n, d), torch.float16, 2100 + s) for s, n in enumerate((Nq, Nk, Nk, Nq)))
    dq, dk, dv = orc.attention_bwd(q, k, v, g, True, 0.3, nthreads=1)
    qr, kr = np.array([0, 5, 20, 35]), np.array([3, 11, 30, 47])
    sq, sk, sv = orc.attention_bwd(q, k, v, g, True, 0.3, q_rows=qr, k_rows=kr, nthreads=2)
    _close(sq, dq.reshape(-1, d)[qr], 0.0, "bwd selected dQ rows")
    _close(sk, dk.reshape(-1, d)[kr], 0.0, "bwd selected dK rows")
    _close(sv, dv.reshape(-1, d)[kr], 0.0, "bwd selected dV rows")


# -- paged K/V cache (Ringi, "Lecture 25", section 8.3, PagedAttention question) --
def _paged_from_contiguous(k, lens, page_size, order):
    """Pin-side paging of contiguous k [B, H_kv, N, d]: sequence b's logical page j
    goes to physical page order[next free]; returns the cache [P, page_size,
    H_kv, d] (unused rows zero) and the block table."""
    B, H_kv, N, d = k.shape
    npg = [-(-n // page_size) for n in lens]
    P = sum(npg)
    cache = torch.zeros((P, page_size, H_kv, d), dtype=k.dtype)
    table = np.full((B, max(1, max(npg))), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        for j in range(npg[b]):
            phys = order[nxt]
            nxt += 1
            table[b, j] = phys
            for r in range(page_size):
                t = j * page_size + r
                if t < lens[b]:
                    cache[phys, r] = k[b, :, t]
    return cache, table


def pin_paged_matches_contiguous(orc):
    """Decode over a shuffled paged cache equals decode over the same keys laid
    out contiguously (per sequence, grouped heads)."""
    B, H, H_kv, N, d, ps = 3, 4, 2, 23, 16, 4
    lens = [23, 9, 1]
    for dt in DTYPES:
        q = _rand((B, H, d), dt, 501)
        k = _rand((B, H_kv, N, d), dt, 502)
        v = _rand((B, H_kv, N, d), dt, 503)
        P = sum(-(-n // ps) for n in lens)
        order = list(np.random.default_rng(504).permutation(P))
        kc, table = _paged_from_contiguous(k, lens, ps, order)
        vc, _ = _paged_from_contiguous(v, lens, ps, order)
        o, lse = orc.attention_paged(q, kc, vc, table, lens, 0.3, nthreads=2)
        for b in range(B):
            n = lens[b]
            ro, rl = orc.attention_gqa(q[b:b + 1, :, None, :].contiguous(), k[b:b + 1, :, :n].contiguous(),
                                       v[b:b + 1, :, :n].contiguous(), False, 0.3, nthreads=1)
            _close(o[b], ro.reshape(H, d), 1e-12, f"paged O, sequence {b}, {dt}")
            _close(lse[b], rl.reshape(H), 1e-12, f"paged LSE, sequence {b}, {dt}")


def pin_paged_brute_force(orc):
    """A tiny paged decode computed by hand: page lookup, dot products and a
    softmax with math.exp, in Python floats."""
    ps, d, H, H_kv = 2, 3, 2, 1
    lens = [3, 4]
    # values on a 1/4 grid are exact in fp16 and bf16
    kc = _rand((5, ps, H_kv, d), torch.float16, 511, -2, 2, 0.25)
    vc = _rand((5, ps, H_kv, d), torch.float16, 512, -2, 2, 0.25)
    q = _rand((2, H, d), torch.float16, 513, -2, 2, 0.25)
    table = np.array([[4, 1], [0, 3]], dtype=np.int32)
    scale = 0.625   # exact in float32, the type the oracle receives
    o, lse = orc.attention_paged(q, kc, vc, table, lens, scale, nthreads=1)
    for b in range(2):
        for h in range(H):
            keys, vals = [], []
            for t in range(lens[b]):
                page, row = int(table[b][t // ps]), t % ps
                keys.append([float(x) for x in kc[page, row, 0]])
                vals.append([float(x) for x in vc[page, row, 0]])
            qq = [float(x) for x in q[b, h]]
            sc = [scale * sum(a * c for a, c in zip(qq, kk)) for kk in keys]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            l = sum(w)
            exp_o = [sum(wi * vv[t] for wi, vv in zip(w, vals)) / l for t in range(d)]
            _close(o[b, h], exp_o, 1e-12, f"paged brute-force O ({b}, {h})")
            _close(lse[b, h], m + math.log(l), 1e-12, f"paged brute-force LSE ({b}, {h})")


def pin_paged_empty_sequence(orc):
    """A sequence with no cached keys gives O = 0 and LSE = -inf; the others are
    unaffected."""
    q = _rand((2, 2, 8), torch.bfloat16, 521)
    kc = _rand((2, 4, 1, 8), torch.bfloat16, 522)
    vc = _rand((2, 4, 1, 8), torch.bfloat16, 523)
    table = np.array([[0, 1], [-1, -1]], dtype=np.int32)
    o, lse = orc.attention_paged(q, kc, vc, table, [6, 0], 0.5, nthreads=1)
    _close(o[1], np.zeros((2, 8)), 0.0, "paged empty sequence O")
    assert np.all(np.isneginf(lse[1])), "paged empty sequence LSE must be -inf"
    o1, l1 = orc.attention_paged(q[:1].contiguous(), kc, vc, table[:1], [6], 0.5, nthreads=1)
    _close(o[0], o1[0], 0.0, "paged O unaffected by an empty neighbour")
    _close(lse[0], l1[0], 0.0, "paged LSE unaffected by an empty neighbour")


def pin_paged_splits(orc):
    """Paged partials split each sequence into chunks of ceil(len / S) keys
    (10 keys, S = 4: [0,3) [3,6) [6,9) [9,10)); they merge back to the whole."""
    B, H, H_kv, d, ps = 1, 2, 1, 8, 4
    n, S = 10, 4
    q = _rand((B, H, d), torch.float16, 531)
    k = _rand((B, H_kv, n, d), torch.float16, 532)
    v = _rand((B, H_kv, n, d), torch.float16, 533)
    kc, table = _paged_from_contiguous(k, [n], ps, [2, 0, 1])
    vc, _ = _paged_from_contiguous(v, [n], ps, [2, 0, 1])
    op, lp = orc.split_partials_paged(q, kc, vc, table, [n], 0.4, S, nthreads=1)
    for s, kr in enumerate([(0, 3), (3, 6), (6, 9), (9, 10)]):
        ro, rl = orc.attention_gqa(q[:, :, None, :].contiguous(), k, v, False, 0.4, key_range=kr, nthreads=1)
        _close(op[s], ro, 1e-12, f"paged split {s} O")
        _close(lp[s], rl, 1e-12, f"paged split {s} LSE")
    oc, lc = orc.combine(op, lp)
    o, lse = orc.attention_paged(q, kc, vc, table, [n], 0.4, nthreads=1)
    _close(oc.reshape(H, d), o[0], 1e-12, "paged combined O")
    _close(lc.reshape(H), lse[0], 1e-12, "paged combined LSE")


# -- packed split-KV decode (Ringi, "Lecture 25", section 7; LLM Infra Atlas, section 2) --
def pin_varlen_decode_splits(orc):
    """Packed-sequence partials split each sequence into chunks of ceil(len / S)
    keys (10 keys, S = 4: [0,3) [3,6) [6,9) [9,10); 2 keys: [0,1) [1,2) and two
    empty splits); every chunk equals attention over that key range of the
    sequence alone, and the merged partials equal varlen attention with one query
    row per sequence."""
    H, H_kv, d, S = 4, 2, 8, 4
    lens = [10, 0, 2]
    B, total = len(lens), sum(lens)
    for dt in DTYPES:
        q = _rand((B, H, d), dt, 541)
        k = _rand((total, H_kv, d), dt, 542)
        v = _rand((total, H_kv, d), dt, 543)
        cu = [0, 10, 10, 12]
        op, lp = orc.split_partials_varlen(q, k, v, cu, 0.35, S, nthreads=1)
        ranges = {0: [(0, 3), (3, 6), (6, 9), (9, 10)], 2: [(0, 1), (1, 2), (2, 2), (2, 2)]}
        for b, rs in ranges.items():
            kb = k[cu[b]:cu[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
            vb = v[cu[b]:cu[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
            for s_, kr in enumerate(rs):
                if kr[0] == kr[1]:
                    assert np.all(op[s_, b] == 0) and np.all(np.isneginf(lp[s_, b])), "empty split"
                    continue
                ro, rl = orc.attention_gqa(q[b:b + 1, :, None, :].contiguous(), kb, vb, False, 0.35,
                                           key_range=kr, nthreads=1)
                _close(op[s_, b], ro[0], 1e-12, f"varlen split {s_} O, sequence {b}, {dt}")
                _close(lp[s_, b], rl[0], 1e-12, f"varlen split {s_} LSE, sequence {b}, {dt}")
        assert np.all(op[:, 1] == 0) and np.all(np.isneginf(lp[:, 1])), "empty sequence gives empty splits"
        oc, lc = orc.combine(op, lp)
        ro, rl = orc.attention_varlen(q, k, v, list(range(B + 1)), cu, False, 0.35, nthreads=1)
        _close(oc.reshape(B, H, d), ro, 1e-12, f"varlen combined O, {dt}")
        _close(lc.reshape(B, H), rl.T, 1e-12, f"varlen combined LSE, {dt}")


def pin_varlen_decode_matches_paged(orc):
    """The same keys as packed sequences and as a shuffled paged cache (pages of
    3 rows) give the same partials: two independent ways of locating a
    sequence's keys."""
    H, H_kv, d, S, ps = 2, 1, 16, 3, 3
    lens = [7, 1, 5]
    B, N = len(lens), max(lens)
    q = _rand((B, H, d), torch.float16, 551)
    kd = _rand((B, H_kv, N, d), torch.float16, 552)
    vd = _rand((B, H_kv, N, d), torch.float16, 553)
    # packed rows of each sequence, back to back
    k = torch.cat([kd[b, :, :n].permute(1, 0, 2) for b, n in enumerate(lens)]).contiguous()
    v = torch.cat([vd[b, :, :n].permute(1, 0, 2) for b, n in enumerate(lens)]).contiguous()
    cu = [0, 7, 8, 13]
    P = sum(-(-n // ps) for n in lens)
    order = list(np.random.default_rng(554).permutation(P))
    kc, table = _paged_from_contiguous(kd, lens, ps, order)
    vc, _ = _paged_from_contiguous(vd, lens, ps, order)
    op, lp = orc.split_partials_varlen(q, k, v, cu, 0.25, S, nthreads=1)
    pp, pl = orc.split_partials_paged(q, kc, vc, table, lens, 0.25, S, nthreads=1)
    _close(op, pp, 0.0, "packed vs paged partial O")
    _close(lp, pl, 0.0, "packed vs paged partial LSE")


VARLEN_DECODE_PINS = [pin_varlen_decode_splits, pin_varlen_decode_matches_paged]


# -- FP8 (e4m3) inputs with per-block scales (Ringi, "Lecture 25", section 5.4) --
def pin_e4m3_decode(orc=None):
    """Values the e4m3 format definition fixes (OCP 8-bit floating point, E4M3FN:
    bias 7, 3 mantissa bits, subnormals m * 2^-9, S.1111.111 NaN, max 448)."""
    from oracle import fp8
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in known.items():
        got = float(fp8.decode_e4m3(np.array([code], dtype=np.uint8))[0])
        assert got == val, f"e4m3 0x{code:02x} decodes to {got}, not {val}"
    assert np.isnan(fp8.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all(), "e4m3 NaN patterns"
    pos = fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "e4m3 positive values must increase with the code"


def pin_e4m3_encode(orc=None):
    """Round to nearest, ties to the even code: every finite value maps back to
    its code, midpoints to the even neighbour, points just off a midpoint to the
    nearer one; the sign bit follows the input."""
    from oracle import fp8
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = fp8.decode_e4m3(codes)
    assert np.array_equal(fp8.encode_e4m3(vals), codes), "e4m3 round trip"
    pos = fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mid = (pos[1:] + pos[:-1]) / 2
    lo_code = np.arange(0x7E)
    even = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    assert np.array_equal(fp8.encode_e4m3(mid), even.astype(np.uint8)), "e4m3 ties to even"
    eps = (pos[1:] - pos[:-1]) * 1e-6
    assert np.array_equal(fp8.encode_e4m3(mid - eps), lo_code.astype(np.uint8)), "e4m3 below a midpoint"
    assert np.array_equal(fp8.encode_e4m3(mid + eps), (lo_code + 1).astype(np.uint8)), "e4m3 above a midpoint"
    assert np.array_equal(fp8.encode_e4m3(-mid[10:20]), even[10:20].astype(np.uint8) | 0x80), "e4m3 sign"


def pin_fp8_quantize_blocks(orc=None):
    """Per-block quantization: descale = amax / 448, the largest element of a
    block maps to +-448, every value lands within the e4m3 rounding of the
    original, an all-zero block gets descale 1."""
    from oracle import fp8
    x = _rand((2, 300, 16), torch.bfloat16, 541) * 3
    x[1, 256:] = 0
    codes, dsc = fp8.quantize_blocks(x, 128)
    assert codes.shape == (2, 300, 16) and dsc.shape == (2, 3)
    xf = x.float().numpy()
    for g in range(2):
        for b in range(3):
            blk = xf[g, b * 128:(b + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            if amax == 0:
                assert dsc[g, b] == 1.0 and not codes[g, b * 128:(b + 1) * 128].any(), "zero block"
                continue
            assert dsc[g, b] == amax / np.float32(448.0), f"descale of block ({g}, {b})"
            k = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert codes[g, b * 128 + k[0], k[1]] & 0x7F == 0x7E, "block maximum must reach 448"
    deq = fp8.dequantize(codes, dsc, 128)
    # e4m3 unit roundoff 2^-4 for normals; below 2^-6 * descale the spacing is 2^-9 * descale
    tol = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * dsc.astype(np.float64)[:, np.arange(300) // 128][:, :, None])
    assert np.all(np.abs(deq - xf) <= tol * (1 + 1e-6)), "quantized values off by more than the e4m3 rounding"


def pin_fp8_attention_matches_fp16(orc):
    """With power-of-two scales every dequantized e4m3 value is exact in fp16, so
    FP8 attention must equal the fp16 oracle on those values (per-block Q and K
    scales, per-head V scales, grouped heads, causal with Nq != Nk)."""
    from oracle import fp8
    B, H, H_kv, Nq, Nk, d = 1, 4, 2, 200, 260, 16
    g = torch.Generator().manual_seed(551)
    small = np.array([c for c in range(256) if abs(fp8.decode_e4m3(np.array([c], np.uint8))[0]) <= 2.0],
                     dtype=np.uint8)
    pick = lambda shape: small[torch.randint(0, small.size, shape, generator=g).numpy()]   # noqa: E731
    q8, k8, v8 = pick((B, H, Nq, d)), pick((B, H_kv, Nk, d)), pick((B, H_kv, Nk, d))
    pw = np.array([2.0 ** -3, 0.5, 1.0, 4.0], dtype=np.float32)
    qd = pw[torch.randint(0, 4, (B, H, 2), generator=g).numpy()]
    kd = pw[torch.randint(0, 4, (B, H_kv, 3), generator=g).numpy()]
    vd = pw[torch.randint(0, 4, (B, H_kv), generator=g).numpy()]
    qx = fp8.dequantize(q8.reshape(B * H, Nq, d), qd.reshape(B * H, 2), 128).reshape(B, H, Nq, d)
    kx = fp8.dequantize(k8.reshape(B * H_kv, Nk, d), kd.reshape(B * H_kv, 3), 128).reshape(B, H_kv, Nk, d)
    vx = fp8.decode_e4m3(v8) * vd[:, :, None, None]
    q16, k16, v16 = (torch.from_numpy(t).half() for t in (qx, kx, vx))
    assert np.array_equal(q16.double().numpy(), qx) and np.array_equal(v16.double().numpy(), vx), "not exact in fp16"
    for causal in (False, True):
        o, lse, amag, _ = fp8.attention_fp8(q8, k8, v8, qd, kd, vd, causal, 0.3)
        ro, rl = orc.attention_gqa(q16, k16, v16, causal, 0.3, nthreads=2)
        _close(o, ro, 1e-12, f"fp8 attention O causal={causal}")
        _close(lse, rl, 1e-12, f"fp8 attention LSE causal={causal}")
        assert np.all(amag + 1e-12 >= np.abs(o)), "sum p|v|/l bounds |O|"


def pin_fp8_error_terms(orc=None):
    """A, U and R of one row worked by hand.  Query (1, 0, ...), keys with first
    coordinates 0, -11 and -9 (all exact e4m3 codes, scales 1), scale sigma =
    float32(ln 2): the scores are 0, -11 sigma, -9 sigma, so the weights relative
    to the maximum are p = (1, e^-11sigma, e^-9sigma) ~ (1, 2^-11, 2^-9); only the
    second lies below 2^-10.  Values v_j = (1, 2, -4) in the first column and
    (0, 0, 0.5) in the second:
        l = 1 + p1 + p2;  O = ((1 + 2 p1 - 4 p2) / l, 0.5 p2 / l)
        A = ((1 + 2 p1 + 4 p2) / l, 0.5 p2 / l);  U = (2 / l, 0)
        R = (sqrt(2^-8 + (2^-14 * 2)^2 + (2^-4 p2 * 4)^2) / l, 2^-4 p2 * 0.5 / l)
    (R's rounding bound is e_j = max(2^-4 p_j, 2^-14): 2^-4 for the largest
    weight, 2^-14 for p1 < 2^-10, 2^-4 p2 for p2)."""
    from oracle import fp8
    d = 16
    code = lambda x: int(fp8.encode_e4m3(np.array([x]))[0])      # noqa: E731
    q8 = np.zeros((1, 1, 1, d), dtype=np.uint8)
    q8[0, 0, 0, 0] = code(1.0)
    k8 = np.zeros((1, 1, 3, d), dtype=np.uint8)
    v8 = np.zeros((1, 1, 3, d), dtype=np.uint8)
    for j, (kk, v0, v1) in enumerate(((0.0, 1.0, 0.0), (-11.0, 2.0, 0.0), (-9.0, -4.0, 0.5))):
        k8[0, 0, j, 0], v8[0, 0, j, 0], v8[0, 0, j, 1] = code(kk), code(v0), code(v1)
    one = lambda *shape: np.ones(shape, dtype=np.float32)       # noqa: E731
    sig = float(np.float32(math.log(2.0)))
    o, lse, A, U, R = fp8.attention_fp8(q8, k8, v8, one(1, 1, 1), one(1, 1, 1), one(1, 1), False,
                                        math.log(2.0), spread=True)
    p1, p2 = math.exp(-11 * sig), math.exp(-9 * sig)
    assert p1 < 2.0 ** -10 <= p2
    l = 1 + p1 + p2
    want = {
        "O": (o, [(1 + 2 * p1 - 4 * p2) / l, 0.5 * p2 / l]),
        "A": (A, [(1 + 2 * p1 + 4 * p2) / l, 0.5 * p2 / l]),
        "U": (U, [2 / l, 0.0]),
        "R": (R, [math.sqrt(2.0 ** -8 + (2.0 ** -14 * 2) ** 2 + (2.0 ** -4 * p2 * 4) ** 2) / l,
                  2.0 ** -4 * p2 * 0.5 / l]),
    }
    for name, (got, exp) in want.items():
        _close(got[0, 0, 0, :2], exp, 1e-15, f"fp8 {name}")
        assert not np.any(got[0, 0, 0, 2:]), f"fp8 {name}: columns with zero values"
    _close(lse[0, 0, 0], math.log(l), 1e-15, "fp8 LSE")


FP8_PINS = [pin_e4m3_decode, pin_e4m3_encode, pin_fp8_quantize_blocks, pin_fp8_attention_matches_fp16,
            pin_fp8_error_terms]

ALL_PINS = [pin_library_reference, pin_torch_sdpa, pin_identical_keys, pin_first_causal_row,
            pin_scale_zero, pin_key_shift, pin_value_shift, pin_key_permutation, pin_empty_rows,
            pin_dominant_score, pin_decoders, pin_split_combine, pin_combine_closed_form,
            pin_worked_examples, pin_varlen_per_sequence, pin_varlen_grouped_heads, pin_varlen_rows,
            pin_dense_grouped_heads, pin_bwd_autograd, pin_bwd_gqa_autograd, pin_bwd_varlen_autograd,
            pin_bwd_finite_differences, pin_bwd_scale_zero, pin_bwd_key_gradient_sums_to_zero, pin_bwd_rows,
            pin_paged_matches_contiguous, pin_paged_brute_force, pin_paged_empty_sequence, pin_paged_splits]
