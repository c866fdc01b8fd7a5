"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * prefill: fa_fwd on the long-context causal workload
    (B=1, H=32, Nq=Nk=8192, d=128, bf16, N(0,1)*0.5) -- the headline `value` --
    and on the two other prefill workloads (prefill_d64: B=16 H=16 N=1024 d=64
    fp16 non-causal; causal_d128: B=4 H=16 N=2048 d=128 fp16 causal), and
  * decode: fa_fwd_splitkv + fa_splitkv_combine on the decode workload
    (B=8, H=32, Nq=1, Nk=32768, d=128, fp16, 16 splits), the same with the 32
    query heads sharing 8 K/V heads (decode_gqa), and the same again with K/V in
    a paged cache of 16-row pages scattered by a seeded permutation
    (decode_paged), and one query row per sequence over 16 packed sequences of
    keys (decode_varlen: lengths log-uniform in [512, 32768], 129054 keys, the
    32 query heads on 8 K/V heads, 16 splits per sequence), and
  * bwd: fa_bwd on the long-context causal workload (dO ~ N(0,1)), and
    bwd_varlen: fa_bwd_varlen on the packed varlen_gqa sequences, and
  * fp8: fa_fwd_fp8 on the long-context workload's inputs quantized to e4m3
    per block (quantized once, untimed), and
  * varlen: fa_fwd_varlen on 16 packed causal sequences (lengths log-uniform in
    [64, 8192], 20752 tokens) with 32 query heads sharing 8 K/V heads, d=128, bf16.
`value` is the prefill throughput in TFLOP/s with FLOPs = 4*B*H*Nq*Nk*d, halved
for causal (Ringi, "Lecture 25", experiment 4); decode is reported as HBM GB/s
over the bytes the method must move (Q + K + V + O + LSE); varlen as TFLOP/s with
the same FLOP convention summed over its sequences.

Each kernel is timed with HIP events recorded on the stream it is launched on;
every block reports the mean (used for the rooflines), median and minimum over
the timed steps.  A decode's split kernel and its combine are each timed alone
(the combine queued behind the split kernel), then once more as one unit with
no marker between them: that unit is the decode line's time.  The default run
times enough steps for a timed region of a few seconds.  The CPU baseline
times the fp64 oracle on the prefill rows (all of them by default: about 5 s on
16 threads).  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_22_amd import fa                          # noqa: E402
from exact_attention_22_amd.inputs import BY_NAME, make_paged, make_qkv, make_varlen, make_varlen_decode  # noqa: E402

METRIC = "attn fwd TFLOPS & % MFMA peak (fp16 d=128 causal N=8K); decode HBM GB/s"
PEAK_TFLOPS = 2500.0         # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
CUS, FLOP_PER_CU_CLK = 256, 4096   # dense bf16/fp16 MFMA FLOPs per CU per clock (2.5 PF / 256 / 2.4 GHz)
PROFILES = os.path.join(ROOT, "profiles")
FWD_SOURCES = ["exact_attention_22_amd/csrc/fa_fwd.hip", "exact_attention_22_amd/csrc/fa_device.h"]
DEC_SOURCES = ["exact_attention_22_amd/csrc/fa_decode.hip", "exact_attention_22_amd/csrc/fa_device.h"]
BWD_SOURCES = ["exact_attention_22_amd/csrc/fa_bwd.hip", "exact_attention_22_amd/csrc/fa_device.h"]


def attn_flops(B, H, Nq, Nk, d, causal):
    """4*B*H*Nq*Nk*d, halved for causal (the pages' TFLOPS convention)."""
    f = 4.0 * B * H * Nq * Nk * d
    return f / 2 if causal else f


def attn_bytes(B, H, Nq, Nk, d, elem=2):
    """Q + K + V + O (elem bytes each) + LSE (fp32): each tensor touched once."""
    return elem * (2 * B * H * Nq * d + 2 * B * H * Nk * d) + 4 * B * H * Nq


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile(name, src_hash, hash_key="source_hash"):
    """key = value lines of profiles/<name>.txt, if that file was taken on this source."""
    path = os.path.join(PROFILES, f"{name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                line = line[1:].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                v = v.rsplit("=", 1)[-1].strip()      # derived lines: "name = formula = value"
                vals[k.strip()] = v.split()[0] if v else ""
    return vals if vals.get(hash_key) == src_hash else None


def read_traffic(kernel_key, src_hash):
    """HBM bytes per launch from profiles/traffic_<key>.txt, if taken on this source."""
    vals = read_profile(f"traffic_{kernel_key}", src_hash)
    try:
        return float(vals["hbm_bytes_per_launch"]) if vals else None
    except (KeyError, ValueError):
        return None


def measured_clock_ghz(counters_name, src_hash):
    """Shader clock under the kernel, GRBM_GUI_ACTIVE / 8 XCDs / duration, from a
    committed counter summary taken on this source (else None)."""
    vals = read_profile(counters_name, src_hash, hash_key="fwd source_hash")
    try:
        return float(vals["gpu_clock_GHz"]) if vals else None
    except (KeyError, ValueError):
        return None


def host_cores():
    """(threads the CPU baseline uses, cores of the host, cores this process may run on,
    CPU quota of its cgroup or None).  The baseline uses every core this process
    may run on, capped by the cgroup quota and by the 16-CPU share one GPU's job
    gets on the GPU hosts."""
    host = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = host
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
            if q != "max":
                quota = max(1, int(int(q) / int(period)))
    except (OSError, ValueError):
        pass
    use = min(affinity, quota or affinity, 16)
    return use, host, affinity, quota


def hbm_copy_rate(dev, stream, mib=1024, reps=10):
    """Device-to-device copy of `mib` MiB by torch, timed with HIP events on the
    stream: a measured ceiling for the streaming (decode) kernels, counted as
    read + write bytes."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    moved = 2 * n * 4
    del src, dst
    gbs = moved / (ms * 1e-3) / 1e9
    return {"GB_per_s": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS, "bytes_per_copy": moved, "us_per_copy": ms * 1e3,
            "what": f"torch device-to-device copy of {mib} MiB, read + write bytes, mean of {reps}"}


def cpu_baseline(q, k, v, w, target_rows):
    """Time the fp64 oracle on evenly spaced rows of the prefill workload."""
    import numpy as np
    from oracle import oracle
    orc = oracle.get()
    nthreads, host, affinity, quota = host_cores()
    total = w.B * w.H * w.Nq
    whole = target_rows <= 0 or target_rows >= total
    rows = np.arange(total, dtype=np.int64) if whole else \
        np.linspace(0, total - 1, num=target_rows).astype(np.int64)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    orc.attention(qc, kc, vc, w.causal, w.scale, rows=None if whole else rows, nthreads=nthreads)
    dt = time.perf_counter() - t0
    i = rows % w.Nq
    visible = np.minimum(w.Nk, i + (w.Nk - w.Nq) + 1) if w.causal else np.full_like(i, w.Nk)
    flops = float(np.sum(visible)) * w.d * 4.0
    what = (f"every query row of {w.name} ({total})" if whole else
            f"{len(rows)} evenly spaced query rows of {w.name} (of {total})")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "cores_host": host, "cores_affinity": affinity, "cpu_quota": quota, "seconds": dt,
            "sample": f"{what}; {flops / 1e9:.1f} GFLOP of visible work in {dt:.1f} s, fp64, {nthreads} threads"}


def stats_us(times_ms):
    return {"avg_us": 1e3 * sum(times_ms) / len(times_ms), "median_us": 1e3 * statistics.median(times_ms),
            "min_us": 1e3 * min(times_ms)}


LEGS = ["prefill", "prefill_d64", "causal_d128", "decode", "decode_gqa", "decode_paged", "decode_varlen", "varlen",
        "bwd", "bwd_varlen", "fp8"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all"] + LEGS, default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=0, help="query rows the CPU baseline times (0: all)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also copy N MiB once (a plain copy of known size for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    fa.lib()
    on = {leg: args.only in ("all", leg) for leg in LEGS}

    wp, wd, wv, wg = BY_NAME["long_causal"], BY_NAME["decode"], BY_NAME["varlen_gqa"], BY_NAME["decode_gqa"]
    wpg, w64, w128 = BY_NAME["decode_paged"], BY_NAME["prefill_d64"], BY_NAME["causal_d128"]
    wdv = BY_NAME["decode_varlen"]
    stream = torch.cuda.current_stream()
    calls = {}    # leg -> list of (sub-leg name, callable); each sub-leg is timed by its own events

    if on["prefill"] or on["bwd"]:
        q, k, v = make_qkv(wp, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
        calls["prefill"] = [("fwd", lambda: fa.fwd(q, k, v, causal=wp.causal, scale=wp.scale, out=o, lse=lse,
                                                  stream=stream))]
    for name, w in (("prefill_d64", w64), ("causal_d128", w128)):
        if on[name]:
            tq, tk, tv = make_qkv(w, device=dev)
            to, tl = torch.empty_like(tq), torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
            calls[name] = [("fwd", lambda tq=tq, tk=tk, tv=tv, to=to, tl=tl, w=w:
                            fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out=to, lse=tl, stream=stream))]
    if on["decode"]:
        dq, dk, dv = make_qkv(wd, device=dev)
        S = wd.splits
        op = torch.empty((S, wd.B, wd.H, wd.Nq, wd.d), dtype=torch.float32, device=dev)
        lp = torch.empty((S, wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
        do_ = torch.empty_like(dq)
        dlse = torch.empty((wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
        split_d = lambda: fa.fwd_splitkv(dq, dk, dv, S, causal=wd.causal, scale=wd.scale, o_part=op,  # noqa: E731
                                         lse_part=lp, stream=stream)
        comb_d = lambda: fa.splitkv_combine(op, lp, wd.dtype, out=do_, lse=dlse, stream=stream)  # noqa: E731
        calls["decode"] = [("split", split_d), ("combine", comb_d), ("total", lambda: (split_d(), comb_d()))]
    if on["decode_gqa"]:
        gq, gk, gv = make_qkv(wg, device=dev)
        gop = torch.empty((wg.splits, wg.B, wg.H, wg.Nq, wg.d), dtype=torch.float32, device=dev)
        glp = torch.empty((wg.splits, wg.B, wg.H, wg.Nq), dtype=torch.float32, device=dev)
        go = torch.empty_like(gq)
        glse = torch.empty((wg.B, wg.H, wg.Nq), dtype=torch.float32, device=dev)
        split_g = lambda: fa.fwd_splitkv_gqa(gq, gk, gv, wg.splits, causal=wg.causal, scale=wg.scale,  # noqa: E731
                                             o_part=gop, lse_part=glp, stream=stream)
        comb_g = lambda: fa.splitkv_combine(gop, glp, wg.dtype, out=go, lse=glse, stream=stream)  # noqa: E731
        calls["decode_gqa"] = [("split", split_g), ("combine", comb_g), ("total", lambda: (split_g(), comb_g()))]
    if on["decode_paged"]:
        pq, pkc, pvc, pbt, psl = make_paged(wpg, device=dev)
        pop = torch.empty((wpg.splits, wpg.B, wpg.H, 1, wpg.d), dtype=torch.float32, device=dev)
        plp = torch.empty((wpg.splits, wpg.B, wpg.H, 1), dtype=torch.float32, device=dev)
        po = torch.empty((wpg.B, wpg.H, 1, wpg.d), dtype=wpg.dtype, device=dev)
        plse = torch.empty((wpg.B, wpg.H, 1), dtype=torch.float32, device=dev)
        split_p = lambda: fa.fwd_splitkv_paged(pq, pkc, pvc, pbt, psl, wpg.splits, scale=wpg.scale,  # noqa: E731
                                               o_part=pop, lse_part=plp, stream=stream)
        comb_p = lambda: fa.splitkv_combine(pop, plp, wpg.dtype, out=po, lse=plse, stream=stream)  # noqa: E731
        calls["decode_paged"] = [("split", split_p), ("combine", comb_p), ("total", lambda: (split_p(), comb_p()))]
    if on["decode_varlen"]:
        vdq, vdk, vdv, vdcu = make_varlen_decode(wdv, device=dev)
        vdop = torch.empty((wdv.splits, wdv.B, wdv.H, 1, wdv.d), dtype=torch.float32, device=dev)
        vdlp = torch.empty((wdv.splits, wdv.B, wdv.H, 1), dtype=torch.float32, device=dev)
        vdo = torch.empty((wdv.B, wdv.H, 1, wdv.d), dtype=wdv.dtype, device=dev)
        vdlse = torch.empty((wdv.B, wdv.H, 1), dtype=torch.float32, device=dev)
        split_v = lambda: fa.fwd_splitkv_varlen(vdq, vdk, vdv, vdcu, max(wdv.seqlens), wdv.splits,  # noqa: E731
                                                scale=wdv.scale, o_part=vdop, lse_part=vdlp, stream=stream)
        comb_v = lambda: fa.splitkv_combine(vdop, vdlp, wdv.dtype, out=vdo, lse=vdlse, stream=stream)  # noqa: E731
        calls["decode_varlen"] = [("split", split_v), ("combine", comb_v), ("total", lambda: (split_v(), comb_v()))]
    if on["varlen"]:
        vq, vk, vv, vcq, vck = make_varlen(wv, device=dev)
        vo = torch.empty_like(vq)
        vlse = torch.empty((wv.H, vq.shape[0]), dtype=torch.float32, device=dev)
        vmax = max(wv.seqlens)
        calls["varlen"] = [("fwd", lambda: fa.fwd_varlen(vq, vk, vv, vcq, vck, vmax, vmax, causal=wv.causal,
                                                         scale=wv.scale, out=vo, lse=vlse, stream=stream))]
    if on["bwd_varlen"]:
        bvq, bvk, bvv, bvcq, bvck = make_varlen(wv, device=dev)
        bvmax = max(wv.seqlens)
        bvo, bvlse = fa.fwd_varlen(bvq, bvk, bvv, bvcq, bvck, bvmax, bvmax, causal=wv.causal, scale=wv.scale)
        gen_v = torch.Generator(device=dev)
        gen_v.manual_seed(wv.seed + 100)
        bvdo = torch.randn(tuple(bvq.shape), generator=gen_v, device=dev, dtype=torch.float32).to(wv.dtype)
        bvdq, bvdk, bvdv = torch.empty_like(bvq), torch.empty_like(bvk), torch.empty_like(bvv)
        bvws = torch.empty(fa.bwd_workspace_bytes(1, wv.H, bvq.shape[0]) // 4, dtype=torch.float32, device=dev)
        calls["bwd_varlen"] = [("bwd", lambda: fa.bwd_varlen(bvq, bvk, bvv, bvo, bvlse, bvdo, bvcq, bvck, bvmax, bvmax,
                                                             causal=wv.causal, scale=wv.scale, dq=bvdq, dk=bvdk,
                                                             dv=bvdv, workspace=bvws, stream=stream))]
    if on["bwd"]:
        fa.fwd(q, k, v, causal=wp.causal, scale=wp.scale, out=o, lse=lse)
        gen = torch.Generator(device=dev)
        gen.manual_seed(wp.seed + 100)
        bdo = torch.randn(tuple(q.shape), generator=gen, device=dev, dtype=torch.float32).to(wp.dtype)
        bdq, bdk, bdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(fa.bwd_workspace_bytes(wp.B, wp.H, wp.Nq) // 4, dtype=torch.float32, device=dev)
        # the backward reads the forward's o and lse: keep them fixed while timing
        bo, blse = o.clone(), lse.clone()
        calls["bwd"] = [("bwd", lambda: fa.bwd(q, k, v, bo, blse, bdo, causal=wp.causal, scale=wp.scale, dq=bdq,
                                               dk=bdk, dv=bdv, workspace=bws, stream=stream))]
        if not on["prefill"]:
            del calls["prefill"]
    if on["fp8"]:
        # long_causal's inputs quantized per block (Q, K: 128 rows; V: per head), untimed
        fq, fk, fv = make_qkv(wp, device=dev)
        G = wp.B * wp.H
        f8 = [fa.quantize_fp8(t.reshape(G, wp.Nq, wp.d), br) for t, br in ((fq, 128), (fk, 128), (fv, wp.Nk))]
        del fq, fk, fv
        fq8, fk8, fv8 = (c.reshape(wp.B, wp.H, wp.Nq, wp.d) for c, _ in f8)
        fqd, fkd = f8[0][1].reshape(wp.B, wp.H, -1), f8[1][1].reshape(wp.B, wp.H, -1)
        fvd = f8[2][1].reshape(wp.B, wp.H)
        fo = torch.empty((wp.B, wp.H, wp.Nq, wp.d), dtype=torch.bfloat16, device=dev)
        flse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
        calls["fp8"] = [("fwd", lambda: fa.fwd_fp8(fq8, fk8, fv8, fqd, fkd, fvd, causal=wp.causal, scale=wp.scale,
                                                   out=fo, lse=flse, stream=stream))]
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    legs = [(leg, sub, fn) for leg in LEGS if leg in calls for sub, fn in calls[leg]]
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(rec):
        e = [ev() for _ in range(len(legs) + 1)]
        e[0].record(stream)
        for i, (_, _, fn) in enumerate(legs):
            fn()
            e[i + 1].record(stream)
        if rec is not None:
            rec.append(e)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    times = {}   # (leg, sub) -> per-step ms
    for i, (leg, sub, _) in enumerate(legs):
        times[(leg, sub)] = [r[i].elapsed_time(r[i + 1]) for r in recs]

    def leg_ms(leg, agg):
        """Per-step time of a whole leg (its sub-legs summed), aggregated."""
        per_step = [sum(times[(lg, s)][j] for lg, s, _ in legs if lg == leg) for j in range(len(recs))]
        return agg(per_step)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "timed_region_s": wall, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    cfg = {}
    mean = lambda xs: sum(xs) / len(xs)   # noqa: E731
    fwd_src = source_hash(FWD_SOURCES)
    clock = measured_clock_ghz("counters_fwd_long_causal", fwd_src)

    def prefill_block(leg, w, label, kernel):
        fl = attn_flops(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
        t = leg_ms(leg, mean)
        tf = fl / (t * 1e-3) / 1e12
        blk = {"TFLOP_per_s": tf, "pct_mfma_peak": 100.0 * tf / PEAK_TFLOPS, "flop_per_launch": fl,
               "TFLOP_per_s_at_median": fl / (leg_ms(leg, statistics.median) * 1e-3) / 1e12,
               "TFLOP_per_s_at_min": fl / (leg_ms(leg, min) * 1e-3) / 1e12,
               **stats_us(times[(leg, "fwd")])}
        roof = {"bound": "mfma", "achieved": tf, "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_TFLOPS,
                "kernel": kernel, "avg_us": t * 1e3, "flop_per_launch": fl, "source_hash": fwd_src}
        cfg[leg] = {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                    "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp16", "causal": w.causal,
                    "input_scale": w.mult, "workload": label}
        return blk, roof

    if on["prefill"]:
        blk, roof = prefill_block("prefill", wp, "long_causal", "fwd_kernel<bf16, d=128, causal>")
        roof["traffic"] = read_traffic("fwd_long_causal", fwd_src)
        if clock:
            peak_clk = CUS * FLOP_PER_CU_CLK * clock * 1e9 / 1e12
            roof.update({"measured_clock_GHz": clock, "peak_at_measured_clock": peak_clk,
                         "frac_at_measured_clock": roof["achieved"] / peak_clk})
        out.update({"value": blk["TFLOP_per_s"], "unit": "TFLOP/s", "dtype": "bf16",
                    "pct_mfma_peak": blk["pct_mfma_peak"]})
        out["prefill"] = blk
        out["roofline"] = roof
        cfg["workload"] = ("long_causal: B=1 H=32 Nq=Nk=8192 d=128 bf16 causal (prefill, timed as value) + "
                           "decode: B=8 H=32 Nq=1 Nk=32768 d=128 fp16 16 splits")
    for leg, w, kernel in (("prefill_d64", w64, "fwd_kernel<fp16, d=64>"),
                           ("causal_d128", w128, "fwd_kernel<fp16, d=128, causal>")):
        if on[leg]:
            blk, roof = prefill_block(leg, w, leg, kernel)
            roof["traffic"] = read_traffic(f"fwd_{leg}", fwd_src)
            out[leg] = blk
            out[f"roofline_{leg}"] = roof
            if args.only == leg:
                out.update({"value": blk["TFLOP_per_s"], "unit": "TFLOP/s", "dtype": "f16"})
                cfg["workload"] = f"{leg}: B={w.B} H={w.H} Nq=Nk={w.Nq} d={w.d} fp16 causal={w.causal}"

    def decode_block(leg, total_bytes, split_bytes, kernel, traffic_key, extra=None):
        # the split kernel and the combine are each timed alone (the combine is queued
        # behind the split kernel, so its events see device time, not launch latency);
        # the total is split + combine timed again as one unit, with no marker between
        t_split, t = mean(times[(leg, "split")]), mean(times[(leg, "total")])
        blk = {"GB_per_s": total_bytes / (t * 1e-3) / 1e9, "hbm_frac": total_bytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "us_total": t * 1e3, "us_splitkv": t_split * 1e3, "us_combine": mean(times[(leg, "combine")]) * 1e3,
               "median_us_total": statistics.median(times[(leg, "total")]) * 1e3,
               "min_us_total": min(times[(leg, "total")]) * 1e3,
               "splitkv": stats_us(times[(leg, "split")]), "algorithmic_bytes": total_bytes, **(extra or {})}
        gbs = split_bytes / (t_split * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "traffic": read_traffic(traffic_key, source_hash(DEC_SOURCES)), "kernel": kernel}
        return blk, roof

    if on["decode"]:
        byts = attn_bytes(wd.B, wd.H, wd.Nq, wd.Nk, wd.d)
        split_bytes = byts - 2 * wd.B * wd.H * wd.d - 4 * wd.B * wd.H   # O and LSE are the combine's
        out["decode"], out["roofline_decode"] = decode_block(
            "decode", byts, split_bytes, "decode_kernel<fp16, d=128>", "decode",
            {"partials_bytes": fa.workspace_bytes(wd.B, wd.H, wd.Nq, wd.d, wd.splits)})
        if not on["prefill"]:
            out.update({"value": out["decode"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode: B=8 H=32 Nq=1 Nk=32768 d=128 fp16 16 splits"
        cfg["decode"] = {"B": wd.B, "H": wd.H, "Nq": wd.Nq, "Nk": wd.Nk, "d": wd.d, "dtype": "fp16",
                         "splits": wd.splits}
    if on["decode_gqa"]:
        # bytes the method must move: Q, O (B*H*d each), K, V (B*H_kv*Nk*d each), LSE
        gb = 2 * (2 * wg.B * wg.H * wg.d + 2 * wg.B * wg.H_kv * wg.Nk * wg.d) + 4 * wg.B * wg.H
        out["decode_gqa"], out["roofline_decode_gqa"] = decode_block(
            "decode_gqa", gb, gb - 2 * wg.B * wg.H * wg.d - 4 * wg.B * wg.H,
            "decode_kernel<fp16, d=128, 4 query heads and 8 wavefronts per workgroup>", "decode_gqa")
        cfg["decode_gqa"] = {"B": wg.B, "H": wg.H, "H_kv": wg.H_kv, "Nq": wg.Nq, "Nk": wg.Nk, "d": wg.d,
                             "dtype": "fp16", "splits": wg.splits}
        if args.only == "decode_gqa":
            out.update({"value": out["decode_gqa"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode_gqa: B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 fp16 16 splits"
    if on["decode_paged"]:
        # bytes the method must move: Q, O, K, V and LSE as decode_gqa, plus the
        # block table (B x pages per sequence int32) once
        kv = 2 * 2 * wpg.B * wpg.H_kv * wpg.Nk * wpg.d
        pgb = 2 * 2 * wpg.B * wpg.H * wpg.d + kv + 4 * wpg.B * wpg.H + 4 * pbt.numel()
        out["decode_paged"], out["roofline_decode_paged"] = decode_block(
            "decode_paged", pgb, pgb - 2 * wpg.B * wpg.H * wpg.d - 4 * wpg.B * wpg.H,
            "decode_paged_hg_kernel<fp16, 4 K/V heads and 16 wavefronts per workgroup>", "decode_paged")
        cfg["decode_paged"] = {"B": wpg.B, "H": wpg.H, "H_kv": wpg.H_kv, "Nq": 1, "Nk": wpg.Nk, "d": wpg.d,
                               "dtype": "fp16", "splits": wpg.splits, "page_size": wpg.page_size}
        if args.only == "decode_paged":
            out.update({"value": out["decode_paged"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode_paged: B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 fp16 16 splits, 16-row pages"
    if on["decode_varlen"]:
        # bytes the method must move: Q, O (B*H*d each), every sequence's K and V
        # once (total_k*H_kv*d each), LSE, and the B+1 offsets
        tk = sum(wdv.seqlens)
        vgb = 2 * 2 * wdv.B * wdv.H * wdv.d + 2 * 2 * tk * wdv.H_kv * wdv.d + 4 * wdv.B * wdv.H + 4 * (wdv.B + 1)
        out["decode_varlen"], out["roofline_decode_varlen"] = decode_block(
            "decode_varlen", vgb, vgb - 2 * wdv.B * wdv.H * wdv.d - 4 * wdv.B * wdv.H,
            "decode_kernel<fp16, d=128, 4 query heads and 8 wavefronts per workgroup, packed>", "decode_varlen")
        cfg["decode_varlen"] = {"sequences": wdv.B, "keys": tk, "max_seqlen_k": max(wdv.seqlens), "H": wdv.H,
                                "H_kv": wdv.H_kv, "Nq": 1, "d": wdv.d, "dtype": "fp16", "splits": wdv.splits}
        if args.only == "decode_varlen":
            out.update({"value": out["decode_varlen"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = ("decode_varlen: 16 packed sequences, 129054 keys, H=32 H_kv=8 Nq=1 d=128 fp16, "
                               "16 splits per sequence")
    if on["varlen"]:
        fl = sum(attn_flops(1, wv.H, n, n, wv.d, wv.causal) for n in wv.seqlens)
        t_var = leg_ms("varlen", mean)
        tf = fl / (t_var * 1e-3) / 1e12
        out["varlen_gqa"] = {"TFLOP_per_s": tf, "pct_mfma_peak": 100.0 * tf / PEAK_TFLOPS, "flop_per_launch": fl,
                             **stats_us(times[("varlen", "fwd")])}
        out["roofline_varlen"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": tf / PEAK_TFLOPS, "traffic": read_traffic("fwd_varlen_gqa", fwd_src),
                                  "kernel": "fwd_kernel<bf16, d=128, causal, varlen>"}
        cfg["varlen"] = {"sequences": wv.B, "tokens": sum(wv.seqlens), "max_seqlen": max(wv.seqlens),
                         "H": wv.H, "H_kv": wv.H_kv, "d": wv.d, "dtype": "bf16", "causal": True}
        if args.only == "varlen":
            out.update({"value": tf, "unit": "TFLOP/s", "dtype": "bf16"})
            cfg["workload"] = "varlen_gqa: 16 packed causal sequences, 20752 tokens, H=32 H_kv=8 d=128 bf16"
    if on["bwd"]:
        # algorithmic work of the backward: its five products (recompute S, dP, dV, dK,
        # dQ) = 2.5 x the forward's two
        fl = 2.5 * attn_flops(wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.causal)
        t_bwd = leg_ms("bwd", mean)
        tb = fl / (t_bwd * 1e-3) / 1e12
        out["bwd"] = {"TFLOP_per_s": tb, "pct_mfma_peak": 100.0 * tb / PEAK_TFLOPS, "flop_per_launch": fl,
                      "source_hash": source_hash(BWD_SOURCES), **stats_us(times[("bwd", "bwd")])}
        out["roofline_bwd"] = {"bound": "mfma", "achieved": tb, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": tb / PEAK_TFLOPS, "traffic": None,
                               "kernel": "bwd_delta + bwd_dkdv + bwd_dq <bf16, d=128, causal>"}
        cfg["bwd"] = {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d, "dtype": "bf16", "causal": True}
        if args.only == "bwd":
            out.update({"value": tb, "unit": "TFLOP/s", "dtype": "bf16"})
            cfg["workload"] = "bwd on long_causal: B=1 H=32 Nq=Nk=8192 d=128 bf16 causal"
    if on["bwd_varlen"]:
        fl = 2.5 * sum(attn_flops(1, wv.H, n, n, wv.d, wv.causal) for n in wv.seqlens)
        t_bv = leg_ms("bwd_varlen", mean)
        tbv = fl / (t_bv * 1e-3) / 1e12
        out["bwd_varlen"] = {"TFLOP_per_s": tbv, "pct_mfma_peak": 100.0 * tbv / PEAK_TFLOPS, "flop_per_launch": fl,
                             **stats_us(times[("bwd_varlen", "bwd")])}
        out["roofline_bwd_varlen"] = {"bound": "mfma", "achieved": tbv, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": tbv / PEAK_TFLOPS, "traffic": None,
                                      "kernel": "bwd_delta + bwd_dkdv + bwd_dq <bf16, d=128, causal, varlen>"}
        cfg["bwd_varlen"] = {"sequences": wv.B, "tokens": sum(wv.seqlens), "max_seqlen": max(wv.seqlens),
                             "H": wv.H, "H_kv": wv.H_kv, "d": wv.d, "dtype": "bf16", "causal": True}
        if args.only == "bwd_varlen":
            out.update({"value": tbv, "unit": "TFLOP/s", "dtype": "bf16"})
            cfg["workload"] = "bwd_varlen on varlen_gqa: 16 packed causal sequences, 20752 tokens, H=32 H_kv=8"
    if on["fp8"]:
        fl = attn_flops(wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.causal)
        t_f8 = leg_ms("fp8", mean)
        t8 = fl / (t_f8 * 1e-3) / 1e12
        out["fp8"] = {"TFLOP_per_s": t8, "pct_mfma_peak": 100.0 * t8 / PEAK_FP8_TFLOPS, "flop_per_launch": fl,
                      **stats_us(times[("fp8", "fwd")])}
        out["roofline_fp8"] = {"bound": "mfma", "achieved": t8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                               "frac": t8 / PEAK_FP8_TFLOPS, "traffic": None,
                               "kernel": "fwd_fp8_kernel<e4m3, d=128, causal>"}
        cfg["fp8"] = {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d, "dtype": "e4m3 in, bf16 out",
                      "causal": True, "scales": "Q, K per 128 rows; V per head"}
        if args.only == "fp8":
            out.update({"value": t8, "unit": "TFLOP/s", "dtype": "fp8"})
            cfg["workload"] = "fp8 on long_causal: B=1 H=32 Nq=Nk=8192 d=128 e4m3 causal"
    out["config"] = cfg
    if any(on[x] for x in ("decode", "decode_gqa", "decode_paged", "decode_varlen")):
        out["hbm_copy"] = hbm_copy_rate(dev, stream)
    if on["prefill"] and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(q, k, v, wp, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
