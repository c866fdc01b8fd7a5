"""Benchmark of the attention forward hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * prefill: fa_fwd on the long-context causal workload
    (B=1, H=32, Nq=Nk=8192, d=128, bf16, N(0,1)*0.5), and
  * decode: fa_fwd_splitkv + fa_splitkv_combine on the decode workload
    (B=8, H=32, Nq=1, Nk=32768, d=128, fp16, 16 splits), the same with the 32
    query heads sharing 8 K/V heads (decode_gqa), and the same again with K/V in
    a paged cache of 16-row pages scattered by a seeded permutation
    (decode_paged), and
  * bwd: fa_bwd on the long-context causal workload (dO ~ N(0,1)), and
  * fp8: fa_fwd_fp8 on the long-context workload's inputs quantized to e4m3
    per block (untimed), and
  * varlen: fa_fwd_varlen on 16 packed causal sequences (lengths log-uniform in
    [64, 8192], 20752 tokens) with 32 query heads sharing 8 K/V heads, d=128, bf16.
`value` is the prefill throughput in TFLOP/s with FLOPs = 4*B*H*Nq*Nk*d, halved
for causal (Ringi, "Lecture 25", experiment 4); decode is reported as HBM GB/s
over the bytes the method must move (Q + K + V + O + LSE); varlen as TFLOP/s with
the same FLOP convention summed over its sequences.

Each kernel is timed with HIP events recorded on the stream it is launched on.
The CPU baseline times the fp64 oracle on a bounded sample of prefill rows.
Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_22_amd import fa                          # noqa: E402
from exact_attention_22_amd.inputs import BY_NAME, make_paged, make_qkv, make_varlen     # noqa: E402

METRIC = "attn fwd TFLOPS & % MFMA peak (fp16 d=128 causal N=8K); decode HBM GB/s"
PEAK_TFLOPS = {torch.bfloat16: 2500.0, torch.float16: 2500.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PROFILES = os.path.join(ROOT, "profiles")
FWD_SOURCES = ["exact_attention_22_amd/csrc/fa_fwd.hip", "exact_attention_22_amd/csrc/fa_device.h"]
DEC_SOURCES = ["exact_attention_22_amd/csrc/fa_decode.hip", "exact_attention_22_amd/csrc/fa_device.h"]


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


def read_traffic(kernel_key, src_hash):
    """HBM bytes per launch from profiles/traffic_<key>.txt, if taken on this source."""
    path = os.path.join(PROFILES, f"traffic_{kernel_key}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(q, k, v, w, target_rows):
    """Time the fp64 oracle on evenly spaced rows of the prefill workload."""
    import numpy as np
    from oracle import oracle
    orc = oracle.get()
    nthreads = oracle.default_threads()
    total = w.B * w.H * w.Nq
    rows = np.linspace(0, total - 1, num=min(target_rows, total)).astype(np.int64)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    orc.attention(qc, kc, vc, w.causal, w.scale, rows=rows, nthreads=nthreads)
    dt = time.perf_counter() - t0
    i = rows % w.Nq
    visible = np.minimum(w.Nk, i + (w.Nk - w.Nq) + 1) if w.causal else np.full_like(i, w.Nk)
    flops = float(np.sum(visible)) * w.d * 4.0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{len(rows)} evenly spaced query rows of {w.name} (of {total}); "
                      f"{flops / 1e9:.1f} GFLOP of visible work in {dt:.1f} s, fp64"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "varlen", "decode_gqa", "decode_paged", "bwd", "fp8"], default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=40000)
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

    wp, wd, wv, wg = BY_NAME["long_causal"], BY_NAME["decode"], BY_NAME["varlen_gqa"], BY_NAME["decode_gqa"]
    do_p, do_d = args.only in ("all", "prefill"), args.only in ("all", "decode")
    do_v = args.only in ("all", "varlen")
    do_g = args.only in ("all", "decode_gqa")
    do_b = args.only in ("all", "bwd")
    do_pg = args.only in ("all", "decode_paged")
    do_f8 = args.only in ("all", "fp8")
    wpg = BY_NAME["decode_paged"]
    if do_p:
        q, k, v = make_qkv(wp, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
    if do_d:
        dq, dk, dv = make_qkv(wd, device=dev)
        S = wd.splits
        op = torch.empty((S, wd.B, wd.H, wd.Nq, wd.d), dtype=torch.float32, device=dev)
        lp = torch.empty((S, wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
        do_ = torch.empty_like(dq)
        dlse = torch.empty((wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
    if do_b:
        if not do_p:
            q, k, v = make_qkv(wp, device=dev)
            o = torch.empty_like(q)
            lse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
        fa.fwd(q, k, v, causal=wp.causal, scale=wp.scale, out=o, lse=lse)
        gen = torch.Generator(device=dev)
        gen.manual_seed(wp.seed + 100)
        bdo = torch.randn(tuple(q.shape), generator=gen, device=dev, dtype=torch.float32).to(wp.dtype)
        bdq, bdk, bdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(fa.bwd_workspace_bytes(wp.B, wp.H, wp.Nq) // 4, dtype=torch.float32, device=dev)
        # the backward reads the forward's o and lse: keep them fixed while timing
        bo, blse = o.clone(), lse.clone()
    if do_g:
        gq, gk, gv = make_qkv(wg, device=dev)
        gop = torch.empty((wg.splits, wg.B, wg.H, wg.Nq, wg.d), dtype=torch.float32, device=dev)
        glp = torch.empty((wg.splits, wg.B, wg.H, wg.Nq), dtype=torch.float32, device=dev)
        go = torch.empty_like(gq)
        glse = torch.empty((wg.B, wg.H, wg.Nq), dtype=torch.float32, device=dev)
    if do_v:
        vq, vk, vv, vcq, vck = make_varlen(wv, device=dev)
        vo = torch.empty_like(vq)
        vlse = torch.empty((wv.H, vq.shape[0]), dtype=torch.float32, device=dev)
        vmax = max(wv.seqlens)
    if do_pg:
        pq, pkc, pvc, pbt, psl = make_paged(wpg, device=dev)
        pop = torch.empty((wpg.splits, wpg.B, wpg.H, 1, wpg.d), dtype=torch.float32, device=dev)
        plp = torch.empty((wpg.splits, wpg.B, wpg.H, 1), dtype=torch.float32, device=dev)
        po = torch.empty((wpg.B, wpg.H, 1, wpg.d), dtype=wpg.dtype, device=dev)
        plse = torch.empty((wpg.B, wpg.H, 1), dtype=torch.float32, device=dev)
    if do_f8:
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
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(rec):
        e = [ev() for _ in range(11)]
        e[0].record(stream)
        if do_p:
            fa.fwd(q, k, v, causal=wp.causal, scale=wp.scale, out=o, lse=lse, stream=stream)
        e[1].record(stream)
        if do_d:
            fa.fwd_splitkv(dq, dk, dv, S, causal=wd.causal, scale=wd.scale, o_part=op, lse_part=lp,
                           stream=stream)
        e[2].record(stream)
        if do_d:
            fa.splitkv_combine(op, lp, wd.dtype, out=do_, lse=dlse, stream=stream)
        e[3].record(stream)
        if do_v:
            fa.fwd_varlen(vq, vk, vv, vcq, vck, vmax, vmax, causal=wv.causal, scale=wv.scale, out=vo,
                          lse=vlse, stream=stream)
        e[4].record(stream)
        if do_g:
            fa.fwd_splitkv_gqa(gq, gk, gv, wg.splits, causal=wg.causal, scale=wg.scale, o_part=gop, lse_part=glp,
                               stream=stream)
        e[5].record(stream)
        if do_g:
            fa.splitkv_combine(gop, glp, wg.dtype, out=go, lse=glse, stream=stream)
        e[6].record(stream)
        if do_b:
            fa.bwd(q, k, v, bo, blse, bdo, causal=wp.causal, scale=wp.scale, dq=bdq, dk=bdk, dv=bdv, workspace=bws,
                   stream=stream)
        e[7].record(stream)
        if do_pg:
            fa.fwd_splitkv_paged(pq, pkc, pvc, pbt, psl, wpg.splits, scale=wpg.scale, o_part=pop, lse_part=plp,
                                 stream=stream)
        e[8].record(stream)
        if do_pg:
            fa.splitkv_combine(pop, plp, wpg.dtype, out=po, lse=plse, stream=stream)
        e[9].record(stream)
        if do_f8:
            fa.fwd_fp8(fq8, fk8, fv8, fqd, fkd, fvd, causal=wp.causal, scale=wp.scale, out=fo, lse=flse, stream=stream)
        e[10].record(stream)
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

    def avg_ms(i, j):
        return sum(r[i].elapsed_time(r[j]) for r in recs) / len(recs)

    t_fwd, t_split, t_comb, t_var = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3), avg_ms(3, 4)
    t_gsplit, t_gcomb = avg_ms(4, 5), avg_ms(5, 6)
    t_bwd = avg_ms(6, 7)
    t_psplit, t_pcomb = avg_ms(7, 8), avg_ms(8, 9)
    t_f8 = avg_ms(9, 10)
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic"}
    cfg = {}
    if do_p:
        fl = attn_flops(wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.causal)
        tflops = fl / (t_fwd * 1e-3) / 1e12
        src = source_hash(FWD_SOURCES)
        out.update({"value": tflops, "unit": "TFLOP/s", "dtype": "bf16",
                    "pct_mfma_peak": 100.0 * tflops / PEAK_TFLOPS[wp.dtype]})
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[wp.dtype],
                           "unit": "TFLOP/s", "frac": tflops / PEAK_TFLOPS[wp.dtype],
                           "traffic": read_traffic("fwd_long_causal", src),
                           "kernel": "fwd_kernel<bf16, d=128, causal>", "avg_us": t_fwd * 1e3,
                           "flop_per_launch": fl, "source_hash": src}
        cfg["workload"] = ("long_causal: B=1 H=32 Nq=Nk=8192 d=128 bf16 causal (prefill, timed as value) + "
                           "decode: B=8 H=32 Nq=1 Nk=32768 d=128 fp16 16 splits")
        cfg.update({"prefill": {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d,
                                "dtype": "bf16", "causal": True, "input_scale": wp.mult}})
    if do_d:
        byts = attn_bytes(wd.B, wd.H, wd.Nq, wd.Nk, wd.d)
        t_dec = t_split + t_comb
        out["decode"] = {"GB_per_s": byts / (t_dec * 1e-3) / 1e9, "hbm_frac": byts / (t_dec * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "us_total": t_dec * 1e3, "us_splitkv": t_split * 1e3, "us_combine": t_comb * 1e3,
                         "algorithmic_bytes": byts,
                         "partials_bytes": fa.workspace_bytes(wd.B, wd.H, wd.Nq, wd.d, S)}
        split_bytes = byts - 2 * wd.B * wd.H * wd.d - 4 * wd.B * wd.H   # O and LSE are the combine's
        out["roofline_decode"] = {"bound": "hbm", "achieved": split_bytes / (t_split * 1e-3) / 1e9,
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": split_bytes / (t_split * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                  "traffic": read_traffic("decode", source_hash(DEC_SOURCES)),
                                  "kernel": "decode_kernel<fp16, d=128>"}
        if not do_p:
            out.update({"value": out["decode"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode: B=8 H=32 Nq=1 Nk=32768 d=128 fp16 16 splits"
        cfg["decode"] = {"B": wd.B, "H": wd.H, "Nq": wd.Nq, "Nk": wd.Nk, "d": wd.d, "dtype": "fp16",
                         "splits": S}
    if do_b:
        # algorithmic work of the backward: its five products (recompute S, dP, dV, dK,
        # dQ) = 2.5 x the forward's two
        fl = 2.5 * attn_flops(wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.causal)
        tb = fl / (t_bwd * 1e-3) / 1e12
        out["bwd"] = {"TFLOP_per_s": tb, "pct_mfma_peak": 100.0 * tb / PEAK_TFLOPS[wp.dtype], "avg_us": t_bwd * 1e3,
                      "flop_per_launch": fl}
        out["roofline_bwd"] = {"bound": "mfma", "achieved": tb, "peak": PEAK_TFLOPS[wp.dtype], "unit": "TFLOP/s",
                               "frac": tb / PEAK_TFLOPS[wp.dtype], "traffic": None,
                               "kernel": "bwd_delta + bwd_dkdv + bwd_dq <bf16, d=128, causal>"}
        cfg["bwd"] = {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d, "dtype": "bf16", "causal": True}
        if not (do_p or do_d):
            out.update({"value": tb, "unit": "TFLOP/s", "dtype": "bf16"})
            cfg["workload"] = "bwd on long_causal: B=1 H=32 Nq=Nk=8192 d=128 bf16 causal"
    if do_g:
        # bytes the method must move: Q, O (B*H*d each), K, V (B*H_kv*Nk*d each), LSE
        gb = 2 * (2 * wg.B * wg.H * wg.d + 2 * wg.B * wg.H_kv * wg.Nk * wg.d) + 4 * wg.B * wg.H
        tg = t_gsplit + t_gcomb
        out["decode_gqa"] = {"GB_per_s": gb / (tg * 1e-3) / 1e9, "hbm_frac": gb / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             "us_total": tg * 1e3, "us_splitkv": t_gsplit * 1e3, "us_combine": t_gcomb * 1e3,
                             "algorithmic_bytes": gb}
        gsplit_bytes = gb - 2 * wg.B * wg.H * wg.d - 4 * wg.B * wg.H
        out["roofline_decode_gqa"] = {"bound": "hbm", "achieved": gsplit_bytes / (t_gsplit * 1e-3) / 1e9,
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gsplit_bytes / (t_gsplit * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                      "traffic": read_traffic("decode_gqa", source_hash(DEC_SOURCES)),
                                      "kernel": "decode_kernel<fp16, d=128, 4 query heads per workgroup>"}
        cfg["decode_gqa"] = {"B": wg.B, "H": wg.H, "H_kv": wg.H_kv, "Nq": wg.Nq, "Nk": wg.Nk, "d": wg.d,
                             "dtype": "fp16", "splits": wg.splits}
        if not (do_p or do_d or do_v):
            out.update({"value": out["decode_gqa"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode_gqa: B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 fp16 16 splits"
    if do_v:
        fl = sum(attn_flops(1, wv.H, n, n, wv.d, wv.causal) for n in wv.seqlens)
        tf = fl / (t_var * 1e-3) / 1e12
        out["varlen_gqa"] = {"TFLOP_per_s": tf, "pct_mfma_peak": 100.0 * tf / PEAK_TFLOPS[wv.dtype],
                             "avg_us": t_var * 1e3, "flop_per_launch": fl}
        out["roofline_varlen"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_TFLOPS[wv.dtype],
                                  "unit": "TFLOP/s", "frac": tf / PEAK_TFLOPS[wv.dtype],
                                  "traffic": read_traffic("fwd_varlen_gqa", source_hash(FWD_SOURCES)),
                                  "kernel": "fwd_kernel<bf16, d=128, causal, varlen>"}
        cfg["varlen"] = {"sequences": wv.B, "tokens": sum(wv.seqlens), "max_seqlen": max(wv.seqlens),
                         "H": wv.H, "H_kv": wv.H_kv, "d": wv.d, "dtype": "bf16", "causal": True}
        if not do_p and not do_d:
            out.update({"value": tf, "unit": "TFLOP/s", "dtype": "bf16"})
            cfg["workload"] = "varlen_gqa: 16 packed causal sequences, 20752 tokens, H=32 H_kv=8 d=128 bf16"
    if do_pg:
        # bytes the method must move: Q, O, K, V and LSE as decode_gqa, plus the
        # block table (B x pages per sequence int32) once
        kv = 2 * 2 * wpg.B * wpg.H_kv * wpg.Nk * wpg.d
        pgb = 2 * 2 * wpg.B * wpg.H * wpg.d + kv + 4 * wpg.B * wpg.H + 4 * pbt.numel()
        tp = t_psplit + t_pcomb
        out["decode_paged"] = {"GB_per_s": pgb / (tp * 1e-3) / 1e9, "hbm_frac": pgb / (tp * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               "us_total": tp * 1e3, "us_splitkv": t_psplit * 1e3, "us_combine": t_pcomb * 1e3,
                               "algorithmic_bytes": pgb}
        psplit_bytes = pgb - 2 * wpg.B * wpg.H * wpg.d - 4 * wpg.B * wpg.H
        out["roofline_decode_paged"] = {"bound": "hbm", "achieved": psplit_bytes / (t_psplit * 1e-3) / 1e9,
                                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": psplit_bytes / (t_psplit * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                        "traffic": read_traffic("decode_paged", source_hash(DEC_SOURCES)),
                                        "kernel": "decode_kernel<fp16, d=128, 4 query heads per workgroup, paged>"}
        cfg["decode_paged"] = {"B": wpg.B, "H": wpg.H, "H_kv": wpg.H_kv, "Nq": 1, "Nk": wpg.Nk, "d": wpg.d,
                               "dtype": "fp16", "splits": wpg.splits, "page_size": wpg.page_size}
        if args.only == "decode_paged":
            out.update({"value": out["decode_paged"]["GB_per_s"], "unit": "GB/s", "dtype": "f16"})
            cfg["workload"] = "decode_paged: B=8 H=32 H_kv=8 Nq=1 Nk=32768 d=128 fp16 16 splits, 16-row pages"
    if do_f8:
        fl = attn_flops(wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.causal)
        t8 = fl / (t_f8 * 1e-3) / 1e12
        out["fp8"] = {"TFLOP_per_s": t8, "pct_mfma_peak": 100.0 * t8 / PEAK_FP8_TFLOPS, "avg_us": t_f8 * 1e3,
                      "flop_per_launch": fl}
        out["roofline_fp8"] = {"bound": "mfma", "achieved": t8, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                               "frac": t8 / PEAK_FP8_TFLOPS, "traffic": None,
                               "kernel": "fwd_fp8_kernel<e4m3, d=128, causal>"}
        cfg["fp8"] = {"B": wp.B, "H": wp.H, "Nq": wp.Nq, "Nk": wp.Nk, "d": wp.d, "dtype": "e4m3 in, bf16 out",
                      "causal": True, "scales": "Q, K per 128 rows; V per head"}
        if args.only == "fp8":
            out.update({"value": t8, "unit": "TFLOP/s", "dtype": "fp8"})
            cfg["workload"] = "fp8 on long_causal: B=1 H=32 Nq=Nk=8192 d=128 e4m3 causal"
    out["config"] = cfg
    if do_p and not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(q, k, v, wp, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
