#!/usr/bin/env python3
"""Benchmark of the forward-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one call of the path's entry point over the whole workload, inputs resident
in HBM.  By default every workload is timed: the headline line is the causal bf16
prefill (B4 H32 S4096 D128); the fp32 MHA, GQA decode, MLA decode and MLA prefill
workloads and those of the next rows (e4m3 caches, e4m3 V, ragged prefill, merge,
quantiser) follow in its "configs" array, each with its own roofline object
(algorithmic work per launch / measured launch duration, against MI355X's published
peak) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak)"
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3, "hbm": 8000.0}   # TFLOP/s, GB/s
# What the HIP events around one call time: the whole call (decode = split kernel + combine).
KERNELS = {"prefill": "prefill kernel", "mla_prefill": "prefill kernel (MLA policy)",
           "prefill_varlen": "prefill kernel (ragged batch)", "merge": "merge_kernel",
           "decode": "gqa_decode_split + combine_kernel (one call)",
           "mla_decode": "mla_decode_split + combine_kernel (one call)",
           "quantize": "quantize_rows_kernel"}


def algorithmic_work(w, lens=None):
    """(flops, bytes) of one call: flops over unmasked (query, key) pairs only; bytes = inputs
    read once + outputs written once (decode: the visible cache rows of each kv head)."""
    if w.kind == "prefill":
        if w.causal:
            off = w.Skv - w.Sq
            pairs = sum(max(0, min(w.Skv, i + off + 1)) for i in range(w.Sq))
        else:
            pairs = w.Sq * w.Skv
        flops = 2 * (w.D + w.Dv) * pairs * w.B * w.Hq
        esz = 4 if w.dtype == "f32" else 2
        byts = esz * w.B * (w.Sq * w.Hq * (w.D + w.Dv) + w.Skv * w.Hkv * (w.D + w.Dv))
        return flops, byts
    if w.kind == "prefill_varlen":
        # each sequence is a causal prefill with its own length; lens = the sequence lengths
        pairs = sum(int(n) * (int(n) + 1) // 2 for n in lens) if w.causal else sum(int(n) ** 2 for n in lens)
        toks = int(sum(lens))
        return 2 * (w.D + w.Dv) * pairs * w.Hq, 2 * toks * (w.Hq + w.Hkv) * (w.D + w.Dv)
    if w.kind == "merge":
        rows = w.B * w.Sq * w.Hq
        return 0, rows * (3 * w.D * 2 + 3 * 4)   # two bf16 parts in, one out; two LSEs in, one out
    if w.kind == "decode":
        sl = int(sum(lens))
        flops = 2 * w.Hq * (w.D + w.Dv) * sl
        if w.dtype == "fp8":   # e4m3 K and V rows plus their two fp32 per-token scales
            byts = sl * w.Hkv * (w.D + w.Dv + 8) + w.B * w.Hq * (w.D + w.Dv) * 2
        else:
            byts = sl * w.Hkv * (w.D + w.Dv) * 2 + w.B * w.Hq * (w.D + w.Dv) * 2
        return flops, byts
    if w.kind == "mla_decode":
        sl = int(sum(lens))
        flops = 2 * w.Hq * (w.D + w.Dv) * sl
        if w.dtype == "fp8":   # e4m3 latent rows plus one fp32 scale per row
            byts = sl * (w.D + 4) + w.B * w.Hq * (w.D + w.Dv) * 2
        else:
            byts = sl * w.D * 2 + w.B * w.Hq * (w.D + w.Dv) * 2
        return flops, byts
    if w.kind == "mla_prefill":
        pairs = w.Sq * (w.Sq + 1) // 2 if w.causal else w.Sq * w.Skv
        f_fp8 = 2 * w.Dn * pairs * w.B * w.Hq
        f_bf16 = 2 * (w.Dr + w.Dv) * pairs * w.B * w.Hq          # rope QK and P.V on bf16 matrix cores
        vbytes = w.Dv + 4 if w.dtype == "fp8v" else 2 * w.Dv    # e4m3 codes + scale, or bf16
        byts = w.B * (w.Sq * w.Hq * (w.Dn + 2 * w.Dr + 2 * w.Dv + 4) + w.Skv * w.Hq * (w.Dn + 4 + vbytes)
                      + w.Skv * w.Hr * 2 * w.Dr)
        return (f_fp8, f_bf16), byts
    if w.kind == "quantize":
        rows = w.B * w.Sq * w.Hq
        return 0, rows * (w.Dn * 4 + w.Dn + 4)        # fp32 rows in, e4m3 codes + fp32 scale out
    raise ValueError(w.kind)


def _strip_comments(text: str) -> str:
    """C/C++ source without // and /* */ comments and blank lines, each line right-stripped
    (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def source_digest() -> str:
    """sha256 over the kernel and ABI sources with comments removed, to tie stored counter
    readings to the code they were taken on (a comment-only edit keeps the digest)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        if n.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, n), encoding="utf-8") as f:
                h.update(n.encode() + b"\0" + _strip_comments(f.read()).encode())
    return h.hexdigest()


# ------------------------------------------------------------------------------- inputs

def setup(w):
    """Device inputs and the step closure for workload w; returns (step, lens, keepalive)."""
    import numpy as np
    import torch

    import attention_flash_attn_fwd_amd as fa
    from workloads import make_decode, make_mla_decode, make_mla_prefill, make_prefill

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    if w.kind == "prefill":
        d = make_prefill(w)
        if w.dtype == "bf16":
            q, k, v = bf16(d["q"]), bf16(d["k"]), bf16(d["v"])
        else:
            q, k, v = (torch.from_numpy(d[n]).cuda() for n in ("q", "k", "v"))
        o = torch.empty_like(q)
        return (lambda i: fa.prefill(q, k, v, causal=w.causal, scale=w.scale, out=o)), None, (q, k, v, o)
    if w.kind == "prefill_varlen":
        from workloads import make_prefill_varlen
        d = make_prefill_varlen(w)
        q, k, v = bf16(d["q"]), bf16(d["k"]), bf16(d["v"])
        cu = torch.from_numpy(d["cu"]).cuda()
        o = torch.empty_like(q)
        mx = int(d["lens"].max())
        return (lambda i: fa.prefill_varlen(q, k, v, cu, cu, mx, causal=w.causal, scale=w.scale, out=o)), \
            d["lens"], (q, k, v, cu, o)
    if w.kind == "merge":
        from workloads import make_merge
        d = make_merge(w)
        oa, ob = bf16(d["o_a"]), bf16(d["o_b"])
        la, lb = torch.from_numpy(d["lse_a"]).cuda(), torch.from_numpy(d["lse_b"]).cuda()
        o, lse = torch.empty_like(oa), torch.empty_like(la)
        return (lambda i: fa.merge(oa, la, ob, lb, out=o, out_lse=lse)), None, (oa, ob, la, lb, o, lse)
    if w.kind == "decode":
        d = make_decode(w)
        q, kv_lens = bf16(d["q"]), torch.from_numpy(d["kv_lens"]).cuda()
        ws = torch.empty(fa.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.Skv), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        if w.dtype == "fp8":
            k, v, ks, vs = (torch.from_numpy(d[n]).cuda() for n in ("k", "v", "k_scale", "v_scale"))
            return (lambda i: fa.decode(q, k, v, kv_lens, scale=w.scale, workspace=ws, out=o, k_scale=ks,
                                        v_scale=vs)), d["kv_lens"], (q, k, v, ks, vs, ws, o)
        caches = [(bf16(d["k"]), bf16(d["v"]))]
        return (lambda i: fa.decode(q, caches[0][0], caches[0][1], kv_lens, scale=w.scale, workspace=ws, out=o)), \
            d["kv_lens"], (q, caches, ws, o)
    if w.kind == "mla_decode":
        d = make_mla_decode(w)
        q, kv_lens = bf16(d["q"]), torch.from_numpy(d["kv_lens"]).cuda()
        # two copies of the latent cache (302 MB bf16, 151 MB e4m3), alternated, so that the
        # 256 MB MALL cannot serve a step from the previous one
        fp8 = w.dtype == "fp8"
        kv0 = torch.from_numpy(d["kv"]).cuda() if fp8 else bf16(d["kv"])
        caches = [kv0, kv0.clone()]
        scales = [torch.from_numpy(d["kv_scale"]).cuda()] * 2 if fp8 else [None, None]
        if fp8:
            scales[1] = scales[0].clone()
        ws = torch.empty(fa.mla_decode_workspace_size(w.B, w.Hq, w.Dv, w.Skv), dtype=torch.uint8, device="cuda")
        o = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda")
        return (lambda i: fa.mla_decode(q, caches[i & 1], kv_lens, dv=w.Dv, scale=w.scale, workspace=ws, out=o,
                                        kv_scale=scales[i & 1])), d["kv_lens"], (q, caches, scales, ws, o)
    if w.kind == "mla_prefill":
        d = make_mla_prefill(w)
        t = {n: (bf16(d[n]) if d[n].dtype == np.uint16 else torch.from_numpy(d[n]).cuda())
             for n in ("q_nope", "k_nope", "q_scale", "k_scale", "q_rope", "k_rope", "v", "v_scale") if n in d}
        o = torch.empty((w.B, w.Sq, w.Hq, w.Dv), dtype=torch.bfloat16, device="cuda")
        return (lambda i: fa.mla_prefill(t["q_nope"], t["q_rope"], t["k_nope"], t["k_rope"], t["v"], t["q_scale"],
                                         t["k_scale"], causal=w.causal, scale=w.scale, out=o,
                                         v_scale=t.get("v_scale"))), None, (t, o)
    if w.kind == "quantize":
        from workloads import make_quantize
        x = torch.from_numpy(make_quantize(w)["x"]).cuda()
        codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device="cuda")
        return (lambda i: fa.quantize_rows_e4m3(x, codes, scale)), None, (x, codes, scale)
    raise ValueError(w.kind)


# ------------------------------------------------------------------------------- CPU oracle

def cpu_baseline(w, lens, budget_s: float):
    """Time the oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    from workloads import make_decode, make_mla_decode, make_mla_prefill, make_prefill
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))

    done_work, t_used, n, what = 0.0, 0.0, 0, ""
    if w.kind in ("prefill", "mla_prefill"):
        pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
        cache = {}
        for b, h in pairs:
            if b not in cache:
                cache = {b: (make_prefill(w, batches=[b]) if w.kind == "prefill" else make_mla_prefill(w, batches=[b]))}
            d = cache[b]
            # the inputs of this (batch, head), decoded to fp64 outside the timed region
            if w.kind == "prefill":
                kvh = h // (w.Hq // w.Hkv)
                dec = oracle.bf16_to_f64 if w.dtype == "bf16" else (lambda x: x.astype(np.float64))
                args = (dec(d["q"][:, :, h:h + 1]), dec(d["k"][:, :, kvh:kvh + 1]), dec(d["v"][:, :, kvh:kvh + 1]))
                fn = lambda rows: oracle.prefill_rows(*args, w.scale, w.causal, 0, 0, rows)
            else:
                s = lambda a: a[:, :, h:h + 1]
                vv = (oracle.e4m3_to_f64(s(d["v"])) * s(d["v_scale"])[..., None].astype(np.float64)
                      if "v_scale" in d else oracle.bf16_to_f64(s(d["v"])))
                args = (oracle.e4m3_to_f64(s(d["q_nope"])), oracle.bf16_to_f64(s(d["q_rope"])),
                        oracle.e4m3_to_f64(s(d["k_nope"])), oracle.bf16_to_f64(d["k_rope"]), vv,
                        s(d["q_scale"]).astype(np.float64), s(d["k_scale"]).astype(np.float64))
                fn = lambda rows: oracle.mla_prefill_rows(*args, w.scale, w.causal, 0, 0, rows)
            t0 = time.perf_counter()
            for r0 in range(0, w.Sq, 1024):
                fn(np.arange(r0, min(w.Sq, r0 + 1024)))
            t_used += time.perf_counter() - t0
            n += 1
            if t_used >= budget_s:
                break
        one = w.with_(B=1, Hq=1, Hkv=1)
        f, _ = algorithmic_work(one)
        done_work = (sum(f) if isinstance(f, tuple) else f) * n
        what = f"{n} (batch, head) pairs x all {w.Sq} query rows"
        return {"value": done_work / t_used / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": what, "seconds": round(t_used, 2)}
    if w.kind == "prefill_varlen":
        from workloads import make_prefill_varlen
        d = make_prefill_varlen(w)
        cu = d["cu"]
        done = 0.0
        for b in range(w.B):
            for h in range(w.Hq):
                s0, s1 = int(cu[b]), int(cu[b + 1])
                sl = lambda x: oracle.bf16_to_f64(x[s0:s1, h:h + 1])[None]
                args = (sl(d["q"]), sl(d["k"]), sl(d["v"]))
                t0 = time.perf_counter()
                for r0 in range(0, s1 - s0, 1024):
                    oracle.prefill_rows(*args, w.scale, w.causal, 0, 0, np.arange(r0, min(s1 - s0, r0 + 1024)))
                t_used += time.perf_counter() - t0
                n += 1
                f, _ = algorithmic_work(w.with_(Hq=1, Hkv=1), lens=[s1 - s0])
                done += f
                if t_used >= budget_s:
                    break
            if t_used >= budget_s:
                break
        return {"value": done / t_used / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"{n} (sequence, head) pairs x all their query rows", "seconds": round(t_used, 2)}
    if w.kind == "merge":
        from workloads import make_merge
        d = make_merge(w.with_(B=1, Sq=min(w.Sq, 512)))
        args = (oracle.bf16_to_f64(d["o_a"]), d["lse_a"].astype(np.float64), oracle.bf16_to_f64(d["o_b"]),
                d["lse_b"].astype(np.float64))
        while t_used < budget_s and n < 200:
            t0 = time.perf_counter()
            oracle.merge_states(*args)
            t_used += time.perf_counter() - t0
            n += 1
        _, byts = algorithmic_work(w.with_(B=1, Sq=d["o_a"].shape[1]))
        return {"value": n * byts / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{n} passes over {d['o_a'].shape[1]} tokens x {w.Hq} heads", "seconds": round(t_used, 2)}
    if w.kind == "quantize":
        from workloads import make_quantize
        d = make_quantize(w, tokens=min(w.Sq, 256))["x"]
        n = 0
        while t_used < budget_s and n < 64:
            t0 = time.perf_counter()
            oracle.quantize_rows(d)
            t_used += time.perf_counter() - t0
            n += 1
        rows = n * d.shape[0] * d.shape[1] * d.shape[2]
        return {"value": rows * (w.Dn * 5 + 4) / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{n} passes over the first {d.shape[1]} tokens x {w.Hq} heads rows", "seconds": round(t_used, 2)}
    # decode: whole sequences (drawing and decoding the inputs is not timed; the oracle call is)
    sel = []
    for b in range(w.B):
        if w.kind == "decode" and w.dtype == "fp8":
            d = make_decode(w, batches=[b], lens=lens)
            L = int(d["kv_lens"][0])
            args = (oracle.bf16_to_f64(d["q"]),
                    oracle.e4m3_to_f64(d["k"][:, :L]) * d["k_scale"][:, :L, :, None].astype(np.float64),
                    oracle.e4m3_to_f64(d["v"][:, :L]) * d["v_scale"][:, :L, :, None].astype(np.float64),
                    d["kv_lens"], w.scale)
            fn = oracle.decode
        elif w.kind == "decode":
            d = make_decode(w, batches=[b], lens=lens)
            L = int(d["kv_lens"][0])
            args = (oracle.bf16_to_f64(d["q"]), oracle.bf16_to_f64(d["k"][:, :L]), oracle.bf16_to_f64(d["v"][:, :L]),
                    d["kv_lens"], w.scale)
            fn = oracle.decode
        else:
            d = make_mla_decode(w, batches=[b], lens=lens)
            L = int(d["kv_lens"][0])
            if w.dtype == "fp8":
                kv = oracle.e4m3_to_f64(d["kv"][:, :L]) * d["kv_scale"][:, :L, None].astype(np.float64)
            else:
                kv = oracle.bf16_to_f64(d["kv"][:, :L])
            args = (oracle.bf16_to_f64(d["q"]), kv, d["kv_lens"], w.Dv, w.scale)
            fn = oracle.mla_decode
        t0 = time.perf_counter()
        fn(*args)
        t_used += time.perf_counter() - t0
        sel.append(L)
        if t_used >= budget_s:
            break
    _, byts = algorithmic_work(w.with_(B=len(sel)), lens=sel)
    return {"value": byts / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sel)} whole sequences (lengths {sel[:4]}...)", "seconds": round(t_used, 2)}


# ------------------------------------------------------------------------------- counters

def copy_calibration(steps: int):
    """A plain copy of exactly 1 GiB (reads 1 GiB, writes 1 GiB) per launch: what FETCH_SIZE and
    WRITE_SIZE read for it gives the factor that turns those counters into bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(dt * 1e3, 4),
                      "GB_per_s": round(2 * n / dt / 1e9, 1)}), flush=True)


# ------------------------------------------------------------------------------- main

def timed(w, step, args):
    """Untimed spin-up and warmup steps, then K timed steps; returns (ms per step by the host
    clock, mean launch duration by HIP events on the launch stream, in ms)."""
    import torch
    # clocks ramp up over the first tens of milliseconds of sustained load: run untimed steps
    # for a fixed time first, then the requested warmup steps
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < args.spinup:
        for i in range(4):
            step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / args.steps, sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / args.steps


DTYPE_NAMES = {"f32": "f32", "bf16": "bf16", "fp8+bf16": "fp8e4m3+bf16",
               "fp8v": "e4m3 nope and V (bf16 P.V), bf16 rope", "fp8": "e4m3 cache, bf16 q/o"}


def measure(w, args, cpu_budget, traffic_rec):
    """One workload: device inputs, timed steps, roofline, oracle baseline.  Returns a dict."""
    import torch
    step, lens, keep = setup(w)
    flops, byts = algorithmic_work(w, lens)
    ms_per_step, launch_ms = timed(w, step, args)
    del keep, step
    torch.cuda.empty_cache()

    if w.kind in ("prefill", "prefill_varlen", "mla_prefill"):
        if w.kind == "mla_prefill":
            f_fp8, f_bf16 = flops
            total = f_fp8 + f_bf16
            t_roof = f_fp8 / (PEAK["fp8"] * 1e12) + f_bf16 / (PEAK["bf16"] * 1e12)
            peak = total / t_roof / 1e12          # mixed-precision peak: frac = T_roof / T_measured
        else:
            total = flops
            peak = PEAK["f32" if w.dtype == "f32" else "bf16"]
        value = total / (ms_per_step * 1e-3) / 1e12
        achieved = total / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "kernel": KERNELS[w.kind]}
        unit = "TFLOP/s"
    else:  # decode, merge and quantisation: HBM-bound
        value = byts / (ms_per_step * 1e-3) / 1e9
        achieved = byts / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK["hbm"], "unit": "GB/s",
                "frac": round(achieved / PEAK["hbm"], 4), "kernel": KERNELS[w.kind]}
        if w.kind in ("decode", "mla_decode"):
            # decode sits near the ridge for MLA: report the matrix-core side too
            fl = 2 * w.Hq * (w.D + w.Dv) * int(sum(lens))
            roof["mfma_frac"] = round(fl / (launch_ms * 1e-3) / 1e12 / PEAK["bf16"], 4)
        unit = "GB/s"
    roof["traffic"] = None if traffic_rec is None else traffic_rec.get("bytes_per_launch")

    cfg = {"workload": w.name, "B": w.B, "Sq": w.Sq, "Skv": w.Skv, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
           "Dv": w.Dv, "causal": w.causal, "parallelism": "none (1 GPU)"}
    if w.kind == "mla_prefill":
        cfg.update({"Dn": w.Dn, "Dr": w.Dr, "Hr": w.Hr})
    if lens is not None and w.kind == "prefill_varlen":
        cfg.update({"seq_lens": [int(x) for x in lens], "total_tokens": int(sum(lens)),
                    "len_range": [w.len_lo, w.len_hi]})
    elif lens is not None:
        cfg.update({"sum_kv_len": int(sum(lens)), "len_range": [w.len_lo, w.len_hi]})
    out = {
        "value": round(value, 3), "unit": unit, "ms_per_step": round(ms_per_step, 4),
        "dtype": "f32->e4m3" if w.kind == "quantize" else "bf16 (fp32 LSE)" if w.kind == "merge" else DTYPE_NAMES[w.dtype],
        "config": cfg, "roofline": roof, "kernel_ms": round(launch_ms, 4),
        "algorithmic": {"flops": flops if not isinstance(flops, tuple) else list(flops), "bytes": byts},
    }
    if cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(w, lens, cpu_budget)
    return out


def main():
    from workloads.shapes import BENCH_DEFAULT, BENCH_ORDER, WORKLOADS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spinup", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup steps, so that GPU clocks settle")
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                    help="one workload alone, or all of them (the headline first)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work in the CPU sample of the headline workload")
    ap.add_argument("--cpu-budget-other", type=float, default=2.0,
                    help="seconds of oracle work in the CPU sample of each other workload")
    ap.add_argument("--traffic", default=None, help="JSON with HBM traffic per launch from rocprofv3 counters (default profiles/traffic.json)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (scales FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 (multi-GPU sharding is a design note, "
              "not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import workload
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    torch.cuda.set_device(0)

    traffic = {}
    tpath = args.traffic or os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        # counters describe the kernels they were taken on: ignore them once the code changed
        if tr.get("source_sha256") == source_digest():
            traffic = tr.get("workloads", {})

    names = [args.workload] if args.workload != "all" else [BENCH_DEFAULT] + [n for n in BENCH_ORDER if n != BENCH_DEFAULT]
    results = []
    for i, name in enumerate(names):
        w = workload(name)
        budget = 0.0 if args.no_cpu_baseline else (args.cpu_budget if i == 0 else args.cpu_budget_other)
        r = measure(w, args, budget, traffic.get(name))
        results.append(r)
        if len(names) > 1:
            print(f"bench: {name}: {r['value']} {r['unit']} ({r['kernel_ms']} ms per launch, "
                  f"{r['roofline']['frac']} of peak)", file=sys.stderr, flush=True)
    head = results[0]
    out = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "spinup_s": args.spinup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1), see workloads/)", "config": head["config"], "roofline": head["roofline"],
        "kernel_ms": head["kernel_ms"], "algorithmic": head["algorithmic"],
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    if len(results) > 1:
        out["configs"] = [dict(r, workload=r["config"]["workload"]) for r in results[1:]]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
