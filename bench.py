"""Throughput of fused RoPE + SDPA on one MI355X.

Workload (N=1): FLUX joint text+image attention, B=1, H=24, S=512+4096=4608, D=128, bf16,
3-axis RoPE (16,56,56) theta=10000, no mask, forward without gradient.  One step is one
forward call (table packing + attention kernel + merge of the cut units) over the whole
batch.  The same run also times the masked FLUX forwards (B=2), the long forward (S=16896)
in bf16 and int8, and the training steps (FLUX B=2 and causal B=4); those legs run first,
so the headline is timed with the GPU at its steady clock.  The CPU oracle is timed last.

TFLOP/s use the dense attention count 4*B*H*Sq*Skv*D for the forward (halved for causal)
and 2.5x that for the backward.  Inputs are generated once on the host and are resident
in HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "fused RoPE+attention TFLOP/s (fwd, fwd+bwd) & % MFMA peak, FLUX S=4608"


def flops_fwd(B, H, S, D, causal=False):
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def _events_time(fn, steps, warmup, stream, before_timed=None):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if before_timed is not None:
        before_timed()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def _source_hash():
    """Hash of the forward kernel's sources with comments and blank lines removed (a comment
    edit does not invalidate counters taken on the same code)."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rope_flash_attention_amd", "csrc")
    for name in ("rs_fwd.hip", "rs_fwd_qk.hip", "rs_fwd_kernel.hpp", "rs_device.hpp", "rs_internal.h",
                 "rs_host.cpp"):  # the forward's sources
        text = open(os.path.join(csrc, name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d.get(kernel_key)
        if e and e.get("source_hash") == _source_hash():
            return e.get("bytes_per_launch")
    except Exception:
        return None
    return None


def cpu_baseline(budget_s=10.0):
    """The CPU float64 oracle on the host cores: the same FLUX forward (all heads), repeated
    until about `budget_s` seconds of wall time are used."""
    import synthetic as syn
    from oracle import rope_sdpa_forward
    from oracle.rope_sdpa_ref import default_workers

    cores = default_workers()
    w = syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    B, H, S, D = w.q.shape
    pairs = [(0, h) for h in range(H)]
    reps, dt = 0, 0.0
    while dt < budget_s:  # whole forward passes until the time budget is used
        t0 = time.perf_counter()
        rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, pairs=pairs, workers=cores)
        dt += time.perf_counter() - t0
        reps += 1
    fl = reps * flops_fwd(1, H, S, D)
    return {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{reps} x the full float64 oracle forward of B=1,H=24,S=4608,D=128 "
                  f"({dt:.2f} s wall on {cores} threads)",
        "cpu_model": _cpu_model(),
    }


def _train_case(t, steps, warmup, stream, causal):
    """Forward with LSE + backward (the training step) and the backward alone, on device
    tensors t = (q, k, v, cos, sin, dO) prepared beforehand."""
    import rope_flash_attention_amd as rfa

    tq, tk, tv, tc, ts, tdo = t
    B, H, S, D = tq.shape
    res = {}

    def fwd_lse():
        res["o"], res["lse"] = rfa.rope_sdpa_fwd_with_lse(tq, tk, tv, tc, ts, is_causal=causal)

    def bwd():
        rfa.rope_sdpa_bwd_explicit(tq, tk, tv, tc, ts, res["o"], res["lse"], tdo, is_causal=causal)

    def step():
        fwd_lse()
        bwd()

    fwd_lse()
    n = max(5, steps // 2)
    # the training step first, then the backward alone (each after its own warm-up calls)
    ms_train = _events_time(step, n, warmup, stream)
    ms_bwd = _events_time(bwd, n, warmup, stream)
    fl_f = flops_fwd(B, H, S, D, causal)
    return {
        "ms_fwd_bwd": round(ms_train, 4),
        "ms_bwd": round(ms_bwd, 4),
        "tflops_fwd_bwd": round(3.5 * fl_f / (ms_train * 1e-3) / 1e12, 2),
        "tflops_bwd": round(2.5 * fl_f / (ms_bwd * 1e-3) / 1e12, 2),
    }


def _prepare(dev, extra, train):
    """Every leg's inputs, generated on the host and copied to the device before any leg
    runs, so that the GPU legs follow each other without host-side pauses."""
    import torch

    import synthetic as syn

    def to_dev(w, names):
        return tuple(getattr(w, n).to(dev) for n in names)

    qkvcs = ("q", "k", "v", "cos", "sin")
    prep = {}
    if extra:
        w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=3000)
        S = w.q.shape[2]
        prep["flux_b2"] = to_dev(w, qkvcs)
        bm = syn.key_padding_mask(syn.key_padding_lengths(3000, 2), 512, S).to(dev)
        prep["mask_bool"] = bm
        prep["mask_add"] = torch.where(bm, torch.zeros((), dtype=torch.bfloat16, device=dev),
                                       torch.full((), float("-inf"), dtype=torch.bfloat16, device=dev)
                                       ).expand(2, 24, S, S).contiguous()
        prep["long"] = to_dev(syn.flux(batch=1, heads=48, grid=128, dtype="bf16", seed=5000), qkvcs)
        c = syn.zimage_chain()
        prep["chain"] = (c.x0.to(dev), [k.to(dev) for k in c.ks], [v.to(dev) for v in c.vs], c.cos.to(dev),
                         c.sin.to(dev))
        prep["gqa"] = to_dev(syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=740, kv_heads=6,
                                      per_sample_tables=True), qkvcs)
        # the autocast layout: fp32 Q/K (to be RMS-normalized in the kernel) beside bf16 V
        q32 = syn.normal(3000, syn.STREAM_Q, tuple(w.q.shape), "f32", 4.0).to(dev)
        k32 = syn.normal(3000, syn.STREAM_K, tuple(w.k.shape), "f32", 4.0).to(dev)
        prep["flux_b2_f32qk"] = (q32, k32) + prep["flux_b2"][2:]
        prep["flux_b2_f32"] = (prep["flux_b2"][0].float(), prep["flux_b2"][1].float()) + prep["flux_b2"][2:]
        prep["norm_w"] = tuple(t.to(dev) for t in syn.norm_weights(3000, 128))
    if train:
        prep["train_flux"] = to_dev(syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=4100, with_grad=True),
                                    qkvcs + ("do",))
        prep["train_causal"] = to_dev(syn.causal_1axis(batch=4, heads=16, seq=2048, dim=128, dtype="bf16",
                                                       seed=4200), qkvcs + ("do",))
    torch.cuda.synchronize()
    return prep


def _extra_cases(prep, steps, warmup, stream):
    """Masked FLUX forwards (B=2) and the long-sequence forward in bf16 and int8 (no-grad)."""
    import torch

    import rope_flash_attention_amd as rfa

    out = {}
    n = max(5, steps // 3)

    def timed(name, w_dev, mask=None, quant=None, note="", **kw):
        q, k, v, c, s = w_dev
        B, H, S, D = q.shape

        def f():
            rfa.rope_scaled_dot_product_attention(q, k, v, c, s, attn_mask=mask, quantization=quant, **kw)

        with torch.no_grad():
            ms = _events_time(f, n, warmup, stream)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops_fwd(B, H, S, D) / (ms * 1e-3) / 1e12, 2),
                     "shape": f"B={B},H={H},S={S},D={D}"}
        if note:
            out[name]["note"] = note

    timed("long_bf16", prep["long"])  # first: its seconds of work bring the clock to its steady value
    timed("long_bf16_k_prepass", prep["long"], k_prepass=True,
          note="K rotated once by a pass of its own (RS_FLAG_K_PREPASS), bit-identical output")
    wd, bm = prep["flux_b2"], prep["mask_bool"]
    timed("no_mask_b2", wd, note="reference for the masked B=2 calls")
    timed("no_mask_b2_k_prepass", wd, k_prepass=True, note="RS_FLAG_K_PREPASS")
    qn, kn = prep["norm_w"]
    timed("f32qk_rmsnorm_b2", prep["flux_b2_f32qk"], q_norm_weight=qn, k_norm_weight=kn,
          note="fp32 Q/K RMS-normalized and rotated in the kernel, bf16 V and O (autocast layout)")
    timed("f32qk_b2", prep["flux_b2_f32"], note="fp32 Q/K (no_mask_b2's values), bf16 V and O")
    timed("mask_bool_key_padding", wd, bm, note="bool [2,1,1,S]; dense flop count")
    timed("mask_all_true", wd, torch.ones_like(bm), note="bool [2,1,1,S] all True (skip path)")
    timed("mask_additive_4d", wd, prep["mask_add"], note="bf16 [2,24,S,S] 0/-inf, 2.04 GB read")
    out["mask_additive_4d"]["mask_read_tb_s"] = round(prep["mask_add"].numel() * 2 / (out["mask_additive_4d"]["ms"] * 1e-3) / 1e12, 3)
    timed("long_int8", prep["long"], quant="int8",
          note="int8 Q'K'^T (Q', K' quantized in the attention kernel, no codes in memory) + bf16 P.V; "
               "flops counted as the dense formula")
    timed("long_int8_prepass", prep["long"], quant="int8_prepass",
          note="the same int8 forward with a quantizer pass writing the codes first (bit-identical output)")
    timed("gqa_per_sample_tables", prep["gqa"],
          note="B=2, 24 query heads over 6 K/V heads, per-sample 3-axis tables; flops as the dense formula")
    out["chain_zimage"] = _chain_case(prep["chain"], n, warmup, stream)
    return out


def _chain_case(c, steps, warmup, stream):
    """The pages' chain benchmark: 12 attention layers at the Z-Image shape (1, 30, 4128, 128)
    bf16, each layer's output the next layer's query.  Fused: one fused RoPE + attention call
    per layer.  Eager: the rotation pass on the query and on the layer's keys (rope_sdpa_rotate,
    written to memory), then plain attention on the rotated tensors (the same kernels without
    rotation).  A step is the whole 12-layer chain."""
    import torch

    import rope_flash_attention_amd as rfa

    x0, ks, vs, cos, sin = c
    B, H, S, D = x0.shape

    def fused():
        x = x0
        for k, v in zip(ks, vs):
            x = rfa.rope_scaled_dot_product_attention(x, k, v, cos, sin)

    def eager():
        x = x0
        for k, v in zip(ks, vs):
            x = rfa.scaled_dot_product_attention(rfa.rope_rotate(x, cos, sin), rfa.rope_rotate(k, cos, sin), v)

    with torch.no_grad():  # two interleaved rounds, each variant's mean reported
        t = [(_events_time(fused, steps, warmup, stream), _events_time(eager, steps, warmup, stream))
             for _ in range(2)]
    ms_f = sum(a for a, _ in t) / 2
    ms_e = sum(b for _, b in t) / 2
    L = len(ks)
    return {"layers": L, "shape": f"B={B},H={H},S={S},D={D}", "ms_per_layer_fused": round(ms_f / L, 4),
            "ms_per_layer_eager": round(ms_e / L, 4), "ms_per_layer_saved": round((ms_e - ms_f) / L, 4),
            "tflops_fused": round(flops_fwd(B, H, S, D) * L / (ms_f * 1e-3) / 1e12, 2),
            "tflops_eager": round(flops_fwd(B, H, S, D) * L / (ms_e * 1e-3) / 1e12, 2)}


def traffic_from_counters(fetch_db, write_db, command):
    """HBM bytes per launch of the forward kernel from two rocprofv3 --pmc runs of
    `bench.py --copy-probe` (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch).  Each
    counter is scaled by what it reads for the 256 MiB device copy of the same run (a copy
    reads and writes 256 MiB)."""
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, avg(value), count(*) from counters_collection "
                           "where counter_name = ? group by kernel_name, grid_size", (counter,)).fetchall()
        return rows

    copy_bytes = 256 << 20
    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = per_kernel(db, counter)
        probe = max((v for n, v, c in rows if "copyBuffer" in n), default=None)
        fwd = [(n, v, c) for n, v, c in rows if "fwd_kernel" in n]
        if probe is None or not fwd:
            raise SystemExit(f"{db}: no copy probe or forward kernel with {counter}")
        scale = copy_bytes / (probe * 1024.0)
        name, v, c = max(fwd, key=lambda x: x[2])
        out[counter] = {"kiB_per_dispatch": v, "copy_probe_kiB": probe, "scale": scale,
                        "bytes_per_launch": v * 1024.0 * scale, "kernel": name, "dispatches": c}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    return {"fwd_bf16_d128_flux_b1": {"bytes_per_launch": total, "source_hash": _source_hash(),
                                      "command": command, "counters": out}}


def pmc_legs(reps):
    """Workloads for rocprofv3 --pmc passes, each call run `reps` times: the tiny fp32 forward
    (B=1, H=2, S=128, D=64), the FLUX forward (B=1, no mask), the FLUX forward with the
    additive 4-D bf16 mask (B=2), the FLUX backward (B=2) and the causal backward (B=4, H=16,
    S=2048), then a 256 MiB device copy whose byte counters scale the others."""
    import torch

    import synthetic as syn
    import rope_flash_attention_amd as rfa

    dev = torch.device("cuda:0")
    w = syn.tiny_fp32()
    t = [x.to(dev) for x in (w.q, w.k, w.v, w.cos, w.sin)]
    with torch.no_grad():
        for _ in range(reps):
            rfa.rope_scaled_dot_product_attention(*t)
    w = syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    t = [x.to(dev) for x in (w.q, w.k, w.v, w.cos, w.sin)]
    with torch.no_grad():
        for _ in range(reps):
            rfa.rope_scaled_dot_product_attention(*t)
    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=3000)
    S = w.q.shape[2]
    t = [x.to(dev) for x in (w.q, w.k, w.v, w.cos, w.sin)]
    bm = syn.key_padding_mask(syn.key_padding_lengths(3000, 2), 512, S).to(dev)
    add = torch.where(bm, torch.zeros((), dtype=torch.bfloat16, device=dev),
                      torch.full((), float("-inf"), dtype=torch.bfloat16, device=dev)).expand(2, 24, S, S).contiguous()
    with torch.no_grad():
        for _ in range(reps):
            rfa.rope_scaled_dot_product_attention(*t, attn_mask=add)
    del add
    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=4100, with_grad=True)
    t = [x.to(dev) for x in (w.q, w.k, w.v, w.cos, w.sin, w.do)]
    o, lse = rfa.rope_sdpa_fwd_with_lse(*t[:5])
    for _ in range(reps):
        rfa.rope_sdpa_bwd_explicit(*t[:5], o, lse, t[5])
    del o, lse, t
    w = syn.causal_1axis(batch=4, heads=16, seq=2048, dim=128, dtype="bf16", seed=4200)
    t = [x.to(dev) for x in (w.q, w.k, w.v, w.cos, w.sin, w.do)]
    o, lse = rfa.rope_sdpa_fwd_with_lse(*t[:5], is_causal=True)
    for _ in range(reps):
        rfa.rope_sdpa_bwd_explicit(*t[:5], o, lse, t[5], is_causal=True)
    del o, lse, t
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_legs": ["tiny_fp32", "flux_fwd_b1", "flux_fwd_b2_additive_4d", "flux_bwd_b2",
                                   "causal_bwd_b4", "copy_256MiB"],
                      "reps": reps}))


def summarize_counters(mfma_db, fetch_db, write_db, command):
    """Per kernel launch (kernel, grid): matrix-core busy fraction and HBM bytes from
    three rocprofv3 --pmc runs of `bench.py --pmc-legs` (SQ_VALU_MFMA_BUSY_CYCLES with
    GRBM_GUI_ACTIVE; FETCH_SIZE; WRITE_SIZE).  SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of
    all 1024 SIMDs and GRBM_GUI_ACTIVE the active cycles of the 8 XCDs, so the busy fraction
    is (MFMA_BUSY / 1024) / (GRBM_GUI_ACTIVE / 8), at the clock the GPU actually ran; that
    clock is GRBM_GUI_ACTIVE / 8 over the dispatch's duration.  Byte counters (KiB per
    dispatch) are scaled by what they read for the 256 MiB copy of the same run."""
    import sqlite3

    def rows(db, counters):
        con = sqlite3.connect(db)
        q = ("select kernel_name, grid_size, counter_name, avg(value), avg(duration) from counters_collection "
             "where counter_name in (%s) group by kernel_name, grid_size, counter_name" % ",".join("?" * len(counters)))
        return con.execute(q, counters).fetchall()

    data = {}
    for db, counters in ((mfma_db, ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")), (fetch_db, ("FETCH_SIZE",)),
                         (write_db, ("WRITE_SIZE",))):
        for name, grid, cname, val, dur in rows(db, counters):
            e = data.setdefault((name, grid), {})
            e[cname] = val
            e.setdefault("dur_ns", dur)
    probe = max(((n, g) for n, g in data if "copyBuffer" in n and "FETCH_SIZE" in data[(n, g)]),
                key=lambda k: data[k]["FETCH_SIZE"], default=None)
    if probe is None:
        raise SystemExit("no copy probe in the counter runs")
    fscale = (256 << 20) / (data[probe]["FETCH_SIZE"] * 1024.0)
    wscale = (256 << 20) / (data[probe]["WRITE_SIZE"] * 1024.0)
    out = [f"command: {command}", "",
           f"copy probe: FETCH_SIZE scale {fscale:.3f}, WRITE_SIZE scale {wscale:.3f} (256 MiB copy)", "",
           f"{'kernel':58s} {'grid':>8s} {'us':>8s} {'GHz':>5s} {'MFMA busy':>9s} {'read MB':>9s} {'write MB':>9s} {'GB/s':>8s}"]
    for (name, grid), e in sorted(data.items(), key=lambda kv: -kv[1].get("dur_ns", 0)):
        if not (name.startswith("_ZN2rs") or "rs::" in name):
            continue
        us = e["dur_ns"] / 1000.0
        ghz = e["GRBM_GUI_ACTIVE"] / 8 / e["dur_ns"] if "GRBM_GUI_ACTIVE" in e else float("nan")
        busy = (e["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024) / (e["GRBM_GUI_ACTIVE"] / 8) if "GRBM_GUI_ACTIVE" in e else float("nan")
        rd = e.get("FETCH_SIZE", float("nan")) * 1024.0 * fscale / 1e6
        wr = e.get("WRITE_SIZE", float("nan")) * 1024.0 * wscale / 1e6
        # (GRBM_GUI_ACTIVE also counts the dispatch's start and drain: clock and busy fraction
        # are only read for dispatches far longer than that)
        clk = f"{ghz:5.2f}" if us >= 50 else f"{'-':>5s}"
        mb = f"{100 * busy:8.1f}%" if us >= 50 else f"{'-':>9s}"
        out.append(f"{name[:58]:58s} {grid:8d} {us:8.1f} {clk} {mb} {rd:9.1f} {wr:9.1f} "
                   f"{(rd + wr) * 1e6 / (us * 1e-6) / 1e9:8.0f}")
    return "\n".join(out)


STALL_PASSES = (
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES",
     "GRBM_GUI_ACTIVE"),
    ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"),
)


def summarize_stalls(a_db, b_db, command):
    """Per kernel launch: how the matrix cores and the waves spend their cycles, from two
    rocprofv3 --pmc runs of `bench.py --pmc-legs` with the counters of STALL_PASSES.
    Fractions of the dispatch's cycles per SIMD (1024 SIMDs; GRBM_GUI_ACTIVE / 8 cycles):
    matrix core busy (SQ_VALU_MFMA_BUSY_CYCLES) and busy while a plain vector instruction
    issues (SQ_VALU_MFMA_COEXEC_CYCLES).  Fractions of the waves' cycles (SQ_WAVE_CYCLES;
    all three in units of 4 cycles): waiting for anything (s_waitcnt, barriers:
    SQ_WAIT_ANY), waiting for an instruction to issue (SQ_WAIT_INST_ANY) and for an LDS
    instruction to issue (SQ_WAIT_INST_LDS).  Instruction mix per matrix instruction:
    SQ_INSTS_VALU (which counts the matrix instructions too) and SQ_INSTS_LDS over
    SQ_INSTS_MFMA."""
    import sqlite3

    data = {}
    for db, counters in zip((a_db, b_db), STALL_PASSES):
        con = sqlite3.connect(db)
        q = ("select kernel_name, grid_size, counter_name, avg(value), avg(duration) from counters_collection "
             "where counter_name in (%s) group by kernel_name, grid_size, counter_name" % ",".join("?" * len(counters)))
        for name, grid, cname, val, dur in con.execute(q, counters).fetchall():
            e = data.setdefault((name, grid), {})
            e[cname if cname not in e else cname + "_b"] = val
            e.setdefault("dur_ns", dur)
    out = [f"command: {command}", "",
           f"{'kernel':58s} {'grid':>8s} {'us':>8s} {'MFMA':>6s} {'co-iss':>6s} {'wait':>6s} {'issue':>6s} "
           f"{'LDSiss':>6s} {'VALU/MF':>7s} {'LDS/MF':>7s}"]
    for (name, grid), e in sorted(data.items(), key=lambda kv: -kv[1].get("dur_ns", 0)):
        if not (name.startswith("_ZN2rs") or "rs::" in name) or e.get("dur_ns", 0) < 50e3:
            continue
        if not all(c in e for c in ("GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_INSTS_MFMA")) or not e["SQ_INSTS_MFMA"]:
            continue
        cyc = e["GRBM_GUI_ACTIVE"] / 8 * 1024
        wave = e["SQ_WAVE_CYCLES"]
        wave_b = e.get("SQ_WAVE_CYCLES_b", wave)
        f = lambda v: f"{100 * v:5.1f}%"
        out.append(f"{name[:58]:58s} {grid:8d} {e['dur_ns'] / 1000:8.1f} {f(e['SQ_VALU_MFMA_BUSY_CYCLES'] / cyc)} "
                   f"{f(e['SQ_VALU_MFMA_COEXEC_CYCLES'] / cyc)} {f(e['SQ_WAIT_ANY'] / wave)} "
                   f"{f(e['SQ_WAIT_INST_ANY'] / wave)} {f(e['SQ_WAIT_INST_LDS'] / wave_b)} "
                   f"{e['SQ_INSTS_VALU'] / e['SQ_INSTS_MFMA']:7.2f} {e['SQ_INSTS_LDS'] / e['SQ_INSTS_MFMA']:7.2f}")
    return "\n".join(out)


def summarize_rocpd(db_path, command):
    """Text summary of a rocprofv3 kernel trace: per kernel and grid size, calls and durations."""
    import sqlite3

    con = sqlite3.connect(db_path)
    rows = con.execute(
        "select name, grid_x / workgroup_x, workgroup_x, count(*), avg(duration) / 1000.0, "
        "min(duration) / 1000.0, max(duration) / 1000.0 from kernels group by name, grid_x "
        "order by sum(duration) desc").fetchall()
    out = [f"command: {command}", "",
           f"{'kernel':70s} {'workgroups':>10s} {'threads':>7s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for name, wg, th, n, avg, mn, mx in rows:
        out.append(f"{name[:70]:70s} {int(wg):10d} {int(th):7d} {n:6d} {avg:10.2f} {mn:10.2f} {mx:10.2f}")
    return "\n".join(out)


def _device_info():
    """CU count and maximum engine clock of the gfx950 agent (from rocminfo), and the dense
    bf16 MFMA peak they give: CUs x max clock x 4096 flop per clock per CU."""
    import re
    import subprocess

    info = {"cus": None, "max_sclk_mhz": None, "peak_bf16_tflops_device": None}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:
        return info
    for agent in txt.split("*******"):
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and clk:
            info["cus"], info["max_sclk_mhz"] = int(cu.group(1)), int(clk.group(1))
            info["peak_bf16_tflops_device"] = round(info["cus"] * info["max_sclk_mhz"] * 1e6 * 4096 / 1e12, 1)
            break
    return info


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _per_step_times(fn, steps, stream):
    """Each of `steps` calls bracketed by its own pair of events: median and minimum (ms)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], t[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the training-step timings")
    ap.add_argument("--no-extra", action="store_true", help="skip the masked / long / int8 forward timings")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize", metavar="DB", help="print a summary of a rocprofv3 results database and exit")
    ap.add_argument("--command", default="", help="command line recorded in the --summarize output")
    ap.add_argument("--pmc-legs", type=int, metavar="REPS",
                    help="run the counter workloads (tiny fp32, FLUX, FLUX additive 4-D, copy probe) and exit")
    ap.add_argument("--counters", nargs=3, metavar=("MFMA_DB", "FETCH_DB", "WRITE_DB"),
                    help="print matrix-core busy fraction and HBM bytes per forward launch and exit")
    ap.add_argument("--stalls", nargs=2, metavar=("A_DB", "B_DB"),
                    help="print matrix-core, issue and wait fractions per kernel launch from two "
                         "rocprofv3 --pmc runs (the counters of STALL_PASSES) and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print HBM bytes per forward launch from two rocprofv3 --pmc results databases and exit")
    args = ap.parse_args()
    if args.summarize:
        print(summarize_rocpd(args.summarize, args.command))
        return
    if args.traffic:
        print(json.dumps(traffic_from_counters(args.traffic[0], args.traffic[1], args.command), indent=1))
        return
    if args.counters:
        print(summarize_counters(*args.counters, args.command))
        return
    if args.stalls:
        print(summarize_stalls(*args.stalls, args.command))
        return
    if args.pmc_legs:
        pmc_legs(args.pmc_legs)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic as syn
    import rope_flash_attention_amd as rfa
    from oracle import rope_sdpa_forward

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    dinfo = _device_info()
    leg_warmup = max(2, args.warmup // 4)

    # ---- headline inputs: FLUX B=1 forward ----------------------------------------------------
    w = syn.flux(batch=1, heads=24, grid=64, dtype="bf16", seed=2000)
    B, H, S, D = w.q.shape
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    cos, sin = w.cos.to(dev), w.sin.to(dev)
    out = {}

    def fwd():
        out["o"] = rfa.rope_scaled_dot_product_attention(q, k, v, cos, sin)

    # Every leg's inputs are made first; then the GPU legs run back to back, the headline
    # last: an idle MI355X starts at a low engine clock and needs some tens of milliseconds
    # of work to reach its steady clock, which the other legs provide (as a serving or
    # training loop would).
    prep = _prepare(dev, not args.no_extra, not args.no_train)
    extra = None
    if not args.no_extra:
        extra = _extra_cases(prep, args.steps, leg_warmup, stream)
    train = None
    if not args.no_train:
        train = _train_case(prep["train_flux"], args.steps, leg_warmup, stream, causal=False)
        train["config"] = "FLUX B=2,H=24,S=4608,D=128,bf16"
        ct = _train_case(prep["train_causal"], args.steps, leg_warmup, stream, causal=True)
        ct["config"] = "causal B=4,H=16,S=2048,D=128,bf16, 1-axis RoPE"
        train["causal"] = ct
    del prep

    with torch.no_grad():
        # W warm-up calls, then K timed calls; during the timed calls the library also records
        # HIP events on the call's stream around each attention kernel (the dominant kernel)
        ms = _events_time(fwd, args.steps, args.warmup, stream,
                          before_timed=lambda: rfa.rope_sdpa_debug_kernel_timing(True))
        k_total_ms, k_launches = rfa.rope_sdpa_debug_kernel_time()
        rfa.rope_sdpa_debug_kernel_timing(False)
        ms_med, ms_min = _per_step_times(fwd, args.steps, stream)
    fl = flops_fwd(B, H, S, D)
    tflops = fl / (ms * 1e-3) / 1e12
    k_ms = k_total_ms / max(1, k_launches)  # attention kernel alone, average per launch
    k_tflops = fl / (k_ms * 1e-3) / 1e12

    # proof that the timed kernel computed the right thing: sampled rows vs the oracle
    rows = np.array([0, 511, 512, 2000, S - 1])
    O_ref, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, rows=rows, pairs=[(0, 0), (0, 23)])
    got = out["o"].float().cpu().numpy()
    got = np.stack([got[0, 0][rows], got[0, 23][rows]])
    err = float(np.abs(got - O_ref).max() / np.abs(O_ref).max())
    if not err <= 2e-2:
        print(json.dumps({"error": f"parity failed in bench: rel err {err}"}))
        sys.exit(1)

    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    base = None if args.no_cpu_baseline else cpu_baseline()

    peak_dev = dinfo.get("peak_bf16_tflops_device")
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_median": round(ms_med, 5),
        "ms_per_step_min": round(ms_min, 5),
        "tflops_median": round(fl / (ms_med * 1e-3) / 1e12, 2),
        "tflops_best": round(fl / (ms_min * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "FLUX joint attention forward, B=1 H=24 S=4608 (512 text + 64x64 image) D=128, "
                               "3-axis RoPE (16,56,56), no mask", "B": B, "H": H, "S": S, "D": D,
                   "parallelism": "none"},
        "pct_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "device": {**dinfo, "pct_of_device_peak": round(100.0 * tflops / peak_dev, 2) if peak_dev else None},
        "roofline": {
            "bound": "mfma",
            "achieved": round(k_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic("fwd_bf16_d128_flux_b1"),
            "kernel": "fwd_kernel<bf16,128,MASK_NONE,ROPE> (attention; Q rotated in its prologue, K rotated "
                      "in the key loop on its way into LDS)",
            "kernel_ms": round(k_ms, 5),
            "kernel_launches": k_launches,
            "note": "achieved = 4*B*H*S^2*D algorithmic flops over the attention kernel's average duration, "
                    "from HIP events the library records on the call's stream around that kernel during "
                    "the timed calls; a timed call (value) is three launches: pack_tables_kernel (the "
                    "caller's cos/sin repacked into (cos, sin) pairs), the attention kernel and "
                    "fwd_merge_kernel (the cut units' pieces)",
            "call_tflops": round(tflops, 2),
        },
        "train": train,
        "forward_variants": extra,
        "parity_rel_err": err,
        "cpu_baseline": base,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
