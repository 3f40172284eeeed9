"""Benchmark of the VDN layer forward on one MI355X.

A step is one ``vdn_forward`` of the whole layer (window softmax, VDA statistics and scans,
readout/gates/projections) over one batch of seeded synthetic inputs that are already resident in
HBM.  Prints one JSON line.  Default workload: one GPU's head share of a 768p clip (512 text
tokens, 75 latent frames x 1536 tokens, chunks of 5 frames, 5 heads of 128, bf16, anchors on).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 768p] [--no-cpu-baseline]
    python bench.py --forward-only ...         # only the timed forwards (for profiler runs)
    python bench.py --summarize-trace DIR --warmup W --steps K
    python bench.py --summarize-counters DIR [DIR ...] [--copy-counters DIR [DIR ...]]

The summaries read rocprofv3 CSV output (``--output-format csv``) of a ``--forward-only`` run: the
kernel trace gives each kernel's mean duration and, for the softmax, the mean of the K timed
dispatches (those after the W warm-up forwards) and the bf16 MFMA fraction it implies; the
counters give per-dispatch averages, the MFMA busy share and the HBM bytes per launch (scaled by
what FETCH_SIZE / WRITE_SIZE read for a plain copy of known size, from ``--copy-calibration``).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E


def key_frames(t, T, C, anchors):
    """Frames whose keys query frame t sees in the softmax (window plus anchors)."""
    c = t // C
    win = {f for f in range(T) if abs(f // C - c) <= 1}
    if anchors and t in (0, T - 1):
        return T
    if anchors:
        win |= {0, T - 1}
    return len(win)


def softmax_flops(w) -> float:
    """Algorithmic flops of the window softmax: 2 (QK) + 2 (PV) multiply-adds per (query, key, dim)."""
    pairs = sum(w.N * (w.n_text + w.N * key_frames(t, w.T, w.C, w.anchors)) for t in range(w.T))
    return 4.0 * w.d * w.H * pairs


def vda_bytes(w) -> float:
    """Algorithmic HBM bytes of the VDA statistics + scan: keys, values and beta of every scanned
    frame and of the text read once, plus the chunk states written."""
    s = 2 if w.dtype == "bf16" else 4
    scanned = w.T - (2 if (w.anchors and w.T > 1) else (1 if w.anchors else 0))
    nc = (w.T + w.C - 1) // w.C
    return w.H * ((scanned * w.N + w.n_text) * (2 * w.d * s + 4)) + 2 * nc * w.d * w.d * 4 * w.H


def stage_rooflines(w, ms):
    """Per-stage rooflines from per-stage milliseconds (the stages run one after the other)."""
    s = 2 if w.dtype == "bf16" else 4
    tok = w.T * w.N * w.H * w.d
    lk = (w.n_text + 63) // 64 * 64 + w.T * w.N
    out = {}
    def hbm(name, nbytes, t):
        if t > 0:
            out[name] = {"bound": "hbm", "ms": t, "algorithmic_GB": nbytes / 1e9,
                         "achieved_GBs": nbytes / (t * 1e-3) / 1e9, "frac": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    t = ms["softmax"]
    out["softmax"] = {"bound": "mfma", "ms": t, "achieved_TFLOPs": softmax_flops(w) / (t * 1e-3) / 1e12,
                      "frac": softmax_flops(w) / (t * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    hbm("prep", 2 * tok * s + 2 * w.n_text * w.H * w.d * s + 2 * w.H * lk * w.d * 2, ms["prep"])
    hbm("vda_stats+scan", vda_bytes(w), ms["vda_stats"] + ms["vda_scan"])
    hbm("epilogue", 3 * tok * s, ms["epilogue"])
    return out


def recorded_traffic(name="softmax_mfma"):
    """HBM bytes per launch of a softmax kernel (``softmax_mfma`` or ``softmax_fp8``) from the
    committed rocprofv3 byte-counter summary, if it was taken on the kernel's current source
    (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_768p_traffic.txt")
    src = os.path.join(ROOT, "linear_video_attention_amd", "csrc", f"{name}.hip")
    try:
        rec = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("source_sha256", "").strip() != sha:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _csv_rows(dirs, suffix):
    import csv
    import glob
    rows = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
            with open(f, newline="") as fh:
                rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize_trace(d, warmup, steps, workload):
    """Markdown summary of a rocprofv3 kernel trace of ``bench.py --forward-only``."""
    rows = _csv_rows([d], "kernel_trace.csv")
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    disp = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"])) for r in rows))
    per = {}
    for a, z, k in disp:
        per.setdefault(k, []).append((z - a) / 1e3)
    total = sum(sum(v) for v in per.values())
    lines = ["| kernel | calls | mean us | min us | total us | % of kernel time |", "|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v)} | {np.mean(v):.1f} | {np.min(v):.1f} | {sum(v):.1f} | {100 * sum(v) / total:.2f} |")
    w = __import__("synth").WORKLOADS[workload]
    flops = softmax_flops(w)
    out = ["\n".join(lines), ""]
    for k in sorted(per):
        if k.startswith("vdn::softmax_mfma_kernel<") and k.endswith("false>"):
            v = per[k]
            timed = v[warmup:warmup + steps]
            if len(timed) != steps:
                raise SystemExit(f"{k}: {len(v)} dispatches, expected at least {warmup + steps}")
            m = float(np.mean(timed))
            out.append(f"{k}: timed dispatches {warmup + 1}..{warmup + steps} of {len(v)}: mean {m:.1f} us, "
                       f"min {min(timed):.1f} us, max {max(timed):.1f} us; {flops / 1e12:.4f} TFLOP per launch "
                       f"-> {flops / (m * 1e-6) / 1e12:.1f} TFLOP/s = {flops / (m * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS:.4f} "
                       f"of the {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s bf16 dense peak")
    return "\n".join(out)


def summarize_counters(dirs, copy_dirs=()):
    """Markdown summary of rocprofv3 counter collections: per-kernel averages per dispatch, the MFMA
    busy share (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs) and HBM
    KiB per dispatch scaled by the copy calibration."""
    acc = {}
    for r in _csv_rows(dirs, "counter_collection.csv"):
        acc.setdefault(_short(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    scale = {}
    if copy_dirs:
        cal = {}
        for r in _csv_rows(copy_dirs, "counter_collection.csv"):
            if "copy" in r["Kernel_Name"].lower() and r["Counter_Name"] in ("FETCH_SIZE", "WRITE_SIZE"):
                cal.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        # the calibration copies 1 GiB: ideal FETCH = WRITE = 2^20 KiB per dispatch
        for c, v in cal.items():
            scale[c] = (1 << 20) / max(v)
    lines = []
    for k, cs in sorted(acc.items()):
        if not k.startswith("vdn::"):
            continue
        avg = {c: float(np.mean(v)) for c, v in cs.items()}
        parts = [f"{c} {v:.4g}" for c, v in sorted(avg.items())]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            parts.append(f"MFMA busy {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * avg['GRBM_GUI_ACTIVE'] / 8):.4f}")
        if "SQ_ACTIVE_INST_VALU" in avg and "GRBM_GUI_ACTIVE" in avg:
            parts.append(f"VALU busy {4 * avg['SQ_ACTIVE_INST_VALU'] / (1024 * avg['GRBM_GUI_ACTIVE'] / 8):.4f}")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in avg and c in scale:
                parts.append(f"{c} scaled {avg[c] * scale[c] * 1024 / 1e9:.4f} GB")
        lines.append(f"- {k}: " + "; ".join(parts))
    if scale:
        lines.append("- copy calibration factors: " + ", ".join(f"{c} x{v:.4f}" for c, v in sorted(scale.items())))
    return "\n".join(lines)


def cpu_baseline(w, inp, budget_rows=32768):
    """Time the CPU oracle on a bounded sample of the workload and scale it to video tokens/s.

    Sample: the full linear-branch state computation (all frames, all heads; a fixed cost of the
    whole layer) plus the softmax and merge of ``budget_rows`` query tokens drawn evenly from all
    frames (all heads).  The softmax time is scaled by (total query-key pairs / sampled pairs),
    the merge by (total rows / sampled rows)."""
    from oracle import vdn_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    rows = np.linspace(0, w.T * w.N - 1, budget_rows).astype(np.int64)
    t0 = time.perf_counter()
    o_l = orc.linear_branch(inp["q"], inp["k"], inp["v"], inp["beta"], inp["text_k"], inp["text_v"],
                            w.T, w.N, w.C, w.anchors, rows)
    t_lin = time.perf_counter() - t0
    t0 = time.perf_counter()
    o_s = orc.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], w.T, w.N, w.C,
                             w.anchors, rows)
    t_sm = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.merge(inp["q"][rows], o_s, o_l, inp["gate_w"], inp["proj_w"])
    t_mg = time.perf_counter() - t0
    pairs_sample = sum(w.n_text + w.N * key_frames(int(r) // w.N, w.T, w.C, w.anchors) for r in rows)
    pairs_total = sum(w.N * (w.n_text + w.N * key_frames(t, w.T, w.C, w.anchors)) for t in range(w.T))
    # the sampled linear-branch time includes its (tiny) per-row readout; treat it as fixed cost
    t_total = t_lin + t_sm * pairs_total / pairs_sample + t_mg * (w.T * w.N) / len(rows)
    return {
        "value": w.T * w.N / t_total,
        "unit": "video tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"all-frame VDA states ({t_lin:.1f} s) + softmax/merge of {len(rows)} of {w.T * w.N} "
                   f"query tokens x {w.H} heads ({t_sm:.1f} s), softmax scaled by query-key pairs"),
        "measured_s": round(t_lin + t_sm + t_mg, 2),
    }


def timed_steps(step, n):
    """Run n steps with a timing event between consecutive steps on torch's current stream (the
    plan's stream); returns the per-step milliseconds."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="768p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--with-overlap", action="store_true",
                    help="also time a plan that runs the linear branch on a side stream (context)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--forward-only", action="store_true",
                    help="only warm-up and timed forwards of the bf16 plan (for profiler runs)")
    ap.add_argument("--fp8", action="store_true", help="with --forward-only: time the FP8 softmax plan instead")
    ap.add_argument("--summarize-trace", metavar="DIR", help="summarise a rocprofv3 kernel trace (CPU only)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR", help="summarise rocprofv3 counters (CPU only)")
    ap.add_argument("--copy-counters", nargs="+", default=(), metavar="DIR",
                    help="counters of a --copy-calibration 1024 run, to scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps, args.workload))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.copy_counters))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the layer's head share runs on one device); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from linear_video_attention_amd import vdn
    from linear_video_attention_amd.vdn import Plan

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(w, seed=0, decay=True)      # alpha is drawn last: other inputs as without it
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(inp[k]).to("cuda").to(tdt).contiguous() for k in ("q", "k", "v", "gate_w", "proj_w")}
    beta = torch.from_numpy(inp["beta"]).to("cuda").contiguous()
    text_kv = torch.from_numpy(np.stack([inp["text_k"], inp["text_v"]])).to("cuda").to(tdt).contiguous()
    alpha = torch.from_numpy(inp["alpha"]).to("cuda").contiguous()
    out = torch.empty_like(dev["q"])
    plan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, fp8=args.forward_only and args.fp8)

    def forward(p, gate=None):
        p.forward(dev["q"], dev["k"], dev["v"], beta, text_kv, dev["gate_w"], dev["proj_w"], out, alpha=gate)

    for _ in range(args.warmup):
        forward(plan)
    torch.cuda.synchronize()
    # timed region: exactly `steps` forwards between two synchronisations; per-stage HIP events
    # (recorded by the library on the stream each stage runs on) and per-step events ride along
    plan.profile_enable(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per_step = timed_steps(lambda: forward(plan), args.steps)
    elapsed = time.perf_counter() - t0
    stage_ms, calls = plan.profile_read()
    ms_step = 1000.0 * elapsed / args.steps
    stages = {k: v / calls for k, v in stage_ms.items()}
    ref = out.clone()
    tokens = w.T * w.N

    sm_ms = stages["softmax_first"]      # the fixed-reference launch alone (the dominant kernel)
    flops = softmax_flops(w)
    achieved = flops / (sm_ms * 1e-3) / 1e12
    vda_ms = stages["vda_stats"] + stages["vda_scan"]
    roofline = {"bound": "mfma", "kernel": "softmax_mfma_kernel", "achieved": achieved,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": recorded_traffic(), "algorithmic_tflop_per_launch": flops / 1e12,
                "avg_launch_ms": sm_ms,
                "timing": "mean over the timed steps of HIP events recorded by the library on the softmax "
                          "stream around the fixed-reference launch of softmax_mfma_kernel alone",
                "softmax_stage_ms": stages["softmax"]}
    if args.forward_only:
        if args.fp8:
            roofline = {"kernel": "softmax_fp8_kernel", "avg_launch_ms": sm_ms,
                        "achieved": achieved, "unit": "TFLOP/s", "peak": MFMA_FP8_PEAK_TFLOPS,
                        "frac": achieved / MFMA_FP8_PEAK_TFLOPS}
        print(json.dumps({"metric": "VDN layer fwd: video tokens/sec (forward-only profiler run)",
                          "value": tokens / (ms_step * 1e-3), "unit": "video tokens/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
                          "stages_ms": stages, "roofline": roofline}), flush=True)
        plan.close()
        return

    # the linear-branch stages after a 1 GB write (cold Infinity Cache), three forwards
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    plan.profile_enable(3)
    for _ in range(3):
        flush.fill_(1.0)
        forward(plan)
    torch.cuda.synchronize()
    cold_ms, cold_calls = plan.profile_read()
    del flush
    vda_cold_ms = (cold_ms["vda_stats"] + cold_ms["vda_scan"]) / cold_calls

    # the same layer with the channel-wise decay gate on the linear branch (context)
    n_dec = max(3, min(args.steps, 10))
    forward(plan, alpha)
    torch.cuda.synchronize()
    plan.profile_enable(n_dec)
    dec = timed_steps(lambda: forward(plan, alpha), n_dec)
    dec_ms, dec_calls = plan.profile_read()
    decay = {"ms_per_step_median": float(np.median(dec)),
             "vda_ms": (dec_ms["vda_stats"] + dec_ms["vda_scan"]) / dec_calls}

    # the backward pass for a seeded output gradient (context): one call recomputes the forward
    # quantities it needs, then runs every transposed stage
    dout = torch.from_numpy(np.random.default_rng(7).standard_normal(out.shape, dtype=np.float32)).to("cuda").to(tdt)
    backward = lambda: plan.backward(dev["q"], dev["k"], dev["v"], beta, text_kv, dev["gate_w"], dev["proj_w"], dout)
    backward()
    torch.cuda.synchronize()
    n_bwd = max(2, min(args.steps, 5))
    bwd_ms = timed_steps(backward, n_bwd)
    bwd_med = float(np.median(bwd_ms))
    # a training step that reuses the forward's intermediates: forward, then vdn_backward_after_forward
    train = lambda: (forward(plan), plan.backward(dev["q"], dev["k"], dev["v"], beta, text_kv, dev["gate_w"],
                                                  dev["proj_w"], dout, after_forward=True))
    train()
    torch.cuda.synchronize()
    train_med = float(np.median(timed_steps(train, n_bwd)))
    backward_info = {"ms_per_call_median": bwd_med, "calls": n_bwd,
                     "train_step_tokens_per_s": tokens / ((float(np.median(per_step)) + bwd_med) * 1e-3),
                     "train_step_after_forward_ms_median": train_med,
                     "train_step_after_forward_tokens_per_s": tokens / (train_med * 1e-3),
                     "softmax_backward_algorithmic_tflop": 3.5 * flops / 1e12}
    del dout
    plan.close()

    # the joint sequence (context): 576 audio tokens after the text (14.4 s at 40 audio latents per
    # second) and the text and audio query rows; forward (vdn_forward_joint) and backward
    # (vdn_backward_joint, which recomputes the forward), seeded extras of the same distributions
    n_audio = 576
    n_ctx = w.n_text + n_audio
    jr = np.random.default_rng(1)
    unit = lambda x: (x / np.linalg.norm(x.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    audio_k = unit(jr.standard_normal((n_audio, w.H, w.d), dtype=np.float32))
    audio_v = jr.standard_normal((n_audio, w.H, w.d), dtype=np.float32)
    ctx_q = torch.from_numpy(unit(jr.standard_normal((n_ctx, w.H, w.d), dtype=np.float32))).to("cuda").to(tdt)
    ctx_kv = torch.from_numpy(np.stack([np.concatenate([inp["text_k"], audio_k]),
                                        np.concatenate([inp["text_v"], audio_v])])).to("cuda").to(tdt).contiguous()
    dctx = torch.from_numpy(jr.standard_normal((n_ctx, w.H, w.d), dtype=np.float32)).to("cuda").to(tdt)
    dout = torch.from_numpy(np.random.default_rng(7).standard_normal(out.shape, dtype=np.float32)).to("cuda").to(tdt)
    jplan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, n_audio=n_audio)
    ctx_out = torch.empty_like(ctx_q)
    jfwd = lambda: jplan.forward(dev["q"], dev["k"], dev["v"], beta, ctx_kv, dev["gate_w"], dev["proj_w"], out,
                                 ctx_q=ctx_q, ctx_out=ctx_out)
    jbwd = lambda: jplan.backward(dev["q"], dev["k"], dev["v"], beta, ctx_kv, dev["gate_w"], dev["proj_w"], dout,
                                  ctx_q=ctx_q, dctx_out=dctx)
    jfwd()
    jbwd()
    torch.cuda.synchronize()
    jf_med = float(np.median(timed_steps(jfwd, max(3, min(args.steps, 10)))))
    jb_med = float(np.median(timed_steps(jbwd, n_bwd)))
    joint_info = {"n_audio": n_audio, "context_query_rows": n_ctx, "forward_ms_median": jf_med,
                  "forward_tokens_per_s": (tokens + n_ctx) / (jf_med * 1e-3),
                  "backward_ms_median": jb_med, "backward_calls": n_bwd}
    del dout, dctx, ctx_q, ctx_kv, ctx_out
    jplan.close()

    # the FP8 (E4M3) softmax variant of the same layer (context: the headline value is bf16)
    fplan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, fp8=True)
    for _ in range(2):
        forward(fplan)
    torch.cuda.synchronize()
    n_f8 = max(3, min(args.steps, 10))
    fplan.profile_enable(n_f8)
    f8_steps = timed_steps(lambda: forward(fplan), n_f8)
    f8_ms, f8_calls = fplan.profile_read()
    sm8 = f8_ms["softmax_first"] / f8_calls
    f8_med = float(np.median(f8_steps))
    fp8_info = {"ms_per_step_median": f8_med, "tokens_per_s": tokens / (f8_med * 1e-3),
                "stages_ms": {k: v / f8_calls for k, v in f8_ms.items()},
                "softmax_kernel": "softmax_fp8_kernel", "softmax_achieved_TFLOPs": flops / (sm8 * 1e-3) / 1e12,
                "softmax_frac_fp8_peak": flops / (sm8 * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
                "fp8_peak_TFLOPs": MFMA_FP8_PEAK_TFLOPS, "softmax_traffic": recorded_traffic("softmax_fp8")}
    fplan.close()

    # the MXFP8 epilogue variant (gate and projection products in MXFP8), alone and with the FP8
    # softmax (context)
    mx_info = {}
    for name, kw in (("fp8_epilogue", {"fp8_epilogue": True}), ("fp8_softmax_and_epilogue", {"fp8": True, "fp8_epilogue": True})):
        mplan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, **kw)
        for _ in range(2):
            forward(mplan)
        torch.cuda.synchronize()
        mplan.profile_enable(n_f8)
        m_steps = timed_steps(lambda: forward(mplan), n_f8)
        m_ms, m_calls = mplan.profile_read()
        mx_info[name] = {"ms_per_step_median": float(np.median(m_steps)),
                         "tokens_per_s": tokens / (float(np.median(m_steps)) * 1e-3),
                         "stages_ms": {k: v / m_calls for k, v in m_ms.items()}}
        mplan.close()

    overlapped = None
    if args.with_overlap:
        # the linear branch on a side stream next to the softmax branch (context only)
        oplan = Plan(w.T, w.N, w.C, w.n_text, w.H, w.d, w.anchors, w.dtype, overlap=True)
        for _ in range(2):
            forward(oplan)
        ov = timed_steps(lambda: forward(oplan), max(3, min(args.steps, 10)))
        overlapped = {"ms_per_step_median": float(np.median(ov)), "outputs_identical": bool(torch.equal(out, ref))}
        oplan.close()

    mfma_onbox = vdn.measure_mfma_bf16_tflops()
    copy_onbox = vdn.measure_copy_gbs(1 << 30)
    vb = vda_bytes(w)
    result = {
        "metric": "VDN layer fwd: video tokens/sec on 1 MI355X + % bf16 MFMA peak / % HBM BW",
        "value": tokens / (ms_step * 1e-3),
        "unit": "video tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; q/k L2-normalised N(0,1), v N(0,1), beta sigmoid(N(0,1)), weights N(0,1/d))",
        "config": {"workload": f"{w.name}: n_text={w.n_text} T={w.T} N={w.N} C={w.C} H={w.H} d={w.d} anchors={int(w.anchors)}",
                   "n_text": w.n_text, "T": w.T, "N": w.N, "C": w.C, "H": w.H, "d": w.d},
        "roofline": dict(roofline, onbox_peak=mfma_onbox, frac_onbox=achieved / mfma_onbox),
        "step_ms": {"median": float(np.median(per_step)), "min": float(np.min(per_step))},
        "stages_ms": stages,
        "stage_rooflines": stage_rooflines(w, stages),
        "vda": {"ms": vda_ms, "ms_cold_cache": vda_cold_ms, "algorithmic_bytes": vb,
                "achieved_GBs": vb / (vda_ms * 1e-3) / 1e9, "frac_hbm": vb / (vda_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "frac_hbm_cold_cache": vb / (vda_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "frac_onbox_copy": vb / (vda_ms * 1e-3) / 1e9 / copy_onbox},
        "onbox": {"mfma_bf16_tflops": mfma_onbox, "copy_gbs": copy_onbox},
    }
    decay["vda_frac_hbm"] = (vb + 4 * w.T * w.H * w.d) / (decay["vda_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
    result["decay_gate"] = decay
    result["backward"] = backward_info
    result["joint"] = joint_info
    result["fp8_softmax"] = fp8_info
    result.update(mx_info)
    if overlapped is not None:
        result["overlapped_branches"] = overlapped
    del dev, beta, text_kv, alpha, out, ref
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
