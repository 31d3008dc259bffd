#!/usr/bin/env python3
"""Benchmark: Hybrid-Engine experience generation on one MI355X.

One step = the generation phase of one RLHF iteration for one batch: fold the
LoRA adapters into the actor (he_fuse_lora), greedy-generate 256 tokens for each
256-token prompt (he_generate: prompt pass + 255 decode steps replayed from a
hipGraph), unfold the adapters (he_unfuse_lora).  Default workload: the OPT-6.7B
shape (32 layers, d 4096, 32 heads, FFN 16384, vocab 50272), bf16, LoRA rank 16,
batch 64, synthetic seeded weights and prompts (pretrained weights and the
prompt dataset are not available; the inputs have their shapes).

Prints one JSON line.  value = generated tokens / s over whole steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
CAL_BYTES = 512 << 20      # calibration copy for the byte counters: 512 MiB read, 512 MiB written
BF16_PEAK = 2.5e15         # MI355X dense bf16 MFMA, flop/s
METRIC = "experience-gen tokens/s + decode HBM roofline %, OPT-6.7B-shape b64 256->256"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic(wl):
    """Algorithmic bytes of the decode steps and flops of the prompt pass."""
    a = wl.actor
    L, d, F, V, B = a.n_layers, a.d_model, a.d_ffn, a.vocab, wl.batch
    es = 2 if a.dtype == "bf16" else 4
    layer_w = (4 * d * d + 2 * d * F) * es + (3 * d + d + F + d + 4 * d) * es   # weights, biases, LN
    step_w = L * layer_w + V * d * es + 2 * d * es + 0 * B                        # + tied head + final LN
    S = wl.prompt_len
    dec_bytes = 0.0
    dec_flops = 0.0
    for j in range(1, wl.gen_len):
        pos = S + j - 1                     # position fed at step j; attends over pos + 1 keys
        kv = 2.0 * L * B * d * es * (pos + 1)   # read pos cached positions + write one
        dec_bytes += step_w + kv
        dec_flops += 2.0 * B * (L * (4 * d * d + 2 * d * F) + d * V) + 4.0 * L * B * d * (pos + 1)
    pre_flops = 2.0 * B * S * L * (4 * d * d + 2 * d * F) + 2.0 * L * d * S * (S + 1) * B + 2.0 * B * d * V
    return dec_bytes, dec_flops, pre_flops, step_w


def cpu_baseline(wl, seed=0):
    """The CPU oracle timed on the sampled rows {0, 1, B/2, B-1} of the workload, whole:
    the LoRA fold of every layer, the prompt pass of those rows and all gen_len - 1
    cached decode steps (greedy, the oracle's own picks), every layer; then one decode
    step of the full batch (its KV cache holds prompt_len positions of synthetic
    contents, since only the step's cost is wanted).  Nothing is extrapolated: the rate
    is the sampled rows' generated tokens over the measured time."""
    import numpy as np

    import synth
    from oracle import opt_he as O

    a = wl.actor
    B = wl.batch
    rows = sorted({0, 1, B // 2, B - 1})
    t0 = time.time()
    params = synth.model_params(a, seed)
    lora = synth.lora_params(a, wl.lora_rank, seed)
    prompts = synth.prompts(wl, seed).numpy()
    log(f"cpu baseline inputs ready in {time.time() - t0:.1f}s")
    om = O.OracleModel(a, params, O.Precision("bf16"), lora=lora, lora_scale=wl.lora_scale,
                       cache_layers=True)
    t = time.time()
    for i in range(a.n_layers):
        om.layer(i)                         # LoRA fold (and widening) of every layer
    t_fold = time.time() - t
    log(f"cpu baseline: fold {t_fold:.1f}s")
    t = time.time()
    lg, cache = om.prefill(prompts[rows], wl.max_seq)
    t_prefill = time.time() - t
    nxt = O.argmax_lowest(lg)
    log(f"cpu baseline: prompt pass {t_prefill:.1f}s")
    t = time.time()
    for j in range(1, wl.gen_len):
        nxt = O.argmax_lowest(om.decode(nxt, cache))
        if j % 32 == 0:
            log(f"cpu baseline: decode step {j} at {time.time() - t:.1f}s")
    t_decode = time.time() - t
    # one decode step of the full batch at position prompt_len (synthetic cache contents)
    full = O.KVCache(a.n_layers, B, a.n_heads, wl.max_seq, a.head_dim)
    full.length = wl.prompt_len
    t = time.time()
    om.decode(prompts[:, -1], full)
    t_full_step = time.time() - t
    del full, cache
    om._layers.clear()
    blas, cores = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            blas, cores = pools[0].get("internal_api", "unknown"), pools[0].get("num_threads")
    except Exception:
        pass
    if cores is None:
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count()
    R, G = len(rows), wl.gen_len
    return {
        "value": R * G / (t_prefill + t_decode), "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"rows {rows} of the batch of {B}, all {a.n_layers} layers: LoRA fold of every layer "
                   f"{t_fold:.1f}s, prompt pass ({wl.prompt_len} tokens) {t_prefill:.1f}s, {G - 1} cached "
                   f"decode steps {t_decode:.1f}s; value = {R} x {G} generated tokens / (prompt pass + decode); "
                   f"one decode step of the full batch of {B} at position {wl.prompt_len} {t_full_step:.2f}s"),
        "step_tokens_per_s": R * G / (t_fold + t_prefill + t_decode),
        "full_batch_decode_step_s": t_full_step,
        "full_batch_decode_tokens_per_s": B / t_full_step,
        "blas": blas, "precision": "float64 with bf16 storage rounding",
    }


# ---------------------------------------------------------------------------------
# rocprofv3 output -> committed summaries (profiles/)
# ---------------------------------------------------------------------------------
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["transformer_decode_amd/csrc/k_gemv.hip", "transformer_decode_amd/csrc/k_attn.hip",
                  "transformer_decode_amd/csrc/k_elem.hip", "transformer_decode_amd/csrc/common.h"]


def kernel_class(name):
    """The bench's kernel classes, from a kernel's demangled name."""
    if "gemv_il_kernel" in name or "gemv_f32_kernel" in name:
        # gemv_il_kernel<MT, FR, NWK, OUT, F8>: OUT 2 is the LM head's pick epilogue
        targs = name.split("<", 1)[1].split(">", 1)[0].split(",") if "<" in name else []
        mode = targs[3].strip() if "gemv_il_kernel" in name and len(targs) > 3 else targs[0].strip() if targs else ""
        return "lmhead" if mode in ("2", "GV_ARGMAX") or "ARGMAX" in name else "gemv_decode"
    if "attn_decode_kernel" in name:
        return "attn_decode"
    if "gemm_" in name:
        return "gemm_prefill"
    if "attn_prefill" in name:
        return "attn_prefill"
    if "lora" in name:
        return "lora"
    if "norm_" in name or "embed_" in name or "reduce_" in name:
        return "embed_norm"
    return "other"


def sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counters_summary(fetch_csv, write_csv, workload, command):
    """Per-class HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the counter reads for the calibration copy of
    CAL_BYTES (the runtime's copy kernel, the dispatches of that size)."""
    import csv
    out = {"workload": workload, "command": command, "sources_sha": sources_sha(), "classes": {}}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = list(csv.DictReader(open(path)))
        cal = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]
               and float(r["Counter_Value"]) * 1024 > CAL_BYTES / 4]
        factor = CAL_BYTES / (sum(cal) / len(cal)) if cal else None
        out[f"{key}_factor"] = factor
        out[f"{key}_calibration_readings_bytes"] = cal
        acc = {}
        for r in rows:
            c = kernel_class(r["Kernel_Name"])
            acc.setdefault(c, []).append(float(r["Counter_Value"]) * 1024)
        for c, v in acc.items():
            e = out["classes"].setdefault(c, {})
            e[f"{key}_raw_bytes_per_dispatch"] = sum(v) / len(v)
            e[f"{key}_bytes_per_dispatch"] = sum(v) / len(v) * (factor or float("nan"))
            e["dispatches"] = len(v)
    for e in out["classes"].values():
        e["traffic_bytes_per_dispatch"] = e.get("fetch_bytes_per_dispatch", 0.0) + e.get("write_bytes_per_dispatch", 0.0)
    return out


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16",)


def mfma_summary(csv_path, workload, command):
    """Per-kernel MFMA work from one rocprofv3 --pmc pass of MFMA_COUNTERS: bf16 MFMA
    flops = MOPS x 512 per dispatch, to set beside the algorithmic 2 M N K.  The rate
    against peak comes from kernel time, not from a busy-cycle ratio."""
    import csv
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        d = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = {}
    for d in disp.values():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in d or d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] <= 0:
            continue
        e = per.setdefault(d["name"], [0, 0.0])
        e[0] += 1
        e[1] += d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    lines = [f"# MFMA work, {workload}", "", "Command (run from the repository root, output under "
             "gpurun_out/):", "", "```", command, "```", "",
             "bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per dispatch (the counter counts 512-flop "
             "units): the work the MFMAs did, to compare with the algorithmic 2 M N K of each GEMM. The rate "
             "against the bf16 peak is taken from kernel time (kernel summaries and the bench line).", "",
             "| kernel | dispatches | MFMA TFLOP per dispatch |", "|---|---|---|"]
    for name, (n, fl) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{name[:100]}` | {n} | {fl / n / 1e12:.4f} |")
    return "\n".join(lines) + "\n"


# One --pmc pass (8 SQ counters): how busy the LDS and the MFMA pipes are per kernel class.
OCC_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
                "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES")


def occupancy_summary(csv_path, workload, command, n_cu=256):
    """Per kernel class, from one rocprofv3 --pmc pass of OCC_COUNTERS: the counters summed
    over the class's dispatches, and ratios to SQ_BUSY_CU_CYCLES (summed over the CUs, so
    busy cycles / CUs / kernel time is the clock the kernels ran at).  MFMA busy cycles are
    counted per SIMD, so their ratio is divided by the 4 SIMDs of a CU."""
    import csv
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        d = disp.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                               "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    cls = {}
    for d in disp.values():
        c = kernel_class(d["name"])
        if c == "other":
            continue
        e = cls.setdefault(c, {"n": 0, "ns": 0.0})
        e["n"] += 1
        e["ns"] += d["ns"]
        for k in OCC_COUNTERS:
            e[k] = e.get(k, 0.0) + d.get(k, 0.0)
    lines = [f"# LDS and MFMA activity, {workload}", "", "Command (run from the repository root, output under "
             "gpurun_out/):", "", "```", command, "```", "",
             "Per kernel class, summed over its dispatches of the run. busy = SQ_BUSY_CU_CYCLES (summed over "
             f"the {n_cu} CUs); clock = busy / CUs / kernel time (meaningful for kernels that keep every CU busy; "
             "it reads low for the 64-WG decode norms in embed_norm); LDS active = SQ_LDS_IDX_ACTIVE / busy; bank "
             "conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; FIFO full = SQ_LDS_DATA_FIFO_FULL / busy; "
             "MFMA busy per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / busy / 4.", "",
             "| class | dispatches | avg us | clock (GHz) | LDS active | bank conflicts | LDS data FIFO full | "
             "MFMA busy per SIMD |", "|---|---|---|---|---|---|---|---|"]
    for c, e in sorted(cls.items(), key=lambda kv: -kv[1]["ns"]):
        busy = e["SQ_BUSY_CU_CYCLES"] or 1.0
        lines.append(f"| {c} | {e['n']} | {e['ns'] / e['n'] / 1e3:.1f} | {busy / n_cu / e['ns']:.2f} | "
                     f"{e['SQ_LDS_IDX_ACTIVE'] / busy:.3f} | "
                     f"{e['SQ_LDS_BANK_CONFLICT'] / max(1.0, e['SQ_LDS_IDX_ACTIVE']):.3f} | "
                     f"{e['SQ_LDS_DATA_FIFO_FULL'] / busy:.3f} | {e['SQ_VALU_MFMA_BUSY_CYCLES'] / busy / 4:.3f} |")
    return "\n".join(lines) + "\n"


def stats_summary(stats_csv, workload, command):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# Kernel time, {workload}", "", "Command (run from the repository root, output under gpurun_out/):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | total ms | share |", "|---|---|---|---|---|"]
    cls = {}
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = r["Name"]
        lines.append(f"| `{n[:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['TotalDurationNs']) / tot * 100:.1f}% |")
        c = cls.setdefault(kernel_class(n), [0, 0.0])
        c[0] += int(r["Calls"])
        c[1] += float(r["TotalDurationNs"])
    lines += ["", "Per class (the bench's kernel classes):", "", "| class | calls | avg us | total ms |", "|---|---|---|---|"]
    for c, (n, t) in sorted(cls.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| {c} | {n} | {t / n / 1e3:.2f} | {t / 1e6:.2f} |")
    lines.append(f"\nTotal kernel time {tot / 1e6:.1f} ms.")
    return "\n".join(lines) + "\n"


def timeline_summary(trace_csv, workload, command):
    """The decode steps of a rocprofv3 kernel trace (dispatch start and end on the GPU's
    clock): each step runs from one step-opening embedding dispatch to the next.  Per
    step the span, the time inside kernels and the idle gaps between dispatches; per
    kernel its average duration and the average gap before the next dispatch."""
    import csv
    import statistics
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    opens = [i for i, r in enumerate(rows) if "embed_norm" in r["Kernel_Name"]]
    steps = []
    for a, b in zip(opens, opens[1:]):
        names = [rows[i]["Kernel_Name"] for i in range(a, b)]
        if any("gemv_il" in n for n in names) and not any("gemm_" in n for n in names):
            steps.append((a, b))
    if steps:   # whole steps only: the interval that spans a generation's end holds other work
        from collections import Counter
        common = Counter(b - a for a, b in steps).most_common(1)[0][0]
        steps = [(a, b) for a, b in steps if b - a == common]
    per, spans, busy, gaps = {}, [], [], []
    for a, b in steps:
        spans.append((int(rows[b]["Start_Timestamp"]) - int(rows[a]["Start_Timestamp"])) / 1e3)
        k_sum = g_sum = 0.0
        for i in range(a, b):
            r = rows[i]
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            gap = (int(rows[i + 1]["Start_Timestamp"]) - int(r["End_Timestamp"])) / 1e3
            k_sum += dur
            g_sum += gap
            gaps.append(gap)
            e = per.setdefault(r["Kernel_Name"].split("(")[0][:90], [0, 0.0, 0.0])
            e[0] += 1
            e[1] += dur
            e[2] += gap
        busy.append(k_sum)
    n = len(steps)
    lines = [f"# Decode-step dispatch timeline, {workload}", "", "Command (run from the repository root, output "
             "under gpurun_out/):", "", "```", command, "```", "",
             f"{n} decode steps of {steps[0][1] - steps[0][0] if steps else 0} dispatches (graph replay). "
             "Times are the GPU's dispatch start and end stamps; a gap is the time from one dispatch's end "
             "to the next one's start. A step is one replay of the decode graph; the gap after its last "
             "dispatch is the time between two graph launches.", "",
             "| per step | mean | median |", "|---|---|---|",
             f"| span (us) | {statistics.mean(spans):.1f} | {statistics.median(spans):.1f} |",
             f"| inside kernels (us) | {statistics.mean(busy):.1f} | {statistics.median(busy):.1f} |",
             f"| gaps between dispatches (us) | {statistics.mean(spans) - statistics.mean(busy):.1f} | "
             f"{statistics.median([s - k for s, k in zip(spans, busy)]):.1f} |",
             f"| gap per dispatch (us) | {statistics.mean(gaps):.2f} | {statistics.median(gaps):.2f} |", "",
             "| kernel | dispatches per step | avg duration (us) | avg gap after (us) |", "|---|---|---|---|"]
    for name, (c, d, g) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{name}` | {c / n:.0f} | {d / c:.2f} | {g / c:.2f} |")
    return "\n".join(lines) + "\n"


def two_round_sequence(wl, a, dev, ldev, prompts, seed):
    """The largest workload's sequence (page 2, section 3: release the workspace after
    generation, retake it before the next): round 1 fuse, generate, unfuse, release;
    round 2 retake, fuse, generate, unfuse, release; then the reward model scores the
    round-2 experience (prompt + answer).  Times of each call, the memory the release
    returns, and whether round 2 repeats round 1's tokens (same adapters; it may part from
    them at a near-tie, since the unfold restores each adapted weight to within one bf16
    spacing and round 2 folds the adapters into those bits)."""
    import torch

    import synth
    from transformer_decode_amd import he

    B, S, G = wl.batch, wl.prompt_len, wl.gen_len
    eng = he.Engine(a, dev)
    ctx, st = eng.ctx, eng.stream
    lt, _keep = eng.lora(ldev, wl.lora_rank, wl.lora_alpha)
    out = [torch.empty(B, G, dtype=torch.int32, device="cuda") for _ in range(2)]
    rec = {}
    torch.cuda.synchronize()
    t_all = time.time()
    for rnd in (1, 2):
        free0 = torch.cuda.mem_get_info()[0]
        t = time.time()
        with torch.cuda.stream(st):
            he.he_retake_cache(ctx, B, wl.max_seq)
            he.he_sync(ctx)
        rec[f"round{rnd}_retake_ms"] = (time.time() - t) * 1e3
        E = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        with torch.cuda.stream(st):
            E[0].record(st)
            he.he_fuse_lora(ctx, lt)
            E[1].record(st)
            he.he_generate(ctx, prompts.data_ptr(), B, S, G, out[rnd - 1].data_ptr())
            E[2].record(st)
            he.he_unfuse_lora(ctx, lt)
            E[3].record(st)
            he.he_sync(ctx)
        free1 = torch.cuda.mem_get_info()[0]
        t = time.time()
        with torch.cuda.stream(st):
            he.he_release_cache(ctx)
            he.he_sync(ctx)
        rec[f"round{rnd}_release_ms"] = (time.time() - t) * 1e3
        free2 = torch.cuda.mem_get_info()[0]
        rec[f"round{rnd}_fuse_ms"] = E[0].elapsed_time(E[1])
        rec[f"round{rnd}_generate_ms"] = E[1].elapsed_time(E[2])
        rec[f"round{rnd}_unfuse_ms"] = E[2].elapsed_time(E[3])
        rec[f"round{rnd}_gen_tokens_per_s"] = B * G / (E[1].elapsed_time(E[2]) / 1e3)
        rec[f"round{rnd}_workspace_GB"] = (free0 - free1) / 1e9
        rec[f"round{rnd}_returned_GB"] = (free2 - free1) / 1e9
    rec["round2_equals_round1"] = bool(torch.equal(out[0], out[1]))
    eng.close()
    rs = wl.reward
    rdev = {k: v.cuda() for k, v in synth.model_params(rs, seed, prefix="rm.").items()}
    exp = torch.cat([prompts, out[1]], dim=1).to(torch.int32).contiguous()
    reward = torch.empty(B, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    eng3 = he.Engine(rs, rdev)
    E = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(eng3.stream):
        he.he_retake_cache(eng3.ctx, B, S + G)
        E[0].record(eng3.stream)
        he.he_score(eng3.ctx, exp.data_ptr(), B, S + G, reward.data_ptr())
        E[1].record(eng3.stream)
        he.he_release_cache(eng3.ctx)
        he.he_sync(eng3.ctx)
    eng3.close()
    torch.cuda.synchronize()
    rec["reward_scoring_ms"] = E[0].elapsed_time(E[1])
    rec["rewards_finite"] = bool(torch.isfinite(reward).all().item())
    rec["wall_s"] = time.time() - t_all
    del rdev
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="opt6.7b")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-phase / per-kernel passes")
    ap.add_argument("--no-extras", action="store_true",
                    help="keep the per-phase and per-kernel passes, skip the other modes (sampling, FP8 decode, "
                         "scoring, the no-graph decode, the reward model)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="for counter collection: a calibration copy, then fuse + prefill + N decode "
                         "steps + unfuse once; prints nothing and exits")
    ap.add_argument("--counters-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection.csv files into "
                         "the per-class traffic summary (no GPU)")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="turn a rocprofv3 --stats kernel_stats.csv into a markdown summary (no GPU)")
    ap.add_argument("--timeline-summary", nargs=2, metavar=("TRACE_CSV", "OUT_MD"),
                    help="write the decode-step dispatch timeline of a rocprofv3 kernel trace")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("MFMA_CSV", "OUT_MD"),
                    help="turn a rocprofv3 --pmc pass of the MFMA counters into a markdown summary (no GPU)")
    ap.add_argument("--occupancy-summary", nargs=2, metavar=("PMC_CSV", "OUT_MD"),
                    help="turn a rocprofv3 --pmc pass of the LDS / MFMA activity counters into a markdown "
                         "summary (no GPU)")
    ap.add_argument("--command", default="", help="the command that produced the csv (recorded; "
                    "default: the standard profiling command for the summary being written)")
    args = ap.parse_args()

    if args.counters_summary:
        f, w, o = args.counters_summary
        cmd = args.command or (
            f"export TMPDIR=/tmp && "
            f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_fetch -o fetch -- "
            f"python3 bench.py --workload {args.workload} --trace-steps 3 && "
            f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_write -o write -- "
            f"python3 bench.py --workload {args.workload} --trace-steps 3 && "
            f"python3 bench.py --workload {args.workload} --counters-summary {f} {w} {o}")
        summ = counters_summary(f, w, args.workload, cmd)
        with open(o, "w") as fh:
            json.dump(summ, fh, indent=1)
        print(json.dumps(summ["classes"], indent=1))
        return
    if args.mfma_summary:
        m_csv, o = args.mfma_summary
        cmd = args.command or (
            f"export TMPDIR=/tmp && "
            f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} -f csv -d gpurun_out/pmc_mfma -o mfma -- "
            f"python3 bench.py --workload {args.workload} --trace-steps 3 && "
            f"python3 bench.py --workload {args.workload} --mfma-summary {m_csv} {o}")
        with open(o, "w") as fh:
            fh.write(mfma_summary(m_csv, args.workload, cmd))
        return
    if args.occupancy_summary:
        p_csv, o = args.occupancy_summary
        cmd = args.command or (
            f"export TMPDIR=/tmp && "
            f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(OCC_COUNTERS)} -f csv -d gpurun_out/pmc_lds -o lds -- "
            f"python3 bench.py --workload {args.workload} --trace-steps 3 && "
            f"python3 bench.py --workload {args.workload} --occupancy-summary {p_csv} {o}")
        with open(o, "w") as fh:
            fh.write(occupancy_summary(p_csv, args.workload, cmd))
        return
    if args.timeline_summary:
        tr_csv, o = args.timeline_summary
        cmd = args.command or (
            f"export TMPDIR=/tmp && "
            f"timeout -k 10 400 rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof -o bench -- "
            f"python3 bench.py --workload {args.workload} --steps 1 --warmup 1 --no-cpu --no-breakdown && "
            f"python3 bench.py --workload {args.workload} --timeline-summary {tr_csv} {o}")
        with open(o, "w") as fh:
            fh.write(timeline_summary(tr_csv, args.workload, cmd))
        return
    if args.stats_summary:
        st_csv, o = args.stats_summary
        cmd = args.command or (
            f"export TMPDIR=/tmp && "
            f"timeout -k 10 400 rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof -o bench -- "
            f"python3 bench.py --workload {args.workload} --steps 1 --warmup 1 --no-cpu --no-breakdown && "
            f"python3 bench.py --workload {args.workload} --stats-summary {st_csv} {o}")
        with open(o, "w") as fh:
            fh.write(stats_summary(st_csv, args.workload, cmd))
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(experience generation is data parallel over prompts: run one process per GPU, "
              f"each on its own batch)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from transformer_decode_amd import he

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    wl = synth.WORKLOADS[args.workload]
    a = wl.actor
    B, S, G = wl.batch, wl.prompt_len, wl.gen_len

    t0 = time.time()
    params = synth.model_params(a, args.seed)
    lora = synth.lora_params(a, wl.lora_rank, args.seed)
    log(f"inputs generated in {time.time() - t0:.1f}s")
    dev = {k: v.cuda() for k, v in params.items()}
    ldev = {k: v.cuda() for k, v in lora.items()}
    del params, lora
    prompts = synth.prompts(wl, args.seed).cuda()
    out = torch.empty(B, G, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"uploaded in {time.time() - t0:.1f}s")

    eng = he.Engine(a, dev, use_graph=not args.no_graph)
    ctx, st = eng.ctx, eng.stream
    lt, _keep = eng.lora(ldev, wl.lora_rank, wl.lora_alpha)

    t = time.time()
    with torch.cuda.stream(st):
        he.he_retake_cache(ctx, B, wl.max_seq)
        he.he_sync(ctx)
    t_retake = time.time() - t

    if args.trace_steps:
        # calibration for the byte counters: a plain copy of known size (torch's own
        # copy kernel) before the traced steps
        src = torch.ones(CAL_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        with torch.cuda.stream(st):
            he.he_fuse_lora(ctx, lt)
            he.he_prefill(ctx, prompts.data_ptr(), B, S, nxt.data_ptr(), 0)
            for _ in range(args.trace_steps):
                he.he_decode_step(ctx, nxt.data_ptr(), nxt.data_ptr(), 0)
            he.he_unfuse_lora(ctx, lt)
            he.he_release_cache(ctx)
            he.he_sync(ctx)
        eng.close()
        log(f"trace run done: prefill + {args.trace_steps} decode steps")
        return

    def step():
        he.he_fuse_lora(ctx, lt)
        he.he_generate(ctx, prompts.data_ptr(), B, S, G, out.data_ptr())
        he.he_unfuse_lora(ctx, lt)

    with torch.cuda.stream(st):
        for _ in range(args.warmup):
            step()
        he.he_sync(ctx)
        log("warmup done")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(st)
        w0 = time.time()
        for i in range(args.steps):
            step()
            evs[i + 1].record(st)
        he.he_sync(ctx)
        torch.cuda.synchronize()
        wall = time.time() - w0
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    value = B * G / (ms / 1e3)
    log(f"timed {args.steps} steps: {ms:.1f} ms/step (wall {wall / args.steps * 1e3:.1f} ms/step)")

    dec_bytes, dec_flops, pre_flops, step_w = algorithmic(wl)
    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if a.dtype == "bf16" else "f32", "data": "synthetic",
        "ms_per_step_each": per_step, "ms_per_step_median": sorted(per_step)[len(per_step) // 2],
        "config": {"workload": f"{wl.name}-shape actor, batch {B}, prompt {S}, generate {G} greedy, "
                               f"LoRA rank {wl.lora_rank} fused before / unfused after",
                   "layers": a.n_layers, "d_model": a.d_model, "heads": a.n_heads, "ffn": a.d_ffn,
                   "vocab": a.vocab, "batch": B, "prompt_len": S, "gen_len": G,
                   "lora_rank": wl.lora_rank, "hip_graph": not args.no_graph},
    }

    if not args.no_breakdown:
        # per-phase times: the same step split into its calls, each bracketed by events
        with torch.cuda.stream(st):
            E = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            nxt = torch.empty(B, dtype=torch.int32, device="cuda")
            E[0].record(st)
            he.he_fuse_lora(ctx, lt)
            E[1].record(st)
            he.he_prefill(ctx, prompts.data_ptr(), B, S, nxt.data_ptr(), 0)
            E[2].record(st)
            for _ in range(G - 1):
                he.he_decode_step(ctx, nxt.data_ptr(), nxt.data_ptr(), 0)
            E[3].record(st)
            he.he_unfuse_lora(ctx, lt)
            E[4].record(st)
            he.he_sync(ctx)
            torch.cuda.synchronize()
        t_fuse, t_pre, t_dec, t_unf = (E[i].elapsed_time(E[i + 1]) / 1e3 for i in range(4))
        res["phases"] = {
            "fuse_ms": t_fuse * 1e3, "prefill_ms": t_pre * 1e3, "decode_ms": t_dec * 1e3,
            "unfuse_ms": t_unf * 1e3, "retake_ms": t_retake * 1e3,
            "gen_tokens_per_s": B * G / (t_pre + t_dec),
            "prefill_tokens_per_s": B * S / t_pre,
            "decode_tokens_per_s": B * (G - 1) / t_dec,
            "decode_hbm_GBps": dec_bytes / t_dec / 1e9,
            "decode_hbm_frac": dec_bytes / t_dec / HBM_PEAK,
            "prefill_TFLOPs": pre_flops / t_pre / 1e12,
            "prefill_mfma_frac": pre_flops / t_pre / BF16_PEAK,
            "decode_bytes_per_step_avg": dec_bytes / (G - 1),
        }
        log(f"phases: {json.dumps(res['phases'])}")

        # per-kernel-class device time from HIP events on the library's stream
        classes = {"attn_decode": he.HE_K_ATTN_DECODE, "gemv_decode": he.HE_K_GEMV_DECODE,
                   "lmhead": he.HE_K_LMHEAD, "gemm_prefill": he.HE_K_GEMM_PREFILL,
                   "attn_prefill": he.HE_K_ATTN_PREFILL, "embed_norm": he.HE_K_EMBED_NORM,
                   "lora": he.HE_K_LORA}
        with torch.cuda.stream(st):
            for k in classes.values():
                he.he_kernel_timer(ctx, k, True)
            step()
            he.he_sync(ctx)
            stats = {n: he.he_kernel_stats(ctx, k) for n, k in classes.items()}
            for k in classes.values():
                he.he_kernel_timer(ctx, k, False)
        kern = {}
        for n, s in stats.items():
            if s.launches:
                kern[n] = {"launches": s.launches, "avg_us": s.total_ms / s.launches * 1e3,
                           "total_ms": s.total_ms,
                           "GBps": s.bytes / (s.total_ms / 1e3) / 1e9 if s.total_ms else None,
                           "TFLOPs": s.flops / (s.total_ms / 1e3) / 1e12 if s.total_ms else None}
        res["kernels"] = kern
        dec_classes = {"attn_decode": "hbm", "gemv_decode": "hbm"}
        dom = max(dec_classes, key=lambda n: stats[n].total_ms)
        s = stats[dom]
        avg_s = s.total_ms / s.launches / 1e3
        per_launch = s.bytes / s.launches
        traffic, traffic_src = None, None
        cpath = os.path.join(PROFILES, f"counters_decode_{args.workload}_b{B}.json")
        if os.path.exists(cpath):
            summ = json.load(open(cpath))
            if summ.get("sources_sha") == sources_sha() and dom in summ.get("classes", {}):
                traffic = summ["classes"][dom]["traffic_bytes_per_dispatch"]
                traffic_src = os.path.relpath(cpath, ROOT)
        res["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": per_launch / avg_s / 1e9,
                           "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                           "frac": per_launch / avg_s / HBM_PEAK, "traffic": traffic,
                           "traffic_source": traffic_src,
                           "bytes_per_launch": per_launch, "avg_launch_us": avg_s * 1e6,
                           "launches": s.launches}
        log(f"roofline: {json.dumps(res['roofline'])}")

        if not args.no_extras:
            # sampled generation (temperature 0.7, Gumbel-max with Philox4x64-10) with per-token
            # log-probabilities, same shape and fused weights: whole-generation time beside the
            # greedy one, and the LM head's time per launch in each mode
            with torch.cuda.stream(st):
                lpb = torch.empty(B, G, dtype=torch.float32, device="cuda")
                smp = he.he_sampling(0.7, 1234)
                E = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                he.he_fuse_lora(ctx, lt)
                he.he_generate_ex(ctx, prompts.data_ptr(), B, S, G, smp, out.data_ptr(), lpb.data_ptr())  # graph capture
                E[0].record(st)
                he.he_generate_ex(ctx, prompts.data_ptr(), B, S, G, smp, out.data_ptr(), lpb.data_ptr())
                E[1].record(st)
                # the same with a top-p 0.9 nucleus (graph captured by the first call)
                smp_p = he.he_sampling(0.7, 1234, 0.9)
                Ep = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                he.he_generate_ex(ctx, prompts.data_ptr(), B, S, G, smp_p, out.data_ptr(), lpb.data_ptr())
                Ep[0].record(st)
                he.he_generate_ex(ctx, prompts.data_ptr(), B, S, G, smp_p, out.data_ptr(), lpb.data_ptr())
                Ep[1].record(st)
                he.he_kernel_timer(ctx, he.HE_K_LMHEAD, True)
                he.he_generate_ex(ctx, prompts.data_ptr(), B, S, 8, smp, out.data_ptr(), lpb.data_ptr())
                lm_s = he.he_kernel_stats(ctx, he.HE_K_LMHEAD)
                he.he_kernel_timer(ctx, he.HE_K_LMHEAD, False)
                he.he_unfuse_lora(ctx, lt)
                he.he_sync(ctx)
                torch.cuda.synchronize()
            t_smp = E[0].elapsed_time(E[1]) / 1e3
            t_topp = Ep[0].elapsed_time(Ep[1]) / 1e3
            lps = lpb.cpu().numpy()
            res["sampled"] = {
                "temperature": 0.7, "gen_ms": t_smp * 1e3, "gen_tokens_per_s": B * G / t_smp,
                "vs_greedy_gen": (t_pre + t_dec) / t_smp,
                "top_p_0.9_gen_ms": t_topp * 1e3, "top_p_vs_greedy_gen": (t_pre + t_dec) / t_topp,
                "lmhead_us_sampled_logprobs": lm_s.total_ms / lm_s.launches * 1e3 if lm_s.launches else None,
                "lmhead_us_greedy": kern["lmhead"]["avg_us"] if "lmhead" in kern else None,
                "mean_logprob": float(lps.mean()), "logprobs_finite": bool((lps == lps).all())}
            log(f"sampled: {json.dumps(res['sampled'])}")

            # weight-only FP8 decode (a separate mode: E4M3 projection weights, half the
            # weight bytes per step): greedy generation beside the bf16 one, and the decode
            # GEMVs' time per launch with their algorithmic (one byte per weight) traffic
            with torch.cuda.stream(st):
                he.he_fuse_lora(ctx, lt)
                he.he_set_fp8_decode(ctx, True)
                Ef = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                he.he_generate(ctx, prompts.data_ptr(), B, S, G, out.data_ptr())     # graph capture
                Ef[0].record(st)
                he.he_generate(ctx, prompts.data_ptr(), B, S, G, out.data_ptr())
                Ef[1].record(st)
                he.he_kernel_timer(ctx, he.HE_K_GEMV_DECODE, True)
                he.he_generate(ctx, prompts.data_ptr(), B, S, 8, out.data_ptr())
                gv8 = he.he_kernel_stats(ctx, he.HE_K_GEMV_DECODE)
                he.he_kernel_timer(ctx, he.HE_K_GEMV_DECODE, False)
                he.he_set_fp8_decode(ctx, False)
                he.he_unfuse_lora(ctx, lt)
                he.he_sync(ctx)
                torch.cuda.synchronize()
            t_f8 = Ef[0].elapsed_time(Ef[1]) / 1e3
            L_, d_, F_ = a.n_layers, a.d_model, a.d_ffn
            w_bf16 = L_ * (4 * d_ * d_ + 2 * d_ * F_) * 2
            w_f8 = L_ * ((4 * d_ * d_ + 2 * d_ * F_) + 4 * (5 * d_ + F_))     # codes + per-row scales
            f8_step_bytes = dec_bytes / (G - 1) - w_bf16 + w_f8
            res["fp8_decode"] = {
                "gen_ms": t_f8 * 1e3, "gen_tokens_per_s": B * G / t_f8, "vs_bf16_gen": (t_pre + t_dec) / t_f8,
                "decode_ms_est": t_f8 * 1e3 - t_pre * 1e3,
                "decode_bytes_per_step_avg": f8_step_bytes,
                "decode_hbm_GBps_est": f8_step_bytes * (G - 1) / (t_f8 - t_pre) / 1e9,
                "gemv_avg_us": gv8.total_ms / gv8.launches * 1e3 if gv8.launches else None,
                "gemv_GBps": gv8.bytes / (gv8.total_ms / 1e3) / 1e9 if gv8.total_ms else None}
            log(f"fp8_decode: {json.dumps(res['fp8_decode'])}")

            # teacher-forced scoring of the finished experience (prompt + the answer just
            # sampled, S + G tokens): log-probabilities of the B x G answer tokens, fused weights
            with torch.cuda.stream(st):
                seq = torch.cat([prompts, out], dim=1).contiguous()
                lpt = torch.empty(B, G, dtype=torch.float32, device="cuda")
                E = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                he.he_fuse_lora(ctx, lt)
                he.he_logprobs(ctx, seq.data_ptr(), B, S + G, S, lpt.data_ptr())
                E[0].record(st)
                for _ in range(2):
                    he.he_logprobs(ctx, seq.data_ptr(), B, S + G, S, lpt.data_ptr())
                E[1].record(st)
                cls = {"gemm": he.HE_K_GEMM_PREFILL, "attn": he.HE_K_ATTN_PREFILL, "vocab": he.HE_K_VOCAB}
                for k in cls.values():
                    he.he_kernel_timer(ctx, k, True)
                he.he_logprobs(ctx, seq.data_ptr(), B, S + G, S, lpt.data_ptr())
                cs = {n: he.he_kernel_stats(ctx, k) for n, k in cls.items()}
                for k in cls.values():
                    he.he_kernel_timer(ctx, k, False)
                he.he_unfuse_lora(ctx, lt)
                he.he_sync(ctx)
                torch.cuda.synchronize()
            t_sc = E[0].elapsed_time(E[1]) / 1e3 / 2
            T = S + G
            L, d, F, V = a.n_layers, a.d_model, a.d_ffn, a.vocab
            sc_flops = (2.0 * B * T * L * (4 * d * d + 2 * d * F) + 2.0 * L * d * T * (T + 1) * B
                        + 2.0 * B * G * d * V)
            lpv = lpt.cpu().numpy()
            tf = lambda st_: st_.flops / (st_.total_ms / 1e3) / 1e12 if st_.total_ms else None
            res["scoring"] = {
                "sequence": T, "prompt_len": S, "answer_len": G, "ms": t_sc * 1e3,
                "scored_tokens_per_s": B * G / t_sc, "TFLOPs": sc_flops / t_sc / 1e12,
                "mfma_frac": sc_flops / t_sc / BF16_PEAK,
                "layer_gemm_ms": cs["gemm"].total_ms, "layer_gemm_TFLOPs": tf(cs["gemm"]),
                "attn_ms": cs["attn"].total_ms,
                "vocab_ms": cs["vocab"].total_ms, "vocab_TFLOPs": tf(cs["vocab"]),
                "mean_logprob": float(lpv.mean()), "logprobs_finite": bool(((lpv == lpv) & (abs(lpv) < float("inf"))).all())}
            log(f"scoring: {json.dumps(res['scoring'])}")

    with torch.cuda.stream(st):
        he.he_release_cache(ctx)
        he.he_sync(ctx)
    eng.close()

    if wl.rounds == 2 and not args.no_breakdown:
        res["sequence"] = two_round_sequence(wl, a, dev, ldev, prompts, args.seed)
        log(f"sequence: {json.dumps(res['sequence'])}")

    if not args.no_breakdown and not args.no_graph and not args.no_extras:
        # the same decode phase launched directly (no hipGraph replay), for the graph gain
        eng2 = he.Engine(a, dev, use_graph=False)
        ctx2, st2 = eng2.ctx, eng2.stream
        lt2, _keep2 = eng2.lora(ldev, wl.lora_rank, wl.lora_alpha)
        with torch.cuda.stream(st2):
            he.he_retake_cache(ctx2, B, wl.max_seq)
            he.he_fuse_lora(ctx2, lt2)
            nxt = torch.empty(B, dtype=torch.int32, device="cuda")
            E = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            he.he_prefill(ctx2, prompts.data_ptr(), B, S, nxt.data_ptr(), 0)
            E[0].record(st2)
            for _ in range(G - 1):
                he.he_decode_step(ctx2, nxt.data_ptr(), nxt.data_ptr(), 0)
            E[1].record(st2)
            he.he_unfuse_lora(ctx2, lt2)
            he.he_release_cache(ctx2)
            he.he_sync(ctx2)
            torch.cuda.synchronize()
        eng2.close()
        t_dec_direct = E[0].elapsed_time(E[1]) / 1e3
        res["phases"]["decode_ms_no_graph"] = t_dec_direct * 1e3
        res["phases"]["graph_speedup"] = t_dec_direct / (res["phases"]["decode_ms"] / 1e3)
        log(f"decode without graph: {t_dec_direct * 1e3:.1f} ms (graph gain x{res['phases']['graph_speedup']:.3f})")

    if not args.no_breakdown and not args.no_extras:
        # reward scoring (the largest workload's OPT-350m-shape reward model, post-LN, its own
        # shape): 128 sequences x 512 tokens, one full causal pass plus the scalar head
        rw = synth.WORKLOADS["opt13b"]
        rs = rw.reward
        RB, RS = rw.batch, rw.max_seq
        rdev = {k: v.cuda() for k, v in synth.model_params(rs, args.seed).items()}
        rids = synth.tokens(args.seed, "reward_ids", (RB, RS), rs.vocab).cuda()
        reward = torch.empty(RB, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        eng3 = he.Engine(rs, rdev)
        with torch.cuda.stream(eng3.stream):
            he.he_retake_cache(eng3.ctx, RB, RS)
            he.he_score(eng3.ctx, rids.data_ptr(), RB, RS, reward.data_ptr())      # warm-up
            E = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            E[0].record(eng3.stream)
            for _ in range(3):
                he.he_score(eng3.ctx, rids.data_ptr(), RB, RS, reward.data_ptr())
            E[1].record(eng3.stream)
            rcls = {"gemm": he.HE_K_GEMM_PREFILL, "attn": he.HE_K_ATTN_PREFILL, "norm": he.HE_K_EMBED_NORM,
                    "head": he.HE_K_SCORE}
            for k in rcls.values():
                he.he_kernel_timer(eng3.ctx, k, True)
            he.he_score(eng3.ctx, rids.data_ptr(), RB, RS, reward.data_ptr())
            rst = {n: he.he_kernel_stats(eng3.ctx, k) for n, k in rcls.items()}
            for k in rcls.values():
                he.he_kernel_timer(eng3.ctx, k, False)
            he.he_release_cache(eng3.ctx)
            he.he_sync(eng3.ctx)
            torch.cuda.synchronize()
        eng3.close()
        t_rm = E[0].elapsed_time(E[1]) / 1e3 / 3
        de, dr, Lr, Fr = rs.embed_dim, rs.d_model, rs.n_layers, rs.d_ffn
        rm_flops = (2.0 * RB * RS * (Lr * (4 * dr * dr + 2 * dr * Fr) + de * dr)   # layers + project_in
                    + 2.0 * Lr * dr * RS * (RS + 1) * RB + 2.0 * RB * dr * de)
        res["reward_scoring"] = {
            "model": "opt-350m shape (post-LN, d 1024, 24 layers, embedding 512)", "batch": RB, "seq_len": RS,
            "ms": t_rm * 1e3, "sequences_per_s": RB / t_rm, "tokens_per_s": RB * RS / t_rm,
            "TFLOPs": rm_flops / t_rm / 1e12, "mfma_frac": rm_flops / t_rm / BF16_PEAK,
            "rewards_finite": bool(torch.isfinite(reward).all().item()),
            "class_ms": {n: v.total_ms for n, v in rst.items()},
            "gemm_TFLOPs": rst["gemm"].flops / (rst["gemm"].total_ms / 1e3) / 1e12 if rst["gemm"].total_ms else None}
        log(f"reward_scoring: {json.dumps(res['reward_scoring'])}")

    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.seed)
        log(f"cpu baseline: {res['cpu_baseline']['value']:.2f} tokens/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
