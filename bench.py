"""Benchmark of the LAGA per-rank attention block on one MI355X.

One step = the whole per-rank hot path on one batch of seeded synthetic input
already resident in HBM: latent RMSNorm -> head-shard up-projection -> causal
attention forward -> attention backward folded into dLatent / dW_kv_b / dgamma.
Workload: B=1, S=16384, 16 local heads (n_h=128 at SP=8, rank 0), DeepSeek-V3
head dims (d_kv=512, d_nope=d_v=128, d_rope=64), bf16 inputs, causal, with the
split-operand precision the training step needs for its parity bars.  The
forward alone is also timed with single fp16 operands (the forward-only
workload's setting), both unfused (norm, up-projection, attention) and fused
(laga_attn_fwd_fused); its headline figures are those of the faster path.

Prints one JSON line with tokens/s, algorithmic TFLOP/s, per-kernel times
(HIP events on the launch stream), the roofline of the dominant kernel, the
fp64 oracle timed on a bounded sample on the host cores, the forward alone at
the other DeepSeek-V3 workloads (S=4096 with 16 local heads, and S=4096 with
all 128 heads on one device), the absorbed form (B2) forward and backward on
the step's inputs with its own FLOPs, and memory: analytic activation bytes of LAGA
against the explicit and absorbed forms, the backward workspace, and the peak
that torch's allocator records over one training step.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "v3_sp8_s16384_h16_train"
METRIC = "MLA attention-block tokens/s and TFLOP/s (fwd, fwd+bwd) vs bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FP16, SPLIT = 0, 1


def alg_flops(d) -> dict:
    """Algorithmic FLOPs: causal pairs only, no recompute, no hi/lo extra passes."""
    pairs = d.S * (d.S + 1) / 2
    attn_fwd = 2 * pairs * (d.d_qk + d.d_v) * d.h * d.B
    kv_up = 2 * d.B * d.S * d.d_kv * d.h * (d.d_nope + d.d_v)
    # The backward's products dP, dV, dK, dq counted once each (no recompute of S):
    # the dK/dV kernel owns dP, dV, dK and the dq kernel owns dq.
    bwd_dkdv = 2 * pairs * (2 * d.d_v + d.d_qk) * d.h * d.B
    bwd_dq = 2 * pairs * d.d_qk * d.h * d.B
    return dict(attn_fwd=attn_fwd, attn_bwd=2 * attn_fwd, bwd_dkdv=bwd_dkdv, bwd_dq=bwd_dq, kv_up=kv_up,
                fold=2 * kv_up, fwd=attn_fwd + kv_up, step=3 * attn_fwd + 3 * kv_up)


def absorbed_flops(d) -> float:
    """The absorbed form's (B2) own forward FLOPs: absorb GEMM, latent attention (score
    width d_kv + d_rope, value width d_kv, causal pairs only), un-absorb GEMM."""
    pairs = d.S * (d.S + 1) / 2
    T = d.B * d.S
    return (2 * T * d.h * d.d_nope * d.d_kv + 2 * pairs * (2 * d.d_kv + d.d_rope) * d.h * d.B
            + 2 * T * d.h * d.d_kv * d.d_v)


def absorbed_bwd_flops(d) -> float:
    """The absorbed form's (B2) own backward FLOPs, each product once (no recompute of the
    scores, P or acc): per causal pair dP = d_acc L^T and dL += P^T d_acc (width d_kv),
    d_q_abs || dq_rope = dS (L || k_pe) and dL || dk_pe += dS^T q (width d_kv + d_rope);
    per token and head d_acc = dO W^v, dq_nope = d_q_abs W^k^T, dW^k and dW^v."""
    pairs = d.S * (d.S + 1) / 2
    T = d.B * d.S
    return (2 * pairs * (4 * d.d_kv + 2 * d.d_rope) * d.h * d.B
            + 2 * T * d.h * d.d_kv * (2 * d.d_v + 2 * d.d_nope))


def activation_bytes(d, kv_bytes: int) -> dict:
    """Bytes one rank keeps for the backward: LAGA vs the explicit (B1) and absorbed (B2) forms."""
    T, h = d.B * d.S, d.h
    common = T * h * d.d_qk * 2 + T * h * d.d_v * 4 + T * h * 4        # q (bf16), o (fp32), lse
    laga = common + T * d.d_kv * 2 + T * d.d_rope * 2 + T * 4 + T * h * (d.d_nope + d.d_v) * kv_bytes
    explicit = common + T * h * (d.d_qk + d.d_v) * kv_bytes             # per-head K (incl. rope band) and V
    absorbed = common + T * d.d_kv * 2 + T * d.d_rope * 2 + T * 4 + 2 * T * h * d.d_kv * kv_bytes
    return dict(laga=laga, explicit=explicit, absorbed=absorbed)


def source_digest(rel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def kernel_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a plain copy), or None
    when no counters were taken or the kernel's source changed since they were."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(kernel)
    if not rec or source_digest(rec["source"]) != rec["source_sha256"]:
        return None
    return rec["bytes_per_launch"]


def calibration_copy(nbytes: int = 256 << 20, reps: int = 3):
    """A plain device copy of known size: the reference point that scales the HBM byte
    counters of the other kernels in a counter-collection run."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# ------------------------------------------------------------ profile summaries
# Bench stage -> (alternatives, each a list of substrings that must all appear in the
# profiler's kernel name: demangled, or mangled where the profiler could not demangle it;
# source file).
_N = "head_latent_attention_laga_amd/csrc/"
PROFILE_KERNELS = {
    "rmsnorm_fwd": ([["rmsnorm_fwd_kernel"]], _N + "norm.hip"),
    "kv_up": ([["gemm_dma_kernel", "EpiKvUp<_Float16, 2"], ["gemm_dma_kernel", "EpiKvUpIDF16_Li2E"]], _N + "gemm.hip"),
    "kv_up_fp16": ([["gemm_dma_kernel", "EpiKvUp<_Float16, 1"], ["gemm_dma_kernel", "EpiKvUpIDF16_Li1E"]],
                   _N + "gemm.hip"),
    "attn_fwd": ([["attn_fwd_kernel<", "MmaBf16, 2, 128"]], _N + "attn_fwd.hip"),
    "attn_fwd_fp16": ([["attn_fwd_kernel<", "MmaBf16, 1, 128"]], _N + "attn_fwd.hip"),
    "fused_prep": ([["fused_prep_kernel"]], _N + "attn_fwd.hip"),
    "attn_fwd_fused": ([["attn_fwd_fused_kernel"]], _N + "attn_fwd.hip"),
    "fused_merge": ([["fused_merge_kernel"]], _N + "attn_fwd.hip"),
    "bwd_delta": ([["bwd_prep_kernel"]], _N + "attn_bwd.hip"),
    "do_convert": ([["do_convert_kernel"]], _N + "attn_bwd.hip"),
    "attn_bwd_dkdv": ([["dkdv_kernel<"], ["dkdv_kernelIDF16_NS_6MmaF16ELi2"]], _N + "attn_bwd.hip"),
    "attn_bwd_dq": ([["dq_kernel<"]], _N + "attn_bwd_dq.hip"),
    "fold_dL": ([["gemm_dma_kernel<", "DKC<2, unsigned short, 64"]], _N + "gemm.hip"),
    "fold_dW": ([["gemm_dma_kernel<", "DRC<2, 128>, laga::(anonymous namespace)::DRC<2, 128>", "EpiStore"]],
                _N + "gemm.hip"),
    "rmsnorm_bwd": ([["rmsnorm_bwd_kernel"]], _N + "norm.hip"),
    "absorb_q": ([["gemm_dma_kernel<", "EpiHalf"]], _N + "gemm.hip"),
    "absorbed_attn": ([["absorbed_attn_kernel"]], _N + "absorbed.hip"),
    # o = acc W^v in the forward and dq_nope = d_q_abs W^k^T in the backward: one kernel at one shape.
    "unabsorb_o": ([["gemm_dma_kernel<", "DKC<1, float, 256, false"]], _N + "gemm.hip"),
    "b2_planes": ([["gemm_dma_kernel<", "EpiPlanes"]], _N + "gemm.hip"),
    "b2_scores": ([["gemm_dma_kernel<", "DKC<2, unsigned short, 128, false>, laga::(anonymous namespace)::DKC<2"]],
                  _N + "gemm.hip"),
    "b2_rowstat": ([["b2_rowstat_kernel"]], _N + "absorbed.hip"),
    "b2_pds": ([["b2_pds_kernel"]], _N + "absorbed.hip"),
    "b2_rows_by_keys": ([["gemm_dma_kernel<", "DKC<2, unsigned short, 128, false>, laga::(anonymous namespace)::DRC<2"]],
                        _N + "gemm.hip"),
    "b2_key_grads": ([["gemm_dma_kernel<", "DRC<2, 128>, laga::(anonymous namespace)::DRC<2, 128>", "EpiAccum"],
                      ["gemm_dma_kernel<", "DRC<2, 128>, laga::(anonymous namespace)::DRC<2, 128>", "EpiPart"]],
                     _N + "gemm.hip"),
    "b2_dw": ([["gemm_dma_kernel<", "DRC<1, 128>, laga::(anonymous namespace)::DRC<2, 128>"]], _N + "gemm.hip"),
}
# Kernels of the forward-only path run once per forward-only workload; their grid
# (work-items) tells the workloads apart.
FWD_ONLY_GRIDS = {
    "kv_up_fp16": {524288: "S=16384 h=16", 131072: "S=4096 h=16", 1048576: "S=4096 h=128"},
    "attn_fwd_fp16": {524288: "S=16384 h=16", 131072: "S=4096 h=16", 1048576: "S=4096 h=128"},
    "attn_fwd_fused": {1048576: "S=16384 h=16", 327680: "S=4096 h=16", 2097152: "S=4096 h=128"},
    "fused_prep": {2359552: "S=16384 h=16", 524544: "S=4096 h=16", 1310976: "S=4096 h=128"},
    "rmsnorm_fwd": {1048576: "S=16384", 262144: "S=4096"},
}


# $REPO: the repository root (absolute: the profiler runs from /tmp); $OUT: the directory
# whose rocprofv3 output the summaries are made from (`--summarize-profiles $OUT`).
PROFILE_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 {opts} --output-format csv "
               "-d $OUT/{d} -o {o} -- python3 $REPO/bench.py {args}")
PROFILE_VARS = ("`$REPO` is the repository root and `$OUT` the directory these summaries were made from "
                "(`python bench.py --summarize-profiles $OUT`).")
PMC_ARGS = "--steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy"
KT_ARGS = "--steps 10 --warmup 5 --no-cpu-baseline"
COUNTER_PASSES = {
    "pmc_a": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
             "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "pmc_b": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_SALU "
             "SQ_WAVES GRBM_GUI_ACTIVE",
}


def profile_stage(kernel_name: str):
    for stage, (alts, _) in PROFILE_KERNELS.items():
        if any(all(x in kernel_name for x in subs) for subs in alts):
            return stage
    return None


def stage_label(stage: str, grid: int) -> str:
    w = FWD_ONLY_GRIDS.get(stage, {}).get(grid)
    return f"{stage} ({w})" if w else stage


def read_counters(path: str):
    """Per stage label: per dispatch {counter: value} with the dispatch's duration in ns."""
    import csv
    import collections
    disp = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        disp[key][r["Counter_Name"]] = float(r["Counter_Value"])
        disp[key]["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        disp[key]["_grid"] = int(r["Grid_Size"])
    per = collections.defaultdict(list)
    copies = []
    stages = {}
    for (name, _), c in disp.items():
        if name == "__amd_rocclr_copyBuffer" and c["_grid"] == 131072:
            copies.append(c)
        if name not in stages:
            stages[name] = profile_stage(name)
        if stages[name]:
            per[stage_label(stages[name], c["_grid"])].append(c)
    return per, copies


def label_order(per) -> list:
    order = {st: i for i, st in enumerate(PROFILE_KERNELS)}
    return sorted(per, key=lambda lb: (order[lb.split(" (")[0]], lb))


def summarize_profiles(out_root: str):
    """Writes profiles/*.md and profiles/traffic.json from the rocprofv3 csv output of
    the commands named in each summary (kt: kernel trace, pmc_fetch / pmc_write: HBM
    bytes, pmc_a / pmc_b: instruction and cycle counters), plus bench.json, the JSON
    line of an unprofiled `python bench.py` on the same box."""
    import csv
    import hashlib
    prof = os.path.join(ROOT, "profiles")
    title = "B=1 S=16384 h=16 (n_h=128, SP=8), V3 dims, bf16 inputs"

    # Kernel trace: per dispatch, grouped by stage and workload.
    import collections
    disp = collections.defaultdict(list)
    stages = {}
    for r in csv.DictReader(open(os.path.join(out_root, "kt", "kt_kernel_trace.csv"))):
        nm = r["Kernel_Name"]
        if nm not in stages:
            stages[nm] = profile_stage(nm)
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        lb = stage_label(stages[nm], grid) if stages[nm] else nm.replace("laga::(anonymous namespace)::", "")[:60]
        disp[lb].append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    # The bench line that the profiled run itself printed (kt.log), and its timed launches:
    # each step kernel runs `warmup` times, then `steps` timed times, then once more
    # for the step's memory measurement.
    line = [ln for ln in open(os.path.join(out_root, "kt.log")) if ln.startswith('{"metric"')]
    prun = json.loads(line[-1]) if line else None
    L = [f"# Kernel trace: LAGA training step, fp16-operand forward (unfused and fused) and absorbed-form (B2) "
         f"forward and backward, {title}", "", "Command (on the MI355X):", "", "```",
         PROFILE_CMD.format(opts="--kernel-trace --stats", d="kt", o="kt", args=KT_ARGS), "```", "", PROFILE_VARS, "",
         "Per launch, from the trace (`kt_kernel_trace.csv`), in us. For the step's kernels, 'timed' is the mean "
         "over the launches inside bench.py's timed region and 'bench' the HIP-event mean that the same run "
         "printed in its JSON line.", "",
         "| stage | launches | mean | median | min | max | timed | bench |", "|---|---|---|---|---|---|---|---|"]
    order = {st: i for i, st in enumerate(PROFILE_KERNELS)}
    for lb in sorted(disp, key=lambda x: (order.get(x.split(" (")[0], 99), x)):
        v = [d for _, d in sorted(disp[lb])]
        timed = bench_ms = ""
        if prun and lb in prun["kernels_ms"]:
            w, k = prun["warmup"], prun["steps"]
            if len(v) >= w + k:
                timed = f"{statistics.mean(v[w:w + k]):.1f}"
            bench_ms = f"{prun['kernels_ms'][lb] * 1e3:.1f}"
        L.append(f"| {lb} | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | {min(v):.1f} | "
                 f"{max(v):.1f} | {timed} | {bench_ms} |")
    bench = json.loads(open(os.path.join(out_root, "bench.json")).read().strip().splitlines()[-1])
    L += ["", "The profiled run's own JSON line (roofline and step):", "", "```",
          json.dumps({k: prun[k] for k in ("ms_per_step", "value", "tflops_step", "roofline")}) if prun else "none",
          "```", "", "An unprofiled `python bench.py --no-cpu-baseline` on the same box:", "", "```",
          "step kernels (ms): " + json.dumps(bench["kernels_ms"]),
          "forward fp16: " + json.dumps(bench["forward_fp16_operands"]),
          "absorbed form: " + json.dumps(bench.get("absorbed_form")),
          f"step {bench['ms_per_step']} ms, {bench['value']} tokens/s, {bench['tflops_step']} TFLOP/s; "
          f"roofline {json.dumps(bench['roofline'])}", "```", ""]
    open(os.path.join(prof, "step_v3_s16384_h16_kernel_trace.md"), "w").write("\n".join(L))

    # HBM bytes: FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on the copies.
    fe, cf = read_counters(os.path.join(out_root, "pmc_fetch", "pmc_counter_collection.csv"))
    wr, cw = read_counters(os.path.join(out_root, "pmc_write", "pmc_counter_collection.csv"))
    copy_kib = 256 * 1024
    sf = copy_kib / statistics.mean(c["FETCH_SIZE"] for c in cf)
    sw = copy_kib / statistics.mean(c["WRITE_SIZE"] for c in cw)
    L = [f"# HBM traffic per kernel launch: {title}", "",
         "Two counter passes (FETCH_SIZE, then WRITE_SIZE), each on its own run:", "", "```",
         PROFILE_CMD.format(opts="--pmc FETCH_SIZE", d="pmc_fetch", o="pmc", args=PMC_ARGS),
         PROFILE_CMD.format(opts="--pmc WRITE_SIZE", d="pmc_write", o="pmc", args=PMC_ARGS), "```", "", PROFILE_VARS, "",
         f"Calibration: `--calibrate-copy` first runs three 256 MiB device copies (`__amd_rocclr_copyBuffer`); per "
         f"copy FETCH_SIZE read {copy_kib / sf:.1f} KiB and WRITE_SIZE {copy_kib / sw:.1f} KiB against {copy_kib} KiB "
         f"moved each way, so the scale factors are fetch x{sf:.4f}, write x{sw:.4f}. GB/s divides the scaled bytes "
         f"by the dispatch's duration in the same (counter-collecting) run.", "",
         "| stage | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB per launch (read + write) | GB/s |",
         "|---|---|---|---|---|---|"]
    js = {"copy_scale": {"fetch": sf, "write": sw}, "kernels": {}}
    for st in label_order(fe):
        if st not in wr:
            continue
        src = PROFILE_KERNELS[st.split(" (")[0]][1]
        f = statistics.mean(c["FETCH_SIZE"] for c in fe[st])
        w = statistics.mean(c["WRITE_SIZE"] for c in wr[st])
        ns = statistics.mean([c["_ns"] for c in fe[st]] + [c["_ns"] for c in wr[st]])
        b = (f * sf + w * sw) * 1024
        L.append(f"| {st} | {len(fe[st])} | {f:.1f} | {w:.1f} | {f * sf * 1024 / 1e6:.1f} + {w * sw * 1024 / 1e6:.1f} = "
                 f"{b / 1e6:.1f} | {b / ns:.0f} |")
        js["kernels"][st] = {"bytes_per_launch": round(b), "fetch_kib": f, "write_kib": w, "source": src,
                             "source_sha256": source_digest(src)}
    open(os.path.join(prof, "hbm_traffic_v3_s16384_h16.md"), "w").write("\n".join(L) + "\n")
    with open(os.path.join(prof, "traffic.json"), "w") as fh:
        json.dump(js, fh, indent=1)

    # Instruction and cycle counters.
    pa, _ = read_counters(os.path.join(out_root, "pmc_a", "pmc_counter_collection.csv"))
    pb, _ = read_counters(os.path.join(out_root, "pmc_b", "pmc_counter_collection.csv"))
    L = [f"# Instruction and cycle counters per kernel launch: {title}", "",
         "Two passes, each on its own run:", "", "```"]
    for d, cs in COUNTER_PASSES.items():
        L.append(PROFILE_CMD.format(opts=f"--pmc {cs}", d=d, o="pmc", args=PMC_ARGS))
    L += ["```", "", PROFILE_VARS, "",
          "Columns (means over the launches): MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
          "SIMDs), the share of SIMD cycles the matrix cores were busy; clock = GRBM_GUI_ACTIVE / 8 / duration; "
          "VALU, LDS and any-instruction active and the wait shares are per wave cycle (SQ_ACTIVE_INST_*, "
          "SQ_WAIT_ANY, SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES); instruction counts are per launch (G = 1e9); "
          "bank conflicts = SQ_LDS_BANK_CONFLICT cycles, with their share of SQ_LDS_IDX_ACTIVE. Durations are "
          "those of the counter-collecting run; the clock is left out for launches under 100 us, where the "
          "counter's window is not the kernel's. Kernels without a workload in parentheses belong to the "
          "training step (S=16384, h=16) or the absorbed form's forward at that shape.", "",
          "| stage | launches | us | clock GHz | MFMA busy | MFMA insts | VALU insts | LDS insts | VALU active | "
          "LDS active | waits (any) | waits (instr.) | bank-conflict cycles |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for st in label_order(pa):
        if st not in pb:
            continue
        a = {k: statistics.mean(c[k] for c in pa[st]) for k in pa[st][0]}
        bb = {k: statistics.mean(c[k] for c in pb[st]) for k in pb[st][0]}
        cyc = a["GRBM_GUI_ACTIVE"] / 8
        wc = a["SQ_WAVE_CYCLES"]
        lds_conf = bb["SQ_LDS_BANK_CONFLICT"]
        lds_act = bb["SQ_LDS_IDX_ACTIVE"]
        clock = f"{cyc / a['_ns']:.2f}" if a["_ns"] > 1e5 else "-"
        L.append(f"| {st} | {len(pa[st])} | {a['_ns'] / 1e3:.1f} | {clock} | "
                 f"{100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1f}% | {bb['SQ_INSTS_MFMA'] / 1e9:.3f} G | "
                 f"{bb['SQ_INSTS_VALU'] / 1e9:.3f} G | {bb['SQ_INSTS_LDS'] / 1e9:.3f} G | "
                 f"{100 * a['SQ_ACTIVE_INST_VALU'] / wc:.1f}% | {100 * a['SQ_ACTIVE_INST_LDS'] / wc:.1f}% | "
                 f"{100 * a['SQ_WAIT_ANY'] / wc:.1f}% | {100 * a['SQ_WAIT_INST_ANY'] / wc:.1f}% | "
                 f"{lds_conf:.3g} ({100 * lds_conf / lds_act if lds_act else 0:.1f}%) |")
    open(os.path.join(prof, "counters_v3_s16384_h16.md"), "w").write("\n".join(L) + "\n")


def host_info() -> dict:
    """CPU model, logical CPU count and the BLAS numpy's oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = {"name": libs[0].get("internal_api"), "version": libs[0].get("version"),
                    "threads": libs[0].get("num_threads")}
    except Exception:  # noqa: BLE001 - informational only
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas": blas}


def cpu_baseline(d) -> dict:
    """The fp64 oracle, untuned, on 4 of the workload's heads (n_h=128 at SP=32, rank 0):
    norm, up-projection of those heads, causal attention forward and backward, and the
    folds, at the full S.  Tokens/s is scaled to the workload's head count."""
    import laga_inputs as li
    import oracle
    sample_heads = 4
    one = li.Dims(B=d.B, S=d.S, n_h=d.n_h, sp_size=d.n_h // sample_heads, sp_rank=0, d_kv=d.d_kv, d_nope=d.d_nope,
                  d_rope=d.d_rope, d_v=d.d_v, dtype=d.dtype)
    inp = li.make_inputs(one, 0, backward=True)
    v = {k: t.value for k, t in inp.items()}
    kw = dict(n_h=one.n_h, sp_size=one.sp_size, sp_rank=0, d_nope=one.d_nope, eps=one.eps)
    t0 = time.perf_counter()
    f = oracle.forward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], **kw)
    oracle.backward(v["q"], v["latent"], v["k_pe"], v["w_kv_b"], v["gamma"], v["d_o"], fwd=f, **kw)
    dt = time.perf_counter() - t0
    info = host_info()
    threads = (info["blas"] or {}).get("threads") or 1
    return {"value": d.B * d.S * sample_heads / (dt * d.h), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd of {sample_heads} of the {d.h} heads at full S={d.S} "
                      f"({dt:.1f} s), scaled by {sample_heads}/{d.h}",
            **info}


def time_fused(p, x, steps: int, warmup: int) -> float:
    """Mean ms of one laga_attn_fwd_fused call (its prep and fused kernels), HIP
    events around each call on the launch stream."""
    import torch
    out = p.alloc_fused()
    for _ in range(warmup):
        p.forward_fused(x, out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        p.forward_fused(x, out)
        ev[i][1].record()
    torch.cuda.synchronize()
    err = int(out["workspace"][32:36].view(torch.int32).item())
    if err != 0:
        raise RuntimeError("laga_attn_fwd_fused reported a consumer that gave up waiting")
    del out
    return statistics.mean(ev[i][0].elapsed_time(ev[i][1]) for i in range(steps))


def forward_summary(d, ks: dict, fused_ms: float) -> dict:
    """The forward-only line: the unfused path (norm, kv_up, attention: per-kernel
    times) next to the fused one; the headline figures are those of the faster."""
    fl = alg_flops(d)
    unfused_ms = sum(ks.values())
    best = "fused" if fused_ms < unfused_ms else "unfused"
    ms = min(fused_ms, unfused_ms)
    return {"path": best, "ms": round(ms, 4), "tokens_s": round(d.B * d.S / (ms / 1e3), 1),
            "tflops": round(fl["fwd"] / (ms / 1e3) / 1e12, 2),
            "frac_peak": round(fl["fwd"] / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fused_ms": round(fused_ms, 4), "unfused_ms": round(unfused_ms, 4),
            "unfused_kv_up_tflops": round(fl["kv_up"] / (ks["kv_up"] / 1e3) / 1e12, 2),
            "unfused_attn_tflops": round(fl["attn_fwd"] / (ks["attn_fwd"] / 1e3) / 1e12, 2),
            "unfused_kernels_ms": {k: round(v, 4) for k, v in ks.items()}}


def time_forward(name: str, steps: int, warmup: int) -> dict:
    """The forward of a forward-only workload with single fp16 operands: the
    unfused path (norm, up-projection, attention; HIP events around each kernel)
    and the fused one."""
    import torch
    import laga_inputs as li
    from head_latent_attention_laga_amd import LagaPath, _lib
    d, _ = li.workload(name)
    x = {k: li.to_torch(t) for k, t in li.make_inputs(d, 0).items()}
    p = LagaPath(d.B, d.S, d.n_h, d.sp_size, d.sp_rank, d.d_kv, d.d_nope, d.d_rope, d.d_v, d.dtype, FP16, d.eps)
    out = p.alloc_forward()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for _ in range(warmup):
        p.forward(x, out)
    torch.cuda.synchronize()
    for i in range(steps):
        e = ev[i]
        e[0].record()
        _lib.latent_norm(p.dims, x["latent"], x["gamma"], out["latent_n"], out["rstd"])
        e[1].record()
        _lib.kv_up(p.dims, out["latent_n"], x["w_kv_b"], out["k_nope"], out["v"])
        e[2].record()
        _lib.attn_fwd(p.dims, x["q"], out["k_nope"], x["k_pe"], out["v"], out["o"], out["lse"])
        e[3].record()
    torch.cuda.synchronize()
    ks = {n: statistics.mean(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(steps))
          for k, n in enumerate(["rmsnorm_fwd", "kv_up", "attn_fwd"])}
    del out
    fused_ms = time_fused(p, x, steps, warmup)
    del x
    torch.cuda.empty_cache()
    return {"workload": name, "B": d.B, "S": d.S, "local_heads": d.h, "n_h": d.n_h, "sp_size": d.sp_size,
            **forward_summary(d, ks, fused_ms)}


def step_peak_memory(d) -> dict:
    """Device memory of one training step as torch's allocator records it: the
    inputs, then the forward's kept outputs, then the backward's workspace and
    gradients, with the peak over the step (nothing else is allocated)."""
    import torch
    import laga_inputs as li
    from head_latent_attention_laga_amd import LagaPath, _lib
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    m0 = torch.cuda.memory_allocated()
    x = {k: li.to_torch(t) for k, t in li.make_inputs(d, 0, backward=True).items()}
    m_in = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    p = LagaPath(d.B, d.S, d.n_h, d.sp_size, d.sp_rank, d.d_kv, d.d_nope, d.d_rope, d.d_v, d.dtype, SPLIT, d.eps)
    fwd = p.forward(x)
    m_fwd = torch.cuda.memory_allocated()
    g = p.alloc_backward()
    m_bwd = torch.cuda.memory_allocated()
    p.backward(x, fwd, x["d_o"], g)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    ws = _lib.attn_bwd_workspace_bytes(p.dims)
    del x, fwd, g
    torch.cuda.empty_cache()
    mb = 2.0 ** 20
    return {"inputs_mb": round((m_in - m0) / mb, 1), "forward_kept_mb": round((m_fwd - m_in) / mb, 1),
            "backward_workspace_mb": round(ws / mb, 1), "gradients_mb": round((m_bwd - m_fwd - ws) / mb, 1),
            "step_peak_mb": round((peak - m0) / mb, 1), "step_peak_above_inputs_mb": round((peak - m_in) / mb, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/*.md and profiles/traffic.json from the rocprofv3 output in DIR, then exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the SP group; runs on more than one GPU "
              "are not part of this path (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import laga_inputs as li
    from head_latent_attention_laga_amd import LagaPath, _lib

    if args.calibrate_copy:
        calibration_copy()
    d, _ = li.workload(WORKLOAD)
    inp = li.make_inputs(d, 0, backward=True)
    x = {k: li.to_torch(t) for k, t in inp.items()}
    dev = torch.device("cuda")
    path = LagaPath(d.B, d.S, d.n_h, d.sp_size, d.sp_rank, d.d_kv, d.d_nope, d.d_rope, d.d_v, d.dtype, SPLIT,
                    d.eps)
    fwd = path.alloc_forward()
    grads = path.alloc_backward()
    fast = LagaPath(d.B, d.S, d.n_h, d.sp_size, d.sp_rank, d.d_kv, d.d_nope, d.d_rope, d.d_v, d.dtype, FP16,
                    d.eps)
    ffwd = fast.alloc_forward()
    torch.cuda.synchronize()

    names = ["rmsnorm_fwd", "kv_up", "attn_fwd"] + list(_lib.BWD_STAGE_NAMES)
    nev = 3 + _lib.LAGA_BWD_STAGES + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]

    def step(e=None):
        dims = path.dims
        if e is not None:
            e[0].record()
        _lib.latent_norm(dims, x["latent"], x["gamma"], fwd["latent_n"], fwd["rstd"])
        if e is not None:
            e[1].record()
        _lib.kv_up(dims, fwd["latent_n"], x["w_kv_b"], fwd["k_nope"], fwd["v"])
        if e is not None:
            e[2].record()
        _lib.attn_fwd(dims, x["q"], fwd["k_nope"], x["k_pe"], fwd["v"], fwd["o"], fwd["lse"])
        g = grads
        bargs = (dims, x["q"], x["latent"], x["gamma"], fwd["rstd"], fwd["k_nope"], x["k_pe"], fwd["v"],
                 x["w_kv_b"], fwd["o"], fwd["lse"], x["d_o"], g["dq"], g["d_latent"], g["d_k_pe"],
                 g["d_w_kv_b"], g["d_gamma"], g["workspace"])
        if e is not None:
            _lib.attn_bwd_traced(*bargs, events=e[3:])
        else:
            _lib.attn_bwd(*bargs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: statistics.mean(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps))
           for k, n in enumerate(names)}
    # Median and minimum over the timed steps: of each kernel, and of a whole
    # step between its first and last event (launch gaps included).
    per_med = {n: statistics.median(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps))
               for k, n in enumerate(names)}
    per_min = {n: min(ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)) for k, n in enumerate(names)}
    step_ev = [ev[i][0].elapsed_time(ev[i][nev - 1]) for i in range(args.steps)]
    ms_step = wall * 1e3 / args.steps
    fl = alg_flops(d)
    tok_s = d.B * d.S / (ms_step / 1e3)

    # Forward alone with single fp16 operands (the forward-only workload's precision).
    fe = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        fast.forward(x, ffwd)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        e = fe[i]
        e[0].record()
        _lib.latent_norm(fast.dims, x["latent"], x["gamma"], ffwd["latent_n"], ffwd["rstd"])
        e[1].record()
        _lib.kv_up(fast.dims, ffwd["latent_n"], x["w_kv_b"], ffwd["k_nope"], ffwd["v"])
        e[2].record()
        _lib.attn_fwd(fast.dims, x["q"], ffwd["k_nope"], x["k_pe"], ffwd["v"], ffwd["o"], ffwd["lse"])
        e[3].record()
    torch.cuda.synchronize()
    fwall = (time.perf_counter() - t1) * 1e3 / args.steps
    fper = {n: statistics.mean(fe[i][k].elapsed_time(fe[i][k + 1]) for i in range(args.steps))
            for k, n in enumerate(["rmsnorm_fwd", "kv_up", "attn_fwd"])}
    fused_ms = time_fused(fast, x, args.steps, args.warmup)
    fsum = forward_summary(d, fper, fused_ms)

    # The absorbed form (B2) on the same inputs: its forward, and the device memory
    # each form's forward allocates for its outputs and kept intermediates (what a
    # training step holds until the backward), read from torch's allocator.
    m0 = torch.cuda.memory_allocated()
    mem_laga_split = path.alloc_forward()
    m1 = torch.cuda.memory_allocated()
    absb = fast.alloc_absorbed()
    m2 = torch.cuda.memory_allocated()
    del mem_laga_split
    ae = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        fast.absorbed_forward(x, absb)
    torch.cuda.synchronize()
    for i in range(args.steps):
        ae[i][0].record()
        fast.absorbed_forward(x, absb)
        ae[i][1].record()
    torch.cuda.synchronize()
    abs_ms = statistics.mean(ae[i][0].elapsed_time(ae[i][1]) for i in range(args.steps))
    # Its backward (every product with bf16 hi + lo terms, like the step's split operands),
    # which recomputes q_abs, the scores, lse and acc from the inputs one chunk of query
    # rows at a time.
    absg = fast.alloc_backward(workspace_bytes=_lib.absorbed_bwd_workspace_bytes(fast.dims))
    be = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(max(1, args.warmup // 2)):
        fast.absorbed_backward(x, absb, x["d_o"], absg)
    torch.cuda.synchronize()
    for i in range(args.steps):
        be[i][0].record()
        fast.absorbed_backward(x, absb, x["d_o"], absg)
        be[i][1].record()
    torch.cuda.synchronize()
    absb_ms = statistics.mean(be[i][0].elapsed_time(be[i][1]) for i in range(args.steps))
    del absb, absg
    abs_step = abs_ms + absb_ms
    abs_step_fl = absorbed_flops(d) + absorbed_bwd_flops(d)
    absorbed = {
        "fwd_ms": round(abs_ms, 4), "fwd_tokens_s": round(d.B * d.S / (abs_ms / 1e3), 1),
        "fwd_tflops_own": round(absorbed_flops(d) / (abs_ms / 1e3) / 1e12, 2),
        "fwd_time_vs_laga_fwd_fp16": round(abs_ms / min(fused_ms, fper["rmsnorm_fwd"] + fper["kv_up"]
                                                        + fper["attn_fwd"]), 3),
        "bwd_ms": round(absb_ms, 4), "bwd_tflops_own": round(absorbed_bwd_flops(d) / (absb_ms / 1e3) / 1e12, 2),
        "step_ms": round(abs_step, 4), "step_tokens_s": round(d.B * d.S / (abs_step / 1e3), 1),
        "step_tflops_own": round(abs_step_fl / (abs_step / 1e3) / 1e12, 2),
        "step_frac_peak_own": round(abs_step_fl / (abs_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_flops_vs_laga": round(abs_step_fl / fl["step"], 3),
        "step_time_vs_laga": round(abs_step / ms_step, 3),
        "bwd_workspace_mb": round(_lib.absorbed_bwd_workspace_bytes(fast.dims) / 2**20, 1),
        "forward_buffers_mb": {"laga_split": round((m1 - m0) / 2**20, 1), "absorbed": round((m2 - m1) / 2**20, 1)},
    }

    # Roofline of the dominant kernel of the step.
    work = {"rmsnorm_fwd": ("hbm", d.B * d.S * d.d_kv * (2 + 4) + 4 * d.B * d.S + 2 * d.d_kv),
            "kv_up": ("mfma", fl["kv_up"]), "attn_fwd": ("mfma", fl["attn_fwd"]),
            "attn_bwd_dkdv": ("mfma", fl["bwd_dkdv"]), "attn_bwd_dq": ("mfma", fl["bwd_dq"]),
            "fold_dL": ("mfma", fl["kv_up"]), "fold_dW": ("mfma", fl["kv_up"])}
    dom = max((n for n in per if n in work), key=lambda n: per[n])
    bound, units = work[dom]
    ach = units / (per[dom] / 1e3) / (1e12 if bound == "mfma" else 1e9)
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    tr = kernel_traffic(dom)
    roofline = {"kernel": dom, "bound": bound, "achieved": round(ach, 2), "peak": peak,
                "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(ach / peak, 4),
                "traffic": tr}

    kvb = _lib.kv_elem_bytes(path.dims)
    act = {k: round(v / 2**20, 1) for k, v in activation_bytes(d, kvb).items()}
    act["laga_backward_workspace"] = round(_lib.attn_bwd_workspace_bytes(path.dims) / 2**20, 1)

    # The other forward-only workloads, then the step's measured memory.
    del x, fwd, grads, ffwd
    torch.cuda.empty_cache()
    other = {"v3_sp8_s4096_h16": time_forward("v3_sp8_s4096_h16", args.steps, args.warmup),
             "v3_sp1_s4096_h128": time_forward("v3_sp1_s4096_h128", args.steps, args.warmup)}
    mem = step_peak_memory(d)
    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LAGA per-rank MLA attention block fwd+bwd, causal, one rank's head shard",
                   "B": d.B, "S": d.S, "local_heads": d.h, "n_h": d.n_h, "sp_size": d.sp_size,
                   "d_kv": d.d_kv, "d_nope": d.d_nope, "d_rope": d.d_rope, "d_v": d.d_v,
                   "operands": "fp16/bf16 hi+lo split, fp32 accumulate", "parallelism": "one GPU (one SP rank)"},
        "tflops_step": round(fl["step"] / (ms_step / 1e3) / 1e12, 2),
        "frac_peak_step": round(fl["step"] / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "forward_fp16_operands": {**fsum, "unfused_wall_ms": round(fwall, 4)},
        "kernels_ms": {k: round(v, 4) for k, v in per.items()},
        "kernels_ms_median": {k: round(v, 4) for k, v in per_med.items()},
        "kernels_ms_min": {k: round(v, 4) for k, v in per_min.items()},
        "step_ms_events": {"median": round(statistics.median(step_ev), 4), "min": round(min(step_ev), 4)},
        "sclk": gpu_sclk(),
        "roofline": roofline,
        "activation_mb": act,
        "memory_step_mb": mem,
        "forward_other_workloads": other,
        "absorbed_form": absorbed,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def gpu_sclk():
    """The shader clock level the driver marks as current in sysfs (None if unavailable).

    Read from the file directly rather than through rocm-smi: a child process
    started under a profiler that preloads its GPU library would initialise the
    GPU before its own exec."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lines = [ln.strip() for ln in f if ln.strip().endswith("*")]
        except OSError:
            continue
        if lines:
            return lines[0]
    return None


if __name__ == "__main__":
    main()
