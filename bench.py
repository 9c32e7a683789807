"""Benchmark of the block-diffusion drafting hot path on one MI355X.

A step is one draft_block call (ingest of the newly committed positions, the block forward, the
LM head and argmax or sampled drafting) followed by verify_greedy on the target's logits, or by
select_streak over K sampled drafts.  The headline workload is the Qwen3-8B-shaped drafter at
batch 32 (block 16, 7 draft layers mixing 9 target layers, cached context lengths uniform in
[256, 3072], argmax drafts, greedy verify).  Inputs are synthetic and resident in HBM before
timing.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    one JSON line for the headline workload
python bench.py --workload NAME | --all-workloads [--cpu-baseline-all]
    one JSON line per workload (qwen3-4b, qwen3-8b, gpt-oss-20b, specdiff2-7b)

Auxiliary modes for the HBM-traffic figure of the dominant kernel (rocprofv3 counter passes):
  python bench.py --calibrate-copy           plain 1 GiB device copies (counter scale factor)
  python bench.py --summarize-traffic DIR    FETCH_SIZE / WRITE_SIZE CSVs of the bench and of the
                                             copy runs -> profiles/traffic_qwen3-8b_bs32.json
"""
import argparse
import json
import re
import os
import sys
import time

import hashlib
import numpy as np

HBM_PEAK = 8.0e12          # bytes/s, MI355X datasheet
MFMA_BF16_PEAK = 2.5e15    # dense bf16 flop/s, MI355X datasheet
WORKLOAD = "qwen3-8b"
WORKLOADS_ALL = ["qwen3-4b", "qwen3-8b", "gpt-oss-20b", "specdiff2-7b"]
METRIC = "drafted 16-tok blocks/s (draft fwd+verify) Qwen3-8B-shape bs=32; % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--all-workloads", action="store_true",
                    help="one JSON line per bf16 workload (Qwen3-4B, Qwen3-8B, GPT-OSS-20B and "
                         "SpecDiff-2 shapes)")
    ap.add_argument("--cpu-baseline-all", action="store_true",
                    help="time the oracle on every workload, not only the headline one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps-only", action="store_true",
                    help="skip the instrumented pass and the cold-ingest timing")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-traffic", metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="MFMA-activity counter passes under DIR -> profiles/mfma_counters_*.json")
    ap.add_argument("--summarize-kernel-stats", metavar="CSV",
                    help="a rocprofv3 kernel_stats.csv -> a markdown table on stdout")
    ap.add_argument("--sweep-block", action="store_true",
                    help="draft_block latency against block length (SpecDiff-2-shaped drafter)")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qwen3-8b_bs32.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mfma_counters_qwen3-8b_bs32.json")
XCDS, SIMDS = 8, 1024       # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
COPY_BYTES = 1 << 30


def strip_comments(src: str) -> str:
    """C/C++ source without comments and blank-space differences (the code the compiler sees)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())


def kernel_source_hash(d=None):
    """Hash of the HIP sources' code (comments and spacing ignored): traffic counters are only
    valid for the build they came from."""
    d = d or os.path.join(ROOT, "block_diffusion_drafter_draft_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        h.update(strip_comments(open(os.path.join(d, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def calibrate_copy():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))


def summarize_traffic(d):
    """Per-launch HBM bytes of each library kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    runs (KiB per dispatch), scaled by what the same counters read for a plain copy of known
    size.  Expects DIR/{fetch,write}/ (bench) and DIR/{copy_fetch,copy_write}/ (copy runs)."""
    import csv
    import glob

    def per_kernel(sub, counter):
        """Counter values per kernel name, restricted to dispatches with the grid of the last
        dispatch of that kernel (the measured steps; the cold ingest runs other grids)."""
        rows = {}
        for f in glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.setdefault(r["Kernel_Name"], []).append(
                        (int(r["Dispatch_Id"]), r["Grid_Size"], float(r["Counter_Value"])))
        vals = {}
        for k, rs in rows.items():
            rs.sort()
            g = rs[-1][1]
            vals[k] = [v for _, gs, v in rs if gs == g]
        return vals

    def copy_factor(sub, counter):
        v = [x for k, xs in per_kernel(sub, counter).items() if "copy" in k.lower() or
             "elementwise" in k.lower() for x in xs]
        v = sorted(v)[-3:]                       # the three 1 GiB copies
        return (sum(v) / len(v) * 1024.0) / COPY_BYTES   # KiB counted per byte moved
    ff, fw = copy_factor("copy_fetch", "FETCH_SIZE"), copy_factor("copy_write", "WRITE_SIZE")
    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    out = {"commands": [
               "REPO=<repository root>; OUT=<output directory>",
               "cd /tmp && export TMPDIR=/tmp",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/traffic/fetch"
               " -o run -- python3 $REPO/bench.py --steps 3 --warmup 1 --profile-steps-only"
               " --no-cpu-baseline",
               "(the same with --pmc WRITE_SIZE into $OUT/traffic/write)",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/traffic/copy_fetch"
               " -o run -- python3 $REPO/bench.py --calibrate-copy",
               "(the same with --pmc WRITE_SIZE into $OUT/traffic/copy_write)",
               "python3 $REPO/bench.py --summarize-traffic $OUT/traffic"],
           "source_hash": kernel_source_hash(), "copy_factor_fetch": round(ff, 4),
           "copy_factor_write": round(fw, 4), "kernels": {}}
    for k in fetch:
        if "dbd::" not in k and not k.startswith("_ZN3dbd"):
            continue
        fb = sum(fetch[k]) / len(fetch[k]) * 1024.0 / ff
        wb = (sum(write.get(k, [0])) / max(1, len(write.get(k, [0])))) * 1024.0 / fw
        out["kernels"][k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                             "dispatches": len(fetch[k])}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps({"copy_factor_fetch": out["copy_factor_fetch"],
                      "copy_factor_write": out["copy_factor_write"],
                      "kernels": len(out["kernels"])}))


def _counter_rows(d):
    """{kernel: {counter: mean value}} over the dispatches of each kernel with the grid of its
    last dispatch (the measured steps; the cold ingest runs other grids), from every
    *counter_collection.csv under d."""
    import csv
    import glob
    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(
                (int(r["Dispatch_Id"]), r["Grid_Size"], float(r["Counter_Value"])))
    out = {}
    for (k, c), rs in rows.items():
        rs.sort()
        g = rs[-1][1]
        v = [x for _, gs, x in rs if gs == g]
        out.setdefault(k, {})[c] = sum(v) / len(v)
    return out


def summarize_counters(d):
    """MFMA activity of each library kernel from rocprofv3 --pmc passes under d.  GRBM_GUI_ACTIVE
    reads the sum over the 8 XCDs, so a kernel's cycles are GRBM_GUI_ACTIVE / 8 (checked against
    the kernel-trace durations at the shader clock); SQ_VALU_MFMA_BUSY_CYCLES counts busy MFMA
    cycles summed over the 1,024 SIMDs, so the busy fraction is BUSY / (1024 x cycles).
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 is the bf16 MFMA flops."""
    cs = _counter_rows(d)
    out = {"commands": [
               "REPO=<repository root>; OUT=<output directory>",
               "cd /tmp && export TMPDIR=/tmp",
               "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
               "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
               "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d $OUT/counters -o run "
               "-- python3 $REPO/bench.py --steps 3 --warmup 1 --profile-steps-only "
               "--no-cpu-baseline",
               "python3 $REPO/bench.py --summarize-counters $OUT/counters"],
           "source_hash": kernel_source_hash(), "xcds": XCDS, "simds": SIMDS, "kernels": {}}
    for k, v in cs.items():
        if "dbd::" not in k and not k.startswith("_ZN3dbd"):
            continue
        g = v.get("GRBM_GUI_ACTIVE")
        if not g:
            continue
        cyc = g / XCDS
        e = {"cycles": round(cyc)}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            e["mfma_busy"] = round(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc), 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in v:
            e["mfma_bf16_flops"] = round(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512)
        if "SQ_WAVE_CYCLES" in v and v["SQ_WAVE_CYCLES"]:
            for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS"):
                if c in v:
                    e[c.lower() + "_per_wave_cycle"] = round(v[c] / v["SQ_WAVE_CYCLES"], 4)
        if "SQ_LDS_BANK_CONFLICT" in v:
            e["lds_bank_conflict_cycles"] = round(v["SQ_LDS_BANK_CONFLICT"])
        out["kernels"][k] = e
    json.dump(out, open(COUNTERS_FILE, "w"), indent=1)
    print(json.dumps({k: e.get("mfma_busy") for k, e in out["kernels"].items()
                      if e.get("mfma_busy")}))


def summarize_kernel_stats(path):
    """A rocprofv3 kernel_stats.csv as a markdown table (calls, average and total time, share)."""
    import csv
    rows = list(csv.DictReader(open(path)))
    print("| kernel | calls | avg us | total ms | % |")
    print("|---|---|---|---|---|")
    for r in rows:
        name = r["Name"] if len(r["Name"]) <= 100 else r["Name"][:97] + "..."
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.2f} |")


def measured_mfma_busy(stage):
    """The counter-measured MFMA busy fraction of the one library kernel the stage launches, from
    the committed counter summary, or None when absent, ambiguous or on other kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    t = json.load(open(COUNTERS_FILE))
    if t.get("source_hash") != kernel_source_hash():
        return None
    ks = [k for k in stage_kernels(stage, t["kernels"]) if "mfma_busy" in t["kernels"][k]]
    if len(ks) != 1:
        return None
    return {"mfma_busy": t["kernels"][ks[0]]["mfma_busy"], "kernel": ks[0]}


# Epilogue kind (a template argument of every GEMM kernel) of each timed GEMM stage whose
# launches all use one epilogue, and the kernel name fragment of the other stages.
STAGE_EPILOGUE = {"gemm_gateup": 4, "gemm_lmhead": 5, "gemm_qkv": 2, "gemm_ctxkv": 3}
STAGE_KERNEL = {"attn": "attn_stream_kernel", "mix": "mix_rmsnorm_kernel"}
# position of the epilogue kind in each GEMM kernel's template argument list
KIND_ARG = {"gemm_bf16_kernel": 3, "gemm_big_kernel": 3, "gemm_w8_kernel": 3,
            "gemm_w8r_kernel": 1}


def gemm_epilogue(name):
    """Epilogue kind of a demangled library GEMM kernel name, or None."""
    m = re.search(r"dbd::(gemm_\w+_kernel)<([^>]*)>", name)
    if not m or m.group(1) not in KIND_ARG:
        return None
    return int(m.group(2).split(",")[KIND_ARG[m.group(1)]])


def stage_kernels(stage, names):
    """The kernel names among `names` that the timed stage launches."""
    if stage in STAGE_EPILOGUE:
        return [k for k in names if gemm_epilogue(k) == STAGE_EPILOGUE[stage]]
    if stage in STAGE_KERNEL:
        return [k for k in names if STAGE_KERNEL[stage] in k]
    return []


def measured_traffic(stage):
    """HBM bytes per launch of the one library kernel the stage launches, from the committed
    counter summary, or None when absent, ambiguous or taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_hash") != kernel_source_hash():
        return None
    ks = stage_kernels(stage, t["kernels"])
    if len(ks) != 1:
        return None
    v = t["kernels"][ks[0]]
    return {"bytes": v["fetch_bytes"] + v["write_bytes"], "kernel": ks[0]}


def algorithmic_costs(wl, ctx, new):
    """Per-stage algorithmic (bytes, flops) of one step: weights, cache and logits read once,
    activations read and written once."""
    sh = wl.shape
    N, B = wl.batch, wl.block_len
    M, D = N * B, wl.n_draft
    Md = N * D
    H, F, V, Ld, Lt = sh.hidden, sh.ffn, sh.vocab, sh.n_layers, sh.n_target_layers
    qd, kd, hd, kvh = sh.q_dim, sh.kv_dim, sh.head_dim, sh.n_kv_heads
    grp = sh.n_q_heads // kvh
    es = 2 if sh.dtype == "bf16" else 4
    T = int(np.sum(new))
    keys = ctx + new + B                              # keys attended per sequence
    c = {}
    if Lt > 0 and T > 0:
        if getattr(sh, "ctx_fusion", "mix") == "fc":
            # fully connected fusion: fusion weights and the concatenated target rows once, the
            # shared feature written once
            c["mix"] = (H * Lt * H * es + T * Lt * H * es + T * H * es, 2 * T * H * Lt * H)
        else:
            c["mix"] = (T * Lt * H * es + Ld * T * H * es, 0)
        c["gemm_ctxkv"] = (Ld * (2 * kd * H * es + T * H * es + T * 2 * kd * es),
                           2 * T * 2 * kd * H * Ld)
    c["gemm_qkv"] = (Ld * ((qd + 2 * kd) * H * es + M * H * es + M * (qd + 2 * kd) * es),
                     2 * M * (qd + 2 * kd) * H * Ld)
    c["attn"] = (Ld * (int(np.sum(keys)) * kvh * hd * 2 * es + 2 * M * qd * es),
                 Ld * int(np.sum(keys)) * kvh * 4 * B * grp * hd)
    c["gemm_o"] = (Ld * (H * qd * es + M * qd * es + 2 * M * H * 4), 2 * M * H * qd * Ld)
    c["gemm_gateup"] = (Ld * (2 * F * H * es + M * H * es + M * F * es), 2 * M * 2 * F * H * Ld)
    c["gemm_down"] = (Ld * (H * F * es + M * F * es + 2 * M * H * 4), 2 * M * H * F * Ld)
    sampling = wl.temperature > 0
    # sampling keeps the fp32 logits, which the drafting stage then reads once
    c["gemm_lmhead"] = (V * H * es + Md * H * es + (Md * V * 4 if sampling else 0),
                        2 * Md * V * H)
    if sampling:
        c["draft"] = (Md * V * 4 + N * wl.n_drafts * D * 4, 0)
    c["rownorm"] = ((2 * Ld + 1) * M * H * (4 + es) + M * H * (es + 4), 0)
    if wl.verify == "streak":
        c["select"] = (N * wl.n_drafts * wl.verify_rows * V * 4, 0)
    else:
        c["verify"] = (N * wl.verify_rows * V * 4, 0)
    return c


class StepSetup:
    """Inputs of one workload resident on the GPU and the timed step: one draft_block call
    (ingest of the newly committed positions for drafters that mix target layers, the block
    forward, the LM head, argmax or sampled drafting), then verify_greedy on the first draft
    (greedy workloads) or select_streak over the K drafts (streak workloads)."""

    def __init__(self, wl, dbd, synth, torch, dev="cuda"):
        self.wl = wl
        sh = self.sh = wl.shape
        N, B, D, V, K = wl.batch, wl.block_len, wl.n_draft, sh.vocab, wl.n_drafts
        self.N, self.B, self.D, self.V, self.K = N, B, D, V, K
        ctx, new = synth.make_lengths(wl, 0)
        self.ctx, self.new = ctx, new
        cap = synth.capacity_for(wl, ctx, new)
        self.W = W = synth.make_weights(sh, 0, dev)
        self.desc = desc = dbd.model_desc(sh, act_pairs=wl.act_pairs)
        self.wst = wst = dbd.weights_struct(W)
        self.tokens = tokens = synth.make_block_tokens(wl, 0, dev)
        dt = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
        ks, vs = dbd.kv_cache_shapes(sh, N, cap)
        self.kv_k = kv_k = torch.zeros(ks, dtype=dt, device=dev)
        self.kv_v = kv_v = torch.zeros(vs, dtype=dt, device=dev)
        self.hidden = None
        T_cold = 0
        if wl.ctx_source == "hidden":
            self.hidden = [synth.make_hidden(sh, int(ctx[i] + new[i]), 0, i, dev)
                           for i in range(N)]
            self.cold_rows = torch.cat([self.hidden[i][: int(ctx[i])] for i in range(N)],
                                       0).contiguous()
            self.step_rows = torch.cat([self.hidden[i][int(ctx[i]):] for i in range(N)],
                                       0).contiguous()
            T_cold, self.T_step = self.cold_rows.shape[0], self.step_rows.shape[0]
        else:
            # the drafter takes its context K/V from the cache: synthetic rotated K/V, no ingest
            Kc, Vc = synth.make_cache_kv(sh, N, int(ctx.max()), 0, dev)
            for i in range(N):
                C = int(ctx[i])
                C8 = (C + 7) // 8 * 8
                kv_k[:, i, :, :C] = Kc[:, i, :, :C]
                vpad = torch.zeros((sh.n_layers, sh.n_kv_heads, C8, sh.head_dim), dtype=dt,
                                   device=dev)
                vpad[:, :, :C] = Vc[:, i, :, :C]
                kv_v[:, i, :, : C8 // 8] = dbd.pack_values(vpad)
            del Kc, Vc
            self.step_rows, self.T_step = None, 0
            new = self.new = np.zeros(N, np.int64)
        self.T_cold = T_cold
        self.ws = torch.empty(dbd.draft_workspace_bytes(desc, N, B, wl.n_anchor,
                                                        max(T_cold, self.T_step), K,
                                                        wl.temperature, cap),
                              dtype=torch.uint8, device=dev)
        self.off_cold = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32),
                                     device=dev)
        self.off_step = torch.tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32),
                                     device=dev)
        self.zeros = torch.zeros(N, dtype=torch.int32, device=dev)
        self.ctx_t = torch.tensor(ctx.astype(np.int32), device=dev)
        self.drafts = torch.empty((N, K, D), dtype=torch.int32, device=dev)
        self.n_acc = torch.empty(N, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(N, dtype=torch.int32, device=dev)
        self.committed = torch.empty((N, D + 1), dtype=torch.int32, device=dev)
        R = wl.verify_rows
        if wl.verify == "streak":
            # verifier logits [N, K, R, V] planted per (sequence, draft) around fixed drafts
            self.v_drafts = synth.make_drafts(N, K, D, V, seed=1, device=dev)
            self.vlogits, _ = synth.make_planted_streak_logits(self.v_drafts, R, V,
                                                               wl.planted_alpha, seed=1,
                                                               device=dev)
            self.vws = torch.empty(dbd.select_workspace_bytes(N, K, R, V), dtype=torch.uint8,
                                   device=dev)
            self.selected = torch.empty(N, dtype=torch.int32, device=dev)
        else:
            self.v_drafts = synth.make_drafts(N, 1, D, V, seed=1, device=dev)[:, 0].contiguous()
            self.vlogits, _ = synth.make_planted_verify_logits(self.v_drafts, R, V,
                                                               wl.planted_alpha, seed=1,
                                                               device=dev)
            self.vws = torch.empty(dbd.verify_workspace_bytes(N, R, V), dtype=torch.uint8,
                                   device=dev)
        self.dbd = dbd

    def cold(self):
        """Fill the cache: cold ingest of every cached position (mixing drafters only)."""
        if self.wl.ctx_source != "hidden":
            return
        self.dbd.draft_block(self.desc, self.wst, self.tokens, self.cold_rows, self.off_cold,
                             self.zeros, self.kv_k, self.kv_v, self.drafts, self.ws, self.T_cold,
                             n_drafts=self.K, temperature=self.wl.temperature,
                             n_anchor=self.wl.n_anchor)

    def step(self, seed=7):
        wl, dbd = self.wl, self.dbd
        dbd.draft_block(self.desc, self.wst, self.tokens, self.step_rows, self.off_step,
                        self.ctx_t, self.kv_k, self.kv_v, self.drafts, self.ws, self.T_step,
                        n_drafts=self.K, temperature=wl.temperature, seed=seed,
                        n_anchor=wl.n_anchor)
        if wl.verify == "streak":
            # the verifier scored the drafts sampled here; its logits are fixed synthetic rows
            dbd.select_streak(self.vlogits, self.drafts, self.selected, self.n_acc, self.bonus,
                              self.committed, self.vws)
        else:
            dbd.verify_greedy(self.vlogits, self.drafts[:, 0], self.n_acc, self.bonus,
                              self.committed, self.vws)


def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def stage_table(dbd, torch, fn, steps, costs):
    """Per-stage kernel time from HIP event pairs the library records around each launch on its
    stream, with the stage's algorithmic GB/s and TFLOP/s."""
    dbd.timing_reset()
    dbd.timing_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    tm = dbd.timing_read()
    dbd.timing_enable(False)
    dbd.timing_reset()
    stages = {}
    for name, (tot, n) in tm.items():
        if n == 0:
            continue
        b, f = costs.get(name, (0, 0))
        t = tot / steps * 1e-3
        stages[name] = {"ms_per_step": round(tot / steps, 4),
                        "launches_per_step": n // steps,
                        "GBps": round(b / t / 1e9, 1) if b else None,
                        "TFLOPs": round(f / t / 1e12, 1) if f else None,
                        "roof_us": round(max(b / HBM_PEAK, f / MFMA_BF16_PEAK) * 1e6, 2)}
    return stages


def dominant_roofline(stages, costs, measured=True):
    """The roofline object of the stage that takes the most time."""
    dom = max(stages, key=lambda k: stages[k]["ms_per_step"])
    b, f = costs[dom]
    n = stages[dom]["launches_per_step"]
    avg_s = stages[dom]["ms_per_step"] / n * 1e-3
    if f and f / b > MFMA_BF16_PEAK / HBM_PEAK:
        ach = f / n / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": round(ach * 1e12 / MFMA_BF16_PEAK, 4)}
    else:
        ach = b / n / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": round(ach * 1e9 / HBM_PEAK, 4)}
    tr = measured_traffic(dom) if measured else None
    mb = measured_mfma_busy(dom) if measured else None
    roof.update({"kernel": dom, "launches_per_step": n,
                 "avg_launch_us": round(avg_s * 1e6, 2),
                 "algorithmic_bytes_per_launch": round(b / n),
                 "algorithmic_flops_per_launch": round(f / n),
                 "traffic": None if tr is None else tr["bytes"],
                 "traffic_kernel": None if tr is None else tr["kernel"],
                 "traffic_source": None if tr is None else os.path.relpath(TRAFFIC_FILE, ROOT),
                 "mfma_busy_counter": None if mb is None else mb["mfma_busy"],
                 "mfma_busy_source": None if mb is None else
                 os.path.relpath(COUNTERS_FILE, ROOT)})
    return roof


def describe(wl):
    sh = wl.shape
    ctx = (f"cached ctx U[{wl.ctx_lo},{wl.ctx_hi}]" if wl.ctx_lo != wl.ctx_hi
           else f"cached ctx {wl.ctx_lo}")
    src = (f"{sh.n_layers} draft layers x {sh.n_target_layers} target layers"
           if sh.n_target_layers else f"{sh.n_layers} layers, context K/V given in the cache")
    draft = ("argmax drafts" if wl.temperature <= 0
             else f"{wl.n_drafts} draft(s) sampled at T={wl.temperature:g}")
    ver = "greedy verify" if wl.verify == "greedy" else "streak self-selection + greedy accept"
    return (f"{wl.name}-shaped drafter: hidden {sh.hidden}, {sh.n_q_heads}q/{sh.n_kv_heads}kv x "
            f"{sh.head_dim}, ffn {sh.ffn}, {src}, vocab {sh.vocab}, block {wl.block_len}, batch "
            f"{wl.batch}, {ctx}, {draft}, {ver}")


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_kernel_stats:
        summarize_kernel_stats(args.summarize_kernel_stats)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep_block:
        sweep_block(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path needs no inter-GPU exchange; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import block_diffusion_drafter_draft_amd as dbd
    import synth

    names = WORKLOADS_ALL if args.all_workloads else [args.workload]
    for name in names:
        out = bench_workload(args, synth.workload(name), dbd, synth, torch)
        print(json.dumps(out), flush=True)
        torch.cuda.empty_cache()


def bench_workload(args, wl, dbd, synth, torch):
    dev = "cuda"
    sh = wl.shape
    t_setup = time.time()
    S = StepSetup(wl, dbd, synth, torch, dev)
    N, B, D, V, K = S.N, S.B, S.D, S.V, S.K
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    S.cold()
    torch.cuda.synchronize()
    ms = time_steps(torch, S.step, args.steps, args.warmup)

    costs = algorithmic_costs(wl, S.ctx, S.new)
    headline = wl.name == WORKLOAD
    stages, cold_info = {}, None
    if not args.profile_steps_only:
        stages = stage_table(dbd, torch, S.step, args.steps, costs)
        if headline:
            dbd.timing_reset()
            dbd.timing_enable(True)
            S.cold()
            torch.cuda.synchronize()
            tc = dbd.timing_read()
            dbd.timing_enable(False)
            dbd.timing_reset()
            mix_b = S.T_cold * (sh.n_target_layers + sh.n_layers) * sh.hidden * 2
            cold_info = {"rows": S.T_cold,
                         "mix_ms": round(tc["mix"][0], 3),
                         "mix_GBps": round(mix_b / (tc["mix"][0] * 1e-3) / 1e9, 1),
                         "ctxkv_gemm_ms": round(tc["gemm_ctxkv"][0], 3),
                         "ctxkv_TFLOPs": round(2 * S.T_cold * 2 * sh.kv_dim * sh.hidden *
                                               sh.n_layers / (tc["gemm_ctxkv"][0] * 1e-3) /
                                               1e12, 1)}
    extras = headline_extras(args, S, dbd, torch) if headline and not args.profile_steps_only \
        else {}
    roofline = dominant_roofline(stages, costs, measured=headline) if stages else None
    step_roof_s = sum(max(b / HBM_PEAK, f / MFMA_BF16_PEAK) for b, f in costs.values())

    cpu = None
    if not args.no_cpu_baseline and (headline or args.cpu_baseline_all):
        cpu = cpu_baseline(S)

    blocks_s = N / (ms * 1e-3)
    metric = (METRIC if headline else
              f"drafted {D}-tok blocks/s (draft fwd+{'select' if wl.verify == 'streak' else 'verify'})"
              f" {wl.name}-shape bs={N}; % roofline")
    out = {
        "metric": metric,
        "value": round(blocks_s, 1), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic",
        "config": {"workload": describe(wl), "batch": N, "block_len": B, "n_drafts": K,
                   "temperature": wl.temperature, "ctx_total": int(np.sum(S.ctx)),
                   "new_rows": int(S.T_step), "act_pairs": wl.act_pairs},
        "drafted_tok_per_s": round(blocks_s * D * K, 1),
        "step_roofline_us": round(step_roof_s * 1e6, 1),
        "step_roofline_frac": round(step_roof_s / (ms * 1e-3), 4),
        "roofline": roofline,
        "stages": stages,
    }
    if headline:
        out["cold_ingest"] = cold_info
        out.update(extras)
    out["cpu_baseline"] = cpu
    out["setup_s"] = round(t_setup, 1)
    return out


def headline_extras(args, S, dbd, torch):
    """Measurements next to the headline step (not part of it): lossless stochastic
    verification, top-p drafting and two-pass block refinement on the same workload."""
    dev = "cuda"
    wl, sh = S.wl, S.sh
    N, D, V = S.N, S.D, S.V
    tlogits = S.vlogits
    n_acc, bonus, committed = S.n_acc, S.bonus, S.committed
    g = torch.Generator(device=dev).manual_seed(2)
    dlog = (tlogits[:, :D] + 0.5 * torch.randn(tlogits[:, :D].shape, generator=g,
                                               device=dev)).contiguous()
    sws = torch.empty(max(dbd.sample_workspace_bytes(N, D, V), 256), dtype=torch.uint8,
                      device=dev)
    sdr = torch.empty((N, 1, D), dtype=torch.int32, device=dev)
    dbd.sample_from_logits(dlog, 1, 1.0, 5, sdr, sws)
    sdr = sdr[:, 0].contiguous()
    vws = torch.empty(dbd.verify_sample_workspace_bytes(N, D, wl.verify_rows, V),
                      dtype=torch.uint8, device=dev)
    it = iter(range(1 << 30))
    vms = time_steps(torch, lambda: dbd.verify_sample(tlogits, dlog, sdr, 1.0, 1.0, next(it),
                                                      n_acc, bonus, committed, vws),
                     args.steps, 3)
    vb = (N * wl.verify_rows + N * D) * V * 4
    vsample = {"ms": round(vms, 4), "logit_bytes": vb,
               "GBps": round(vb / (vms * 1e-3) / 1e9, 1),
               "hbm_frac": round(vb / (vms * 1e-3) / HBM_PEAK, 4),
               "mean_accepted": round(float(n_acc.float().mean().item()), 3)}
    # top-p nucleus drafting on the same draft logits (8 draws per position, p = 0.9)
    tws = torch.empty(dbd.sample_top_p_workspace_bytes(N, D, V), dtype=torch.uint8, device=dev)
    tout = torch.empty((N, 8, D), dtype=torch.int32, device=dev)
    tms = time_steps(torch, lambda: dbd.sample_top_p(dlog, 8, 1.0, 0.9, next(it), tout, tws),
                     args.steps, 3)
    tb = N * D * V * 4
    top_p = {"ms": round(tms, 4), "logit_bytes": tb, "draws_per_position": 8, "p": 0.9,
             "GBps": round(tb / (tms * 1e-3) / 1e9, 1),
             "hbm_frac": round(tb / (tms * 1e-3) / HBM_PEAK, 4)}
    # block refinement (Mask-Predict, two passes): the step's forward with its LM-head logits
    # kept, refine_block re-masking the floor(D/2) least confident drafts, the forward again on
    # the partly filled block (no new rows), the final update, the same greedy verify
    rlog = torch.empty((N, D, V), dtype=torch.float32, device=dev)
    rws = torch.empty(dbd.refine_workspace_bytes(N, D, V), dtype=torch.uint8, device=dev)
    gws = torch.empty(dbd.verify_workspace_bytes(N, wl.verify_rows, V), dtype=torch.uint8,
                      device=dev)
    rblk = S.tokens.clone()
    conf = torch.zeros((N, D), dtype=torch.int64, device=dev)
    r_acc = torch.empty(N, dtype=torch.int32, device=dev)
    r_bonus = torch.empty(N, dtype=torch.int32, device=dev)
    r_com = torch.empty((N, D + 1), dtype=torch.int32, device=dev)
    ctx2 = torch.tensor((S.ctx + S.new).astype(np.int32), device=dev)
    off0 = torch.zeros(N + 1, dtype=torch.int32, device=dev)

    def refined_step():
        rblk.copy_(S.tokens)
        conf.zero_()
        dbd.draft_block(S.desc, S.wst, rblk, S.step_rows, S.off_step, S.ctx_t, S.kv_k, S.kv_v,
                        S.drafts, S.ws, S.T_step, logits_out=rlog)
        dbd.refine_block(rlog, rblk, conf, wl.n_anchor, sh.mask_token_id, D // 2, rws)
        dbd.draft_block(S.desc, S.wst, rblk, None, off0, ctx2, S.kv_k, S.kv_v, S.drafts, S.ws,
                        0, logits_out=rlog)
        dbd.refine_block(rlog, rblk, conf, wl.n_anchor, sh.mask_token_id, 0, rws)
        dbd.verify_greedy(tlogits, rblk[:, wl.n_anchor:], r_acc, r_bonus, r_com, gws)

    rms = time_steps(torch, refined_step, args.steps, 2)
    ums = time_steps(torch, lambda: dbd.refine_block(rlog, rblk, conf, wl.n_anchor,
                                                     sh.mask_token_id, D // 2, rws),
                     args.steps, 0)
    refinement = {"rule": "mask-predict", "passes": 2, "remasked": D // 2,
                  "ms_per_step": round(rms, 4), "blocks_per_s": round(N / (rms * 1e-3), 1),
                  "refine_block_ms": round(ums, 4),
                  "refine_block_GBps": round(tb / (ums * 1e-3) / 1e9, 1)}
    return {"verify_sample": vsample, "top_p_sampling": top_p, "refinement": refinement}


def sweep_block(args, gammas=(8, 16, 32, 64), ctx_len=256):
    """draft_block latency against the block length gamma for the SpecDiff-2-shaped drafter (28
    layers, hidden 3584, 8 joint drafts at T = 1.5, batch 4) over a cached context of 256
    positions: the forward over gamma masks plus drafting.  The SpecDiff-2 notes (latency
    analysis) find the diffusion drafter's latency nearly flat in gamma until the GPU saturates;
    this measures the same shape of curve with synthetic weights."""
    import torch
    sys.path.insert(0, ROOT)
    import block_diffusion_drafter_draft_amd as dbd
    import synth
    dev = "cuda"
    base = synth.workload("specdiff2-7b")
    sh = base.shape
    N, K, T = base.batch, base.n_drafts, base.temperature
    W = synth.make_weights(sh, 0, dev)
    desc, wst = dbd.model_desc(sh, act_pairs=base.act_pairs), dbd.weights_struct(W)
    Kc, Vc = synth.make_cache_kv(sh, N, ctx_len, 0, dev)
    points = []
    for g in gammas:
        cap = ((ctx_len + g + 63) // 64) * 64
        ks, vs = dbd.kv_cache_shapes(sh, N, cap)
        kv_k = torch.zeros(ks, dtype=Kc.dtype, device=dev)
        kv_v = torch.zeros(vs, dtype=Vc.dtype, device=dev)
        kv_k[:, :, :, :ctx_len] = Kc
        kv_v[:, :, :, : ctx_len // 8] = dbd.pack_values(Vc)
        tokens = torch.full((N, g), sh.mask_token_id, dtype=torch.int32, device=dev)
        off = torch.zeros(N + 1, dtype=torch.int32, device=dev)
        ctx = torch.full((N,), ctx_len, dtype=torch.int32, device=dev)
        drafts = torch.empty((N, K, g), dtype=torch.int32, device=dev)
        ws = torch.empty(dbd.draft_workspace_bytes(desc, N, g, 0, 0, K, T, cap),
                         dtype=torch.uint8, device=dev)
        run = lambda: dbd.draft_block(desc, wst, tokens, None, off, ctx, kv_k, kv_v, drafts, ws,
                                      0, n_drafts=K, temperature=T, seed=7, n_anchor=0)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        # the same call captured once in a HIP graph and replayed: the ~10 launches per layer
        # are short at these sizes, so launch gaps are a visible part of the eager time.  Every
        # replay is checked against the eager drafts (same seed), with eager work in between.
        ref = drafts.clone()
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            run()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            run()
        for _ in range(3):
            drafts.fill_(-1)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(drafts, ref), "graph replay differs from the eager call"
            run()
            torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / args.steps
        dbd.timing_reset()
        dbd.timing_enable(True)
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        tm = dbd.timing_read()
        dbd.timing_enable(False)
        dbd.timing_reset()
        stages = {k: round(v[0] / args.steps, 3) for k, v in tm.items() if v[1]}
        points.append({"gamma": g, "ms": round(ms, 3), "graph_ms": round(gms, 3),
                       "drafted_tok_per_s": round(N * K * g / (gms * 1e-3), 1),
                       "stage_ms": stages})
        print(f"gamma {g}: {ms:.3f} ms eager, {gms:.3f} ms graph", file=sys.stderr, flush=True)
        del graph, kv_k, kv_v, ws
    print(json.dumps({"sweep": "block_len", "workload": f"specdiff2-7b-shaped drafter, batch {N}, "
                      f"{K} drafts at T={T}, cached context {ctx_len}",
                      "unit": "ms per draft_block (eager; graph = one HIP graph replay)",
                      "points": points}), flush=True)


def host_info():
    """The host's CPU model and thread counts (the machine the oracle baseline runs on)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu": model, "host_threads": os.cpu_count(), "threads_allowed": aff}


def cpu_baseline(S, min_s=10.0, max_seqs=8):
    """The oracle as it stands, on a bounded sample of the same workload.  For sequences 0, 1, ...
    (until min_s seconds of CPU work or max_seqs sequences) it runs the step the GPU runs for
    that sequence: the context K/V of the newly committed positions (drafters that mix target
    layers; the K/V of the cached positions are computed beforehand, untimed, as the GPU keeps
    them in its cache), the drafter forward, drafting from the fp32-rounded logits (argmax or
    the integer-exact sampler) and greedy verification or streak selection."""
    import torch
    from threadpoolctl import threadpool_info
    from oracle import accept, dnc, drafter as od
    wl, sh = S.wl, S.sh
    Wc = {k: v.detach().to("cpu") for k, v in S.W.items()}
    vl = S.vlogits
    t, seqs, lens = 0.0, 0, []
    while seqs < min(max_seqs, wl.batch) and t < min_s:
        i = seqs
        C, n = int(S.ctx[i]), int(S.new[i])
        toks = S.tokens[i].to("cpu").numpy()
        if wl.ctx_source == "hidden":
            h = S.hidden[i].to("cpu")
            cached = [od.context_kv(sh, Wc, l, h[:C]) for l in range(sh.n_layers)]
        else:
            import block_diffusion_drafter_draft_amd as dbd
            cached = [(S.kv_k[l, i, :, :C].to("cpu"),
                       dbd.unpack_values(S.kv_v[l, i]).to("cpu")[:, :C]) for l in
                      range(sh.n_layers)]
        vrow = vl[i: i + 1].to("cpu").numpy()
        t0 = time.perf_counter()
        if wl.ctx_source == "hidden" and n > 0:
            kv = []
            for l in range(sh.n_layers):
                k1, v1 = od.context_kv(sh, Wc, l, h[C:C + n], pos0=C)
                kv.append((np.concatenate([cached[l][0], k1], 1),
                           np.concatenate([cached[l][1], v1], 1)))
        else:
            kv = cached
        out = od.drafter_forward(sh, Wc, toks, wl.n_anchor, ctx_kv=kv)
        d = dnc.sample_drafts(out["logits"].astype(np.float32)[None], wl.n_drafts,
                              wl.temperature, 7)
        if wl.verify == "streak":
            accept.select_streak(vrow, d)
        else:
            accept.verify_greedy(vrow, d[:, 0])
        t += time.perf_counter() - t0
        seqs += 1
        lens.append(C + n)
        del kv, cached
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(seqs / t, 4), "unit": "blocks/s", "cores": int(threads),
            "kind": "oracle", **host_info(),
            "sample": f"{seqs} of {wl.batch} sequences (context {lens}): the oracle's ingest of "
                      f"the new positions, fp64 drafter forward from the cached context, "
                      f"drafting and {wl.verify} verification, {t:.1f} s; cores = the BLAS "
                      f"threads the oracle ran with"}


if __name__ == "__main__":
    main()
