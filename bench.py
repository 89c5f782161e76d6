"""Throughput of the batched speculative-decoding verification step on one MI355X.

One step = one spec_verify call (every kernel of the path) over one batch of
synthetic logits resident in HBM. Default workload: B=64 sequences, K=8 drafts,
V=128256, bf16 logits, temperature 0.7, target perturbation sd 1.0. Four copies
of the inputs rotate so that the 256 MB Infinity Cache cannot serve one step's
rows from the previous step.

Prints one JSON line: verified (sequence, position) rows per second, effective
HBM bandwidth of the compulsory bytes, a roofline entry for the dominant kernel
(the fused verification kernel, or the statistics pass of a filtered call: its
algorithmic bytes over its HIP-event duration on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X
METRIC = "verified rows/sec + effective HBM GB/s (% of ~8 TB/s), B=64 K=8 V=128256 bf16"
# kernels of a call, in launch order: one fused kernel without filters; the
# statistics, filter and draw passes with top-k
STAGES = {1: ["k_verify"], 3: ["k_stats", "k_filter", "k_draw"]}


def traffic_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")


class HipEvents:
    """Timing events made directly with the HIP runtime, flagged to skip the
    system-scope fence a default event performs (that fence writes back and
    invalidates caches, which would sit between the kernels being timed)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            self.handles.append(h.value)

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.handles[a], self.handles[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def close(self):
        for h in self.handles:
            self.hip.hipEventDestroy(h)
        self.handles = []


# The sources each counted kernel is compiled from (its own file and the
# headers it includes); a change to any of them voids its counter record.
KERNEL_SOURCES = {
    "k_verify": ["sv_fused.hip", "sv_rows.h", "sv_device.h", "sv_launch.h"],
    "k_stats": ["sv_verify.hip", "sv_rows.h", "sv_device.h", "sv_launch.h"],
    "k_lm_stats": ["sv_lmhead.hip", "sv_rows.h", "sv_device.h", "sv_launch.h"],
}


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_13_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(os.listdir(csrc))
    for f in names:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--sd-t", type=float, default=None, help="target perturbation sd")
    ap.add_argument("--sets", type=int, default=4, help="rotating input copies")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the other workloads in the headline run")
    ap.add_argument("--top-k", type=int, default=None,
                    help="override the workload's top-k (0: none)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="override the workload's top-p (1: none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle sample (0 disables)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--path", choices=["verify", "accept", "lmhead", "multi"], default="verify",
                    help="verify: the verification step (default); accept: the "
                         "acceptance statistics (spec_verify_accept_stats); lmhead: "
                         "verification from LM-head hidden states (spec_verify_lmhead, "
                         f"workload {W.LMHEAD_NAME}); multi: several draft chains per "
                         f"sequence (spec_verify_multi, workload {MULTI_NAME})")
    ap.add_argument("--traffic-from", metavar="DIR", default=None,
                    help="only summarise rocprofv3 counter runs: DIR/{fetch,write,cal_fetch,"
                         "cal_write} hold FETCH_SIZE / WRITE_SIZE runs of this bench command and "
                         "of --calibrate-copy; writes the traffic file bench.py reads")
    return ap.parse_args()


def calibrate_copy():
    """A plain 1 GiB device-to-device copy, for scaling the HBM byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}),
          flush=True)


def _counter_per_dispatch(run_dir, counter):
    """(kernel name, summed counter value) per dispatch of one rocprofv3 --pmc run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"bench.py: no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (fn, int(r["Dispatch_Id"]))
                name, v = per.get(key, (r["Kernel_Name"], 0.0))
                per[key] = (name, v + float(r["Counter_Value"]))
    return [per[k] for k in sorted(per)]


def traffic_summary(args):
    """HBM bytes per launch of the dominant kernel from FETCH_SIZE / WRITE_SIZE
    runs, each scaled by what the counter reads for a plain copy of known size."""
    import statistics
    d = args.traffic_from
    lm = args.path == "lmhead"
    if lm:
        # the sampling call's statistics GEMM (the greedy call's is k_lm_stats<true>)
        kernel, workload, match, extra = "k_lm_stats", W.LMHEAD_NAME, "k_lm_stats<false>", \
            "--path lmhead"
    else:
        stages = STAGES[1] if W.WORKLOADS[args.workload].get("top_k", 0) <= 0 else STAGES[3]
        kernel = stages[0] if len(stages) == 1 else "k_stats"
        workload, match, extra = args.workload, None, f"--no-other-configs --workload {args.workload}"
    cal_bytes_kib = (1 << 30) / 1024.0

    def calib(sub, counter):
        vals = [v for name, v in _counter_per_dispatch(os.path.join(d, sub), counter)
                if "copy" in name.lower()]
        if not vals:
            raise SystemExit(f"bench.py: no copy dispatch in {sub}")
        return cal_bytes_kib / statistics.median(vals)

    # The counter runs are `--steps 20 --warmup 2`: the first dispatch of the
    # kernel draws the draft tokens (a smaller call), the next 22 are the warmup
    # and timed steps; the calls after them (stage events, acceptance
    # statistics, the sd_t sweep) are left out.
    def kern(sub, counter):
        def wanted(name):
            if match:
                return match in name
            return f"::{kernel}<" in name or name.startswith(kernel)
        vals = [v for name, v in _counter_per_dispatch(os.path.join(d, sub), counter)
                if wanted(name)]
        return statistics.median(vals[1:23] if len(vals) > 1 else vals)

    fs, ws_ = calib("cal_fetch", "FETCH_SIZE"), calib("cal_write", "WRITE_SIZE")
    fk, wk = kern("fetch", "FETCH_SIZE"), kern("write", "WRITE_SIZE")
    hbm = (fk * fs + wk * ws_) * 1024.0
    out = {
        "kernel": kernel, "workload": workload,
        "sd_t": None if lm else
                (W.WORKLOADS[args.workload].get("sd_t") if args.sd_t is None else args.sd_t),
        "source_sha256": kernel_source_digest(kernel),
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
        "fetch_scale": fs, "write_scale": ws_, "hbm_bytes_per_launch": hbm,
        "commands": [
            f"rocprofv3 --pmc {c} --output-format csv -d <out>/{sub} -o run -- python3 bench.py "
            f"--cpu-seconds 0 --steps 20 --warmup 2 {extra}"
            for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))] + [
            f"rocprofv3 --pmc {c} --output-format csv -d <out>/{sub} -o run -- python3 bench.py "
            "--calibrate-copy" for c, sub in (("FETCH_SIZE", "cal_fetch"), ("WRITE_SIZE", "cal_write"))]
            + [f"python3 bench.py --traffic-from <out> "
               + ("--path lmhead" if lm else f"--workload {args.workload}")],
    }
    with open(traffic_file(kernel, workload), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        traffic_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences shard across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import speculative_decoding_verification_13_amd as sv

    if args.path == "lmhead":
        bench_lmhead(args, sv)
        return
    if args.path == "multi":
        bench_multi(args, sv)
        return
    w = W.make(args.workload, sd_t=args.sd_t)
    if args.top_k is not None:
        w["top_k"] = args.top_k
    if args.top_p is not None:
        w["top_p"] = args.top_p
    if args.path == "accept":
        bench_accept(args, w, sv)
        return
    # the CPU oracle first: its worker processes fork before this process uses the GPU
    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    B, V = w["B"], w["V"]
    cu = w["cu_draft"]
    n_draft = int(cu[-1])
    n_target = n_draft + B
    T, top_k, top_p = w["temperature"], w["top_k"], w["top_p"]

    # --- device-resident inputs (rotating copies) --------------------------------
    draft0 = w["draft"].to(dev)
    target0 = w["target"].to(dev)
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(dev)
    greedy_d = torch.from_numpy(w["greedy"].astype(np.uint8)).to(dev) if w["greedy"].any() else None
    uni_d = torch.from_numpy(w["uniforms"]).to(dev)

    # Draft tokens: the draft model's own draw from its rows, made by the library
    # (each draft row as a K = 0 "sequence": plain sampling with its uniform).
    zeros_cu = torch.zeros(n_draft + 1, dtype=torch.int32, device=dev)
    u_draft = torch.from_numpy(w["u_draft"]).to(dev)
    g_rows = (torch.from_numpy(W.draft_row_greedy_mask(w).astype(np.uint8)).to(dev)
              if w["greedy"].any() else None)
    tok_out, _ = sv.spec_verify_ragged(None, draft0, None, u_draft, zeros_cu, g_rows, n_draft,
                                       V, T, top_k, top_p, total_draft_rows=0)
    tokens_d = tok_out.clone()
    del zeros_cu

    sets = []
    for s in range(max(1, args.sets)):
        if s == 0:
            sets.append((draft0, target0))
        else:
            sets.append((draft0.clone(), target0.clone()))
    ws = sv.make_workspace(B, n_draft, V, top_k, top_p, dev)
    out = torch.empty(n_target, dtype=torch.int32, device=dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)

    # Dense workloads without a greedy mask go through the dense entry point (the
    # launch the full-size parity test checks); stage events need the diag one.
    dense = not w["ragged"] and greedy_d is None
    K = w["K"]
    dense_sets = [(d.view(B, K, V), t.view(B, K + 1, V)) for d, t in sets] if dense else None

    def step(k, events=None):
        if events is None and dense:
            d, t = dense_sets[k % len(sets)]
            sv.spec_verify(d, t, tokens_d.view(B, K), uni_d.view(B, K + 1), B, K, V, T, top_k,
                           top_p, out_tokens=out.view(B, K + 1), num_accepted=num, workspace=ws)
            return
        d, t = sets[k % len(sets)]
        diag = None if events is None else {"stage_events": events}
        sv.spec_verify_ragged(d, t, tokens_d, uni_d, cu_d, greedy_d, B, V, T, top_k, top_p,
                              total_draft_rows=n_draft, out_tokens=out, num_accepted=num,
                              workspace=ws, diag=diag)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # the timed steps: K calls back to back on the stream, nothing else enqueued
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    host_enqueue = time.perf_counter() - t_wall
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps

    # Host cost of the C entry point alone: the same call with its arguments
    # marshalled once (the binding's Python checks and conversions excluded).
    c_enqueue_us = None
    if dense:
        L = sv.lib()
        d, t = dense_sets[0]
        cargs = [ctypes.c_void_p(d.data_ptr()), ctypes.c_void_p(t.data_ptr()),
                 ctypes.c_void_p(tokens_d.data_ptr()), ctypes.c_void_p(uni_d.data_ptr()), B, K, V,
                 T, top_k, top_p, sv._lib.DTYPE_CODES[t.dtype], ctypes.c_void_p(out.data_ptr()),
                 ctypes.c_void_p(num.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                 ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)]
        torch.cuda.synchronize()
        t_c = time.perf_counter()
        for k in range(args.steps):
            L.spec_verify(*cargs)
        c_enqueue_us = (time.perf_counter() - t_c) / args.steps * 1e6
        torch.cuda.synchronize()

    # The same K steps again with stage events on the launch stream: before the
    # first kernel, between the kernels and after the last (HIP events without
    # the system-scope fence). They give each kernel's duration; recording them
    # lengthens a step, so the step time above is taken without them.
    nst = sv.num_stages(top_k, top_p) + 1
    hev = HipEvents(nst * args.steps)
    ev_sets = [hev.handles[nst * k:nst * (k + 1)] for k in range(args.steps)]
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(k, ev_sets[k])
    stop.record()
    torch.cuda.synchronize()
    ms_step_events = start.elapsed_time(stop) / args.steps
    per_stage = np.array([[hev.elapsed_ms(nst * k + i, nst * k + i + 1) for i in range(nst - 1)]
                          for k in range(args.steps)])
    per_call = np.array([hev.elapsed_ms(nst * k, nst * k + nst - 1) for k in range(args.steps)])
    hev.close()
    stage_ms = per_stage.mean(axis=0).tolist()
    # A step of one launch (the one-kernel path) takes that kernel's average
    # duration from the timed region's own events: K back-to-back launches on
    # the launch stream over K, which bounds the kernel's time from above and
    # carries none of the stage events' overhead. Steps of several kernels
    # take the dominant kernel's mean from the stage events.
    single = nst - 1 == 1
    k1_ms = ms_step if single else stage_ms[0]

    names = STAGES.get(nst - 1, [f"stage{i}" for i in range(nst - 1)])
    if nst - 1 == 3 and top_k <= 0:
        names = ["k_stats", "k_nucleus", "k_draw"]  # top-p alone
    dominant = names[0]
    rows = int((w["Ks"] + 1).sum())
    comp = W.compulsory_bytes(w)
    esize = target0.element_size()
    greedy = w["greedy"].astype(bool)
    algo_rows = int(((w["Ks"] + 1) + np.where(greedy, 0, w["Ks"])).sum()) if T > 0 else rows
    algo_bytes_k1 = algo_rows * V * esize
    achieved = algo_bytes_k1 / (k1_ms * 1e-3) / 1e9
    eff = comp / (ms_step * 1e-3) / 1e9

    n_acc = num.cpu().numpy()

    # The same call with the acceptance statistics as side outputs (beta per
    # draft position and the expected accepted count): the verification's row
    # statistics are reused by one more pass over the row pairs.
    beta_d = torch.empty(max(n_draft, 1), dtype=torch.float32, device=dev)[:n_draft]
    exp_d = torch.empty(B, dtype=torch.float32, device=dev)
    with_stats = None
    if T > 0 and n_draft > 0:
        def step_stats(k):
            d, t = sets[k % len(sets)]
            sv.spec_verify_ragged(d, t, tokens_d, uni_d, cu_d, greedy_d, B, V, T, top_k, top_p,
                                  total_draft_rows=n_draft, out_tokens=out, num_accepted=num,
                                  workspace=ws, diag={"beta": beta_d, "expected_accepted": exp_d})
        for k in range(args.warmup):
            step_stats(k)
        torch.cuda.synchronize()
        start.record()
        for k in range(args.steps):
            step_stats(k)
        stop.record()
        torch.cuda.synchronize()
        ms_stats = start.elapsed_time(stop) / args.steps
        with_stats = {
            "ms_per_step": ms_stats, "entry_point": "spec_verify_diag (beta, expected_accepted)",
            "passes_over_rows": 2 if top_k <= 0 and top_p >= 1.0 else 4,
            "mean_beta": float(beta_d.float().mean().cpu()),
            "mean_expected_accepted": float(exp_d.float().mean().cpu()),
        }

    # The other workloads, in the headline run only (the default command).
    others = {}
    if (args.workload == W.HEADLINE and args.sd_t is None and args.top_k is None
            and args.top_p is None and not args.no_other_configs):
        for name in OTHER_CONFIGS:
            others[name] = time_config(name, sv, dev, max(10, args.steps // 4), args.warmup)

    # The other target-perturbation settings of a swept workload (the same
    # draft rows and draft tokens, targets drawn with the other spread), each
    # timed like the headline steps.
    sweep = {}
    spec = W.WORKLOADS[args.workload]
    if args.sd_t is None and spec.get("sd_t_sweep"):
        for sd in spec["sd_t_sweep"]:
            if sd == w["sd_t"]:
                continue
            wt = W.make(args.workload, sd_t=sd)
            t_sets = [wt["target"].to(dev) for _ in range(len(sets))]
            t_dense = [t.view(B, K + 1, V) for t in t_sets] if dense else None

            def step_sd(k):
                if dense:
                    sv.spec_verify(dense_sets[k % len(sets)][0], t_dense[k % len(sets)],
                                   tokens_d.view(B, K), uni_d.view(B, K + 1), B, K, V, T, top_k,
                                   top_p, out_tokens=out.view(B, K + 1), num_accepted=num,
                                   workspace=ws)
                else:
                    sv.spec_verify_ragged(sets[k % len(sets)][0], t_sets[k % len(sets)], tokens_d,
                                          uni_d, cu_d, greedy_d, B, V, T, top_k, top_p,
                                          total_draft_rows=n_draft, out_tokens=out,
                                          num_accepted=num, workspace=ws)
            for k in range(args.warmup):
                step_sd(k)
            torch.cuda.synchronize()
            start.record()
            for k in range(args.steps):
                step_sd(k)
            stop.record()
            torch.cuda.synchronize()
            ms_sd = start.elapsed_time(stop) / args.steps
            na = num.cpu().numpy()
            sweep[str(sd)] = {
                "ms_per_step": ms_sd, "rows_per_s": rows / (ms_sd * 1e-3),
                "effective_frac_of_peak": comp / (ms_sd * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "mean_accepted": float(na.mean()),
                "all_accepted_frac": float((na == w["Ks"]).mean()),
                "errors": int((na < 0).sum()),
            }
            del t_sets, t_dense

    traffic = None
    tfile = traffic_file(dominant, args.workload)
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("source_sha256") == kernel_source_digest(tr.get("kernel")) and tr.get("workload") == args.workload \
                and args.sd_t in (None, tr.get("sd_t")):
            traffic = tr.get("hbm_bytes_per_launch")

    res = {
        "metric": METRIC,
        "value": rows / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "B": B, "K": w["K"], "V": V, "input_dtype": w["dtype"],
            "temperature": T, "top_k": top_k, "top_p": top_p, "sd_t": w["sd_t"],
            "rows_per_step": rows, "rotating_sets": len(sets),
            "entry_point": "spec_verify" if dense else "spec_verify_ragged",
        },
        "effective_GBps": eff,
        "effective_frac_of_peak": eff / PEAK_HBM_GBPS,
        "compulsory_bytes_per_step": comp,
        "roofline": {
            "kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes_k1, "avg_launch_ms": k1_ms,
            "avg_launch_from": "timed region / steps" if single else "stage events",
            "avg_launch_ms_stage_events": stage_ms[0],
        },
        "stage_ms": dict(
            zip(names, stage_ms),
            call_mean=float(per_call.mean()), call_median=float(np.median(per_call)),
            ms_per_step_with_stage_events=ms_step_events),
        "acceptance": {
            "mean_accepted": float(n_acc.mean()),
            "all_accepted_frac": float((n_acc == w["Ks"]).mean()),
            "errors": int((n_acc < 0).sum()),
        },
        "with_accept_stats": with_stats,
        "sd_t_sweep": sweep or None,
        "other_configs": others or None,
        "wall_s": wall,
        "host_enqueue_us_per_step": host_enqueue / args.steps * 1e6,
        "host_enqueue_us_per_step_c_abi": c_enqueue_us,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


_CPU = {}


# Every other logit workload, timed in the headline run so that its line
# carries them all: the small cases (C0, C1: latency-bound, report-only), the
# filtered batch and the ragged half-greedy batch.
OTHER_CONFIGS = ["tiny_f32_B4_K4_V1024", "bf16_B32_K4_V32000",
                 "f16_B256_K4_V151936_topk50_topp0.9", "bf16_B512_Kragged_V128256_halfgreedy"]


def time_config(name, sv, dev, steps, warmup):
    """One workload's verification step, timed as the headline's: inputs in HBM
    (four rotating copies when a copy fits in the 256 MB Infinity Cache), the
    draft tokens drawn by the library, K calls back to back between two events."""
    w = W.make(name)
    B, V = w["B"], w["V"]
    cu = w["cu_draft"]
    n_draft = int(cu[-1])
    n_target = n_draft + B
    T, top_k, top_p = w["temperature"], w["top_k"], w["top_p"]
    d0, t0 = w["draft"].to(dev), w["target"].to(dev)
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(dev)
    greedy_d = torch.from_numpy(w["greedy"].astype(np.uint8)).to(dev) if w["greedy"].any() else None
    uni_d = torch.from_numpy(w["uniforms"]).to(dev)
    zeros_cu = torch.zeros(n_draft + 1, dtype=torch.int32, device=dev)
    g_rows = (torch.from_numpy(W.draft_row_greedy_mask(w).astype(np.uint8)).to(dev)
              if w["greedy"].any() else None)
    tokens_d, _ = sv.spec_verify_ragged(None, d0, None, torch.from_numpy(w["u_draft"]).to(dev),
                                        zeros_cu, g_rows, n_draft, V, T, top_k, top_p,
                                        total_draft_rows=0)
    comp = W.compulsory_bytes(w)
    nsets = 1 if comp > (256 << 20) else 4
    sets = [(d0, t0)] + [(d0.clone(), t0.clone()) for _ in range(nsets - 1)]
    ws = sv.make_workspace(B, n_draft, V, top_k, top_p, dev)
    out = torch.empty(n_target, dtype=torch.int32, device=dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)

    def step(k):
        d, t = sets[k % nsets]
        sv.spec_verify_ragged(d, t, tokens_d, uni_d, cu_d, greedy_d, B, V, T, top_k, top_p,
                              total_draft_rows=n_draft, out_tokens=out, num_accepted=num,
                              workspace=ws)

    for k in range(warmup):
        step(k)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    n_acc = num.cpu().numpy()
    res = {
        "ms_per_step": ms, "rows_per_s": n_target / (ms * 1e-3),
        "effective_GBps": comp / (ms * 1e-3) / 1e9,
        "effective_frac_of_peak": comp / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "compulsory_bytes_per_step": comp, "steps": steps, "rotating_sets": nsets,
        "entry_point": "spec_verify_ragged",
        "mean_accepted": float(n_acc[n_acc >= 0].mean()) if (n_acc >= 0).any() else None,
        "errors": int((n_acc < 0).sum()),
    }
    del sets, d0, t0, ws
    torch.cuda.empty_cache()
    return res


def bench_accept(args, w, sv):
    """Acceptance statistics (pass probability per draft position, expected
    accepted drafts per sequence) on the same workload: two passes over the
    draft rows and the non-bonus target rows."""
    cu = w["cu_draft"]
    B, V = w["B"], w["V"]
    n_draft = int(cu[-1])
    T, top_k, top_p = w["temperature"], w["top_k"], w["top_p"]
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        draft, target = W.raw_numpy(w["draft"]), W.raw_numpy(w["target"])
        t0, done, b = time.perf_counter(), 0, 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            d0, d1 = int(cu[b % B]), int(cu[b % B + 1])
            oracle.acceptance_stats(draft[d0:d1], target[d0 + b % B:d1 + b % B + 1], B=1, V=V,
                                    dtype=w["dtype"], temperature=T, cu_draft=[0, d1 - d0],
                                    top_k=top_k, top_p=top_p)
            done += d1 - d0
            b += 1
        el = time.perf_counter() - t0
        cpu = {"value": done / el, "unit": "draft positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{b} sequences of the same workload one by one in {el:.1f} s, "
                         "numpy float64, one process", "cpu_model": _cpu_model()}
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    draft0, target0 = w["draft"].to(dev), w["target"].to(dev)
    sets = [(draft0, target0)] + [(draft0.clone(), target0.clone())
                                  for _ in range(max(1, args.sets) - 1)]
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(dev) if w["ragged"] else None
    ws = sv.make_workspace(B, n_draft, V, top_k, top_p, dev)
    beta = torch.empty(n_draft, dtype=torch.float32, device=dev)
    exp = torch.empty(B, dtype=torch.float32, device=dev)

    def step(k):
        d, t = sets[k % len(sets)]
        sv.spec_verify_accept_stats(d, t, cu_d, B, V, T, top_k, top_p, total_draft_rows=n_draft,
                                    beta=beta, expected_accepted=exp, workspace=ws)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    hev = HipEvents(2 * args.steps)
    stream = torch.cuda.current_stream().cuda_stream
    rec = hev.hip.hipEventRecord
    rec.argtypes = [hev.ct.c_void_p, hev.ct.c_void_p]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # per call, on the launch stream (events without the system-scope fence)
    for k in range(args.steps):
        rec(hev.handles[2 * k], stream)
        step(k)
        rec(hev.handles[2 * k + 1], stream)
    torch.cuda.synchronize()
    call_ms = float(np.mean([hev.elapsed_ms(2 * k, 2 * k + 1) for k in range(args.steps)]))
    hev.close()
    esize = target0.element_size()
    pass_bytes = 2 * n_draft * V * esize  # draft rows and their target rows
    algo = 2 * pass_bytes
    achieved = algo / (call_ms * 1e-3) / 1e9
    rec_out = {
        "metric": "acceptance statistics: draft positions/s (pass probability per position, "
                  "expected accepted drafts per sequence)",
        "value": n_draft / (ms_step * 1e-3), "unit": "draft positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "V": V, "input_dtype": w["dtype"],
                   "temperature": T, "top_k": top_k, "top_p": top_p, "sd_t": w["sd_t"],
                   "draft_positions_per_step": n_draft, "rotating_sets": len(sets),
                   "entry_point": "spec_verify_accept_stats"},
        "roofline": {"kernel": "k_stats + k_beta + k_expect (whole call)", "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": algo, "avg_launch_ms": call_ms},
        "mean_beta": float(beta.float().nanmean().item()),
        "mean_expected_accepted": float(exp.float().nanmean().item()),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec_out), flush=True)


LM_STAGES = ["gemm_stats", "merge", "decide_and_draw"]


MULTI_NAME = "multi_bf16_B64_M4_K4_V128256"
MULTI = dict(B=64, M=4, K=4, V=128256, dtype="bf16", temperature=0.7, seed=3100)


def bench_multi(args, sv):
    """Several draft chains per sequence: B=64 sequences with M=4 chains of K=4
    drafts each, V=128256 bf16, T=0.7 (the logit workloads' recipe per chain).
    A step is one spec_verify_multi call: the row statistics of every draft and
    target row, then the walk over the chains."""
    import oracle
    c = MULTI
    B, M, K, V, T = c["B"], c["M"], c["K"], c["V"], c["temperature"]
    w = W.make_multi(**c)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    draft0 = w["draft"].to(dev)
    # draft tokens: each chain's own draw from its rows (the library, K = 0)
    n_rows = B * M * K
    zeros_cu = torch.zeros(n_rows + 1, dtype=torch.int32, device=dev)
    tok, _ = sv.spec_verify_ragged(None, draft0.view(n_rows, V), None,
                                   torch.from_numpy(w["u_draft"].reshape(-1)).to(dev), zeros_cu,
                                   None, n_rows, V, T, total_draft_rows=0)
    toks = tok.cpu().numpy().reshape(B, M, K)
    target_raw = w["target"].clone()
    W.share_target_prefixes(w["target"], toks)
    target0 = w["target"].to(dev)
    tokens_d = torch.from_numpy(np.ascontiguousarray(toks, np.int32)).to(dev)
    uni_d = torch.from_numpy(w["uniforms"]).to(dev)
    sets = [(draft0, target0)] + [(draft0.clone(), target0.clone())
                                  for _ in range(max(1, args.sets) - 1)]
    n = int(sv.lib().spec_verify_multi_workspace_bytes(B, M, K, V, 0, 1.0))
    ws = sv._lib._zeroed_workspace(max(n, 256), dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)
    chain = torch.empty(B, dtype=torch.int32, device=dev)

    def step(k):
        d, t = sets[k % len(sets)]
        sv.spec_verify_multi(d, t, tokens_d, uni_d, B, M, K, V, T, out_tokens=out,
                             num_accepted=num, out_chain=chain, workspace=ws)
    for k in range(args.warmup):
        step(k)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    n_acc = num.cpu().numpy()
    comp = (B * M * K + B * M * (K + 1)) * V * target0.element_size()

    # The same chains verified with filters and greedily: draft tokens drawn
    # by the library from the filtered rows (the argmax at temperature 0), the
    # target rows of equal prefixes made equal again, each timed as above on
    # one copy of the inputs (591 MB, beyond the Infinity Cache).
    u_draft_d = torch.from_numpy(w["u_draft"].reshape(-1)).to(dev)

    def variant(temp, top_k, top_p):
        vt, _ = sv.spec_verify_ragged(None, draft0.view(n_rows, V), None, u_draft_d, zeros_cu,
                                      None, n_rows, V, temp, top_k, top_p, total_draft_rows=0)
        vtoks = vt.cpu().numpy().reshape(B, M, K)
        tgt = target_raw.clone()
        W.share_target_prefixes(tgt, vtoks)
        tgt_d = tgt.to(dev)
        vtok_d = torch.from_numpy(np.ascontiguousarray(vtoks, np.int32)).to(dev)
        vws = sv._lib._zeroed_workspace(
            max(int(sv.lib().spec_verify_multi_workspace_bytes(B, M, K, V, top_k, top_p)), 256),
            dev)

        def vstep():
            sv.spec_verify_multi(draft0, tgt_d, vtok_d, uni_d, B, M, K, V, temp, top_k, top_p,
                                 out_tokens=out, num_accepted=num, out_chain=chain, workspace=vws)
        for _ in range(args.warmup):
            vstep()
        nsteps = max(10, args.steps // 4)
        torch.cuda.synchronize()
        start.record()
        for _ in range(nsteps):
            vstep()
        stop.record()
        torch.cuda.synchronize()
        va = num.cpu().numpy()
        return {"ms_per_step": start.elapsed_time(stop) / nsteps, "steps": nsteps,
                "temperature": temp, "top_k": top_k, "top_p": top_p,
                "mean_accepted": float(va[va >= 0].mean()) if (va >= 0).any() else None,
                "errors": int((va < 0).sum())}
    variants = {"top_k50_top_p0.9": variant(T, 50, 0.9), "top_p0.9": variant(T, 0, 0.9),
                "greedy": variant(0.0, 0, 1.0)}
    cpu = None
    if args.cpu_seconds > 0:
        draft, target = W.raw_numpy(w["draft"].reshape(-1, V)), W.raw_numpy(w["target"].reshape(-1, V))
        t0, done = time.perf_counter(), 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            b = done % B
            oracle.verify_multi(draft[b * M * K:(b + 1) * M * K],
                                target[b * M * (K + 1):(b + 1) * M * (K + 1)], toks[b],
                                w["uniforms"][b], B=1, M=M, K=K, V=V, dtype=c["dtype"],
                                temperature=T)
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": done / el, "unit": "sequences/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} sequences of the same workload one by one in {el:.1f} s, "
                         "numpy float64, one process", "cpu_model": _cpu_model()}
    print(json.dumps({
        "metric": "verified sequences/sec, several draft chains per sequence",
        "value": B / (ms * 1e-3), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": MULTI_NAME, "B": B, "M": M, "K": K, "V": V,
                   "input_dtype": c["dtype"], "temperature": T, "rotating_sets": len(sets),
                   "entry_point": "spec_verify_multi"},
        "effective_GBps": comp / (ms * 1e-3) / 1e9,
        "effective_frac_of_peak": comp / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "compulsory_bytes_per_step": comp,
        "acceptance": {"mean_accepted": float(n_acc.mean()), "errors": int((n_acc < 0).sum())},
        "variants": variants,
        "cpu_baseline": cpu,
    }), flush=True)


def bench_lmhead(args, sv):
    """Verification from LM-head hidden states: the draft and target rows'
    logits formed on the matrix cores, reduced in the GEMM epilogue and
    stored, the merge of the tile partials, and the decision and draw."""
    w = W.make_lmhead()
    B, K, V, dq, dp, T = w["B"], w["K"], w["V"], w["d_draft"], w["d_target"], w["temperature"]
    s = W.LM_H_SCALE * W.LM_W_SCALE
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        t_all, done, b = 0.0, 0, 0
        while t_all < args.cpu_seconds and b < B:
            hq, hp = w["hq"][b * K:(b + 1) * K], w["hp"][b * (K + 1):(b + 1) * (K + 1)]
            lq = oracle.lmhead_logits(hq, w["wq"], s)
            toks, _ = oracle.sample_rows(lq, w["u_draft"][b * K:(b + 1) * K], V=V, dtype="f64",
                                         temperature=T)
            t0 = time.perf_counter()
            oracle.verify_lmhead(hq, w["wq"], hp, w["wp"], toks,
                                 w["uniforms"][b * (K + 1):(b + 1) * (K + 1)], B=1, K=K, V=V,
                                 temperature=T, draft_scale=s, target_scale=s)
            t_all += time.perf_counter() - t0
            done += K + 1
            b += 1
        cpu = {"value": done / t_all, "unit": "rows/s", "cores": os.cpu_count(), "kind": "oracle",
               "sample": f"{b} sequences of the same workload one by one in {t_all:.1f} s "
                         "(logits by the BLAS behind numpy on the host's cores, then the float64 "
                         "verification), draft tokens drawn outside the timed part",
               "cpu_model": _cpu_model()}
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    hq = W.lmhead_to_device(w["hq"], W.LM_H_SCALE, dev)
    wq = W.lmhead_to_device(w["wq"], W.LM_W_SCALE, dev)
    hp = W.lmhead_to_device(w["hp"], W.LM_H_SCALE, dev)
    wp = W.lmhead_to_device(w["wp"], W.LM_W_SCALE, dev)
    uni = torch.from_numpy(w["uniforms"]).to(dev)
    # Draft tokens: the draft model's own draw from its logit rows (formed here
    # in fp32, exact for these integer-valued inputs, for the input only), made
    # by the library's K = 0 call.
    n_draft = B * K
    lq = hq.float() @ wq.float().T
    zeros_cu = torch.zeros(n_draft + 1, dtype=torch.int32, device=dev)
    u_draft = torch.from_numpy(w["u_draft"]).to(dev)
    tok_out, _ = sv.spec_verify_ragged(None, lq, None, u_draft, zeros_cu, None, n_draft, V, T, 0,
                                       1.0, total_draft_rows=0)
    toks = tok_out.clone().view(B, K)
    # greedy drafting for the greedy call: each draft row's argmax (the
    # library's K = 0 call at temperature 0)
    g_out, _ = sv.spec_verify_ragged(None, lq, None, None, zeros_cu, None, n_draft, V, 0.0, 0,
                                     1.0, total_draft_rows=0)
    toks_greedy = g_out.clone().view(B, K)
    del lq, zeros_cu
    ws = sv.make_lmhead_workspace(B, K, V, dev)
    out = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    num = torch.empty(B, dtype=torch.int32, device=dev)

    def step(ev=None):
        sv.spec_verify_lmhead(hq, wq, hp, wp, toks, uni, B, K, V, T, out_tokens=out,
                              num_accepted=num, workspace=ws, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    nst = len(LM_STAGES) + 1
    hev = HipEvents(nst * args.steps)
    for k in range(args.steps):
        step(hev.handles[nst * k:nst * (k + 1)])
    torch.cuda.synchronize()
    per = np.array([[hev.elapsed_ms(nst * k + i, nst * k + i + 1) for i in range(nst - 1)]
                    for k in range(args.steps)])
    hev.close()
    stage_ms = per.mean(axis=0).tolist()
    n_sampling = num.cpu().numpy()
    # the same shape verified greedily: the target rows alone, no rows stored
    def greedy_step(ev=None):
        sv.spec_verify_lmhead(None, None, hp, wp, toks_greedy, None, B, K, V, 0.0,
                              out_tokens=out, num_accepted=num, workspace=ws, stage_events=ev)

    for _ in range(args.warmup):
        greedy_step()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        greedy_step()
    stop.record()
    torch.cuda.synchronize()
    ms_greedy = start.elapsed_time(stop) / args.steps
    hev = HipEvents(nst * args.steps)
    for k in range(args.steps):
        greedy_step(hev.handles[nst * k:nst * (k + 1)])
    torch.cuda.synchronize()
    gper = np.array([[hev.elapsed_ms(nst * k + i, nst * k + i + 1) for i in range(nst - 1)]
                     for k in range(args.steps)])
    hev.close()
    g_stage = gper.mean(axis=0).tolist()
    ng = num.cpu().numpy()
    rows = B * (K + 1)
    flops_t = 2.0 * rows * V * dp
    flops_d = 2.0 * n_draft * V * dq
    greedy = {"ms_per_step": ms_greedy, "rows_per_s": rows / (ms_greedy * 1e-3),
              "statistics_gemm_ms": g_stage[0],
              "statistics_gemm_frac_of_peak": flops_t / (g_stage[0] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
              "stage_ms": dict(zip(LM_STAGES, g_stage)),
              "mean_accepted": float(ng[ng >= 0].mean()) if (ng >= 0).any() else None,
              "errors": int((ng < 0).sum()),
              "note": "temperature 0: target rows only (argmax partials), greedy draft tokens"}
    t_ms = stage_ms[0]
    achieved = (flops_t + flops_d) / (t_ms * 1e-3) / 1e12
    weight_bytes = 2.0 * V * (dq + dp)
    n = n_sampling
    # HBM bytes per launch of the statistics GEMM from the counter record,
    # while the kernel's sources are the ones it was taken on
    lm_traffic = None
    tfile = traffic_file("k_lm_stats", W.LMHEAD_NAME)
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        if tr.get("source_sha256") == kernel_source_digest("k_lm_stats"):
            lm_traffic = tr.get("hbm_bytes_per_launch")
    rec_out = {
        "metric": f"LM-head verification ({W.LMHEAD_NAME}): verified rows/s, hidden states and "
                  "LM-head weights in",
        "value": rows / (ms_step * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": W.LMHEAD_NAME, "B": B, "K": K, "V": V, "d_draft": dq,
                   "d_target": dp, "temperature": T, "operand_dtype": "bf16",
                   "accumulate": "f32", "rows_per_step": rows,
                   "entry_point": "spec_verify_lmhead"},
        "tflops_per_step": (flops_t + flops_d) / 1e12,
        "effective_TFLOPs": (flops_t + flops_d) / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": "k_lm_stats (draft and target rows, one launch)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": lm_traffic,
                     "algorithmic_flops_per_launch": flops_t + flops_d, "avg_launch_ms": t_ms},
        "weight_bytes_per_pass": weight_bytes,
        "stage_ms": dict(zip(LM_STAGES, stage_ms)),
        "acceptance": {"mean_accepted": float(n.mean()), "errors": int((n < 0).sum())},
        "greedy": greedy,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec_out), flush=True)


def _cpu_model():
    """The host CPU's model name (as lscpu prints it), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_one(b):
    """Oracle verification of sequence b of the prepared sample (one task)."""
    import oracle
    c = _CPU
    cu = c["cu"]
    d0, d1 = int(cu[b]), int(cu[b + 1])
    t0, t1 = d0 + b, d1 + b + 1
    oracle.verify(c["draft"][d0:d1], c["target"][t0:t1], c["toks"][d0:d1], c["uniforms"][t0:t1],
                  B=1, V=c["V"], dtype=c["dtype"], cu_draft=np.array([0, d1 - d0]),
                  temperature=c["T"], top_k=c["top_k"], top_p=c["top_p"],
                  greedy=c["greedy"][b:b + 1])
    return t1 - t0


def cpu_baseline(w, budget_s):
    """The float64 oracle, as it stands, on the same workload: a third of the
    budget in this process over the first 16 sequences, the rest with every
    sequence mapped over a pool of worker processes (forked before this process
    touches the GPU). Returns the pool rate as the baseline."""
    import multiprocessing as mp

    import oracle
    B, V = w["B"], w["V"]
    cu = w["cu_draft"]
    draft = W.raw_numpy(w["draft"])
    target = W.raw_numpy(w["target"])
    toks, _ = oracle.sample_rows(draft, w["u_draft"], V=V, dtype=w["dtype"],
                                 temperature=w["temperature"], top_k=w["top_k"],
                                 top_p=w["top_p"], greedy=W.draft_row_greedy_mask(w))
    _CPU.update(draft=draft, target=target, toks=toks, uniforms=w["uniforms"], cu=cu, V=V,
                dtype=w["dtype"], T=w["temperature"], top_k=w["top_k"], top_p=w["top_p"],
                greedy=w["greedy"])
    n_one = min(B, 16)
    t0 = time.perf_counter()
    rows_one = 0
    while True:
        for b in range(n_one):
            rows_one += _cpu_one(b)
        el_one = time.perf_counter() - t0
        if el_one >= budget_s / 3:
            break
    workers = max(1, min(16, os.cpu_count() or 1))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_one, range(min(B, workers)))
        t0 = time.perf_counter()
        rows_pool = 0
        passes = 0
        while True:
            rows_pool += sum(pool.map(_cpu_one, range(B), chunksize=1))
            passes += 1
            el_pool = time.perf_counter() - t0
            if el_pool >= budget_s * 2 / 3:
                break
    return {
        "value": rows_pool / el_pool, "unit": "rows/s", "cores": workers, "kind": "oracle",
        "sample": f"all {B} sequences of the same workload, {passes} passes in {el_pool:.1f} s, "
                  f"numpy float64, sequences mapped over {workers} worker processes",
        "single_process": {"value": rows_one / el_one, "unit": "rows/s", "cores": 1,
                           "sample": f"first {n_one} sequences cycled for {el_one:.1f} s"},
        "host_cpus": os.cpu_count(),
        "cpu_model": _cpu_model(),
    }


if __name__ == "__main__":
    main()
