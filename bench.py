#!/usr/bin/env python3
"""Throughput of the state-mediated selective SSM scan on one MI355X.

One step = the whole hot path over one batch of synthetic input: the forward
chunked scan (writing the chunk-boundary states the reverse pass needs) and the
fused reverse-mode pass.  The default workload is the largest one that fits one
GPU: the HybridMamba training step (batch 2, L 16384, 32 heads, P 64, N 64 = 32
per-row-decay rows + 16 rotating pairs, rank 2, two-endpoint writes, bf16, forward
+ reverse), seeded synthetic inputs already resident in HBM.  Each timed step is
followed by a 1 GiB scratch write outside its events, so every step starts with
cold caches; the value is the median over the timed steps.

Prints ONE JSON line: metric, value (Mtokens/s; a token is one (batch, position)
across all heads), ms_per_step, the step-time percentiles and the warm-cache figure,
the roofline of the dominant kernel (timed live with HIP events on the stream the
kernels run on) and of the forward scan, the saved-for-backward and peak memory,
and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "SSM-core fwd/bwd Mtokens/s (bf16) and % of HBM/MFMA roofline on 1 MI355X"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def algorithmic_bytes(desc: dict, io_bytes: int, direction: str) -> int:
    """Compulsory HBM bytes of one launch: every input read once, every output
    written once (per-head parameters and chunk states excluded)."""
    b, L, H, G = desc["batch"], desc["seqlen"], desc["nheads"], desc["ngroups"]
    P, N, R, O = desc["headdim"], desc["dstate"], desc["rank_in"], desc["rank_out"]
    te = 1 if desc["two_endpoint"] else 0
    tok = b * L
    if direction == "fwd":
        per_h = (R * P + O * P) * io_bytes + 4 + 8 * te            # x, y, dt, beta, gamma
        per_g = (R * N + O * N) * io_bytes                          # B, C
    else:
        per_h = (2 * R * P + O * P) * io_bytes + 8 + 16 * te        # x, dx, dy, dt, ddt (+beta/gamma, grads)
        per_g = 2 * (R * N + O * N) * io_bytes                      # B, C, dB, dC
    return tok * (H * per_h + G * per_g)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ssm_fwd.hip", "ssm_bwd.hip", "ssm_device.hpp", "ssm_local.hpp", "ssm_kernels.hpp",
              "ssm_exact.hpp"):
        p = os.path.join(ROOT, "selective_diagonal_ssm_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, mode: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's reading), only if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}_{mode}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.startswith(("kernel_hash", "traffic_bytes_per_launch")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    v = rec.get(f"traffic_bytes_per_launch {kernel}")
    return int(v) if v else None


def decode_source_hash() -> str:
    p = os.path.join(ROOT, "selective_diagonal_ssm_amd", "csrc", "ssm_decode.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16] if os.path.exists(p) else ""


def measured_decode_traffic(workload: str):
    """HBM bytes per recurrent step from the committed rocprofv3 summary of that workload,
    only if it was taken on the current recurrent-step source; else None."""
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}_decode.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.startswith(("decode_kernel_hash", "traffic_bytes_per_launch")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("decode_kernel_hash") != decode_source_hash():
        return None
    v = rec.get("traffic_bytes_per_launch ssm_decode_kernel")
    return int(v) if v else None


def decode_bytes(desc: dict, io_bytes: int) -> int:
    """Compulsory HBM bytes of one recurrent step over all slices: the fp32 state
    read and written once, plus x, x_prev, y, B, B_prev, C and the per-slice scalars."""
    b, H, G = desc["batch"], desc["nheads"], desc["ngroups"]
    P, N, R, O = desc["headdim"], desc["dstate"], desc["rank_in"], desc["rank_out"]
    te = 1 if desc["two_endpoint"] else 0
    per_h = 2 * N * P * 4 + ((1 + te) * R * P + O * P) * io_bytes + 4 + 8 * te
    per_g = ((1 + te) * R * N + O * N) * io_bytes
    return b * (H * per_h + G * per_g)


def cpu_baseline(prob: dict, mode: str, target_s: float = 15.0, h0=None):
    import oracle

    oracle.build(force=False)
    d = prob["desc"]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    all_slices = [(b, h) for b in range(d["batch"]) for h in range(d["nheads"])]

    def run(sl):
        t0 = time.perf_counter()
        oracle.fwd(prob, slices=sl, h0=h0)
        if mode == "fwdbwd":
            oracle.bwd(prob, prob["dy"], slices=sl)
        return time.perf_counter() - t0

    k = min(len(all_slices), threads)
    t_cal = run(all_slices[:k])
    k2 = int(min(len(all_slices), max(k, k * target_s / max(t_cal, 1e-3))))
    k2 = max(threads, (k2 // threads) * threads) if k2 >= threads else k2
    k2 = min(k2, len(all_slices))
    sample = all_slices[:k2]
    # a whole-workload pass that is short is repeated up to ~2/3 of the target time
    reps, t = 0, 0.0
    while reps == 0 or (k2 == len(all_slices) and t < target_s * 2 / 3 and reps < 64):
        t += run(sample)
        reps += 1
    tokens = reps * k2 * d["seqlen"] / d["nheads"]  # (batch, position) tokens across all heads
    return {"value": tokens / t / 1e6, "unit": "Mtokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{k2} of {len(all_slices)} (batch, head) slices x {reps} pass(es), full "
                      f"length {d['seqlen']}, "
                      f"{ {'fwdbwd': 'forward + reverse', 'fwd': 'forward'}.get(mode, 'recurrent steps')}"
                      f", fp64, {t:.1f} s"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


FLUSH_BYTES = 1 << 30  # scratch written between timed steps: beyond L2 and the 256 MB cache


def pct(v, q):
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hybrid_bwd", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--mode", default="fwdbwd", choices=["fwd", "fwdbwd", "decode"])
    ap.add_argument("--decode-batch", type=int, default=256,
                    help="batch of the recurrent-step measurement (--mode decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="time back-to-back steps with no scratch write between them "
                         "(warm caches; not the reported number)")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload (forward for the forward workloads, forward + "
                         "reverse for the backward ones) and print their geometric means")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for HBM counter scaling)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch

        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(every (batch, head) slice is independent; see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)

    if args.mode == "decode":
        run_decode(args)
        return
    if args.suite:
        run_suite(args)
        return
    out = measure(args.workload, args.mode, args.steps, args.warmup, flush=not args.no_flush,
                  cpu=not args.no_cpu_baseline)
    print(json.dumps(out), flush=True)


def measure(workload: str, mode: str, steps: int, warmup: int, flush: bool = True,
            cpu: bool = True) -> dict:
    """One bench line for `workload`: `steps` timed steps (forward, or forward + reverse),
    each followed by a write of FLUSH_BYTES of scratch outside its events."""
    import torch

    import selective_diagonal_ssm_amd as ssm

    prob = workloads.make_problem(workload, seed=0, with_dy=(mode == "fwdbwd"))
    d = prob["desc"]
    io = prob["dtype"]
    torch.cuda.reset_peak_memory_stats()
    t = workloads.to_device(prob)
    chunk = prob.get("chunk", 0)
    desc = ssm.make_desc(d, io, chunk)
    dev = t["x"].device
    y = torch.empty((d["batch"], d["seqlen"], d["nheads"], d["rank_out"], d["headdim"]),
                    dtype=t["x"].dtype, device=dev)
    saved = None
    grads = {}
    saved_bytes = ssm.saved_bytes(desc) if mode == "fwdbwd" else 0
    if mode == "fwdbwd":
        saved = torch.empty((saved_bytes + 3) // 4, dtype=torch.float32, device=dev)
        grads = {"dx": torch.empty_like(t["x"]), "dB": torch.empty_like(t["B"]),
                 "dC": torch.empty_like(t["C"]), "ddt": torch.empty_like(t["dt"]),
                 "dA": torch.empty_like(t["A"])}
        if d["n_pairs"]:
            grads["domega"] = torch.empty_like(t["omega"])
        if d["two_endpoint"]:
            grads["dbeta"] = torch.empty_like(t["dt"])
            grads["dgamma"] = torch.empty_like(t["dt"])
        if d["has_D"]:
            grads["dD"] = torch.empty_like(t["D"])
    ws_f = ssm.workspace_bytes(desc, False)
    ws_b = ssm.workspace_bytes(desc, True) if mode == "fwdbwd" else 0
    ws = torch.empty(max(ws_f, ws_b, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd(events=None):
        ssm.scan_fwd(desc, t["x"], t["B"], t["C"], t["dt"], t["A"], y, omega=t.get("omega"),
                     beta=t.get("beta"), gamma=t.get("gamma"), D=t.get("D"), saved=saved, ws=ws,
                     stream=stream, events=events)

    def bwd(events=None):
        ssm.scan_bwd(desc, t["x"], t["B"], t["C"], t["dy"], t["dt"], t["A"], saved, grads["dx"],
                     grads["dB"], grads["dC"], grads["ddt"], omega=t.get("omega"),
                     beta=t.get("beta"), gamma=t.get("gamma"), D=t.get("D"), dA=grads.get("dA"),
                     domega=grads.get("domega"), dbeta=grads.get("dbeta"),
                     dgamma=grads.get("dgamma"), dD=grads.get("dD"), ws=ws, stream=stream,
                     events=events)

    for _ in range(warmup):
        fwd()
        if mode == "fwdbwd":
            bwd()
    torch.cuda.synchronize()
    # M3: every buffer of the step is allocated and one step has run
    peak_bytes = torch.cuda.max_memory_allocated()
    input_bytes = sum(v.numel() * v.element_size() for k, v in t.items() if k != "dy")
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if flush else None

    # HIP events recorded by the library on the stream the kernels run on.  Each
    # record costs GPU time between kernels, so the per-kernel breakdown comes from a
    # pass of its own (events around every kernel); the timed region records events
    # around each step and around the dominant kernel of that breakdown only.
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # event slots: forward (0, 1); reverse pass: adjoints (0, 1), chunk gradients
    # (1, 2), parameter sums (2, 3)
    slots = {"ssm_fwd_kernel": ("f", 0, 1), "ssm_bwd_adjoint": ("b", 0, 1),
             "ssm_bwd_chunk": ("b", 1, 2), "ssm_bwd_params": ("b", 2, 3)}

    def run(steps, which=None, flush_between=True):
        """`steps` steps with events around each step and around every kernel
        (which=None) or one kernel only; a scratch write follows each step, outside its
        events.  Returns (per-step ms list, per-kernel per-step ms lists)."""
        evf = [[mk() for _ in range(2)] for _ in range(steps)]
        evb = [[mk() for _ in range(4)] for _ in range(steps)]
        evs = [[mk(), mk()] for _ in range(steps)]
        for e in [e for row in evf + evb + evs for e in row]:
            e.record(stream)  # materialize the handles
        torch.cuda.synchronize()
        args_f, args_b = [], []
        for k in range(steps):
            if which is None:
                args_f.append(evf[k])
                args_b.append(evb[k])
            else:
                side, i, j = slots[which]
                row = evf[k] if side == "f" else evb[k]
                sel = [e if n in (i, j) else None for n, e in enumerate(row)]
                args_f.append(sel if side == "f" else None)
                args_b.append(sel if side == "b" else None)
        for k in range(steps):
            if scratch is not None and flush_between:
                scratch.fill_(float(k))  # evicts L2 and the Infinity Cache
            evs[k][0].record(stream)
            fwd(args_f[k])
            if mode == "fwdbwd":
                bwd(args_b[k])
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        names = [which] if which else (list(slots) if mode == "fwdbwd" else ["ssm_fwd_kernel"])
        per = {}
        for n in names:
            side, i, j = slots[n]
            rows = evf if side == "f" else evb
            per[n] = [r[i].elapsed_time(r[j]) for r in rows]
        return [a.elapsed_time(b) for a, b in evs], per

    _, kern = run(min(steps, 10))                   # breakdown pass (untimed)
    kern_ms = {k: float(np.median(v)) for k, v in kern.items()}
    dominant = max(kern_ms, key=kern_ms.get)
    warm_steps, _ = run(min(steps, 10), dominant, flush_between=False)  # warm caches
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_ms, timed = run(steps, dominant)           # the timed region
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = float(np.median(step_ms))
    tokens = d["batch"] * d["seqlen"]
    value = tokens / (ms_per_step * 1e-3) / 1e6

    io_bytes = 2 if io == "bf16" else 4
    # the dominant kernel; the compulsory bytes of a direction are carried by its
    # main kernel (the reverse pass's chunk-gradient kernel reads every input and
    # writes every gradient; its boundary-adjoint and parameter kernels are overhead)
    kms = float(np.mean(timed[dominant]))  # its mean launch duration over the timed region
    direction = "fwd" if dominant == "ssm_fwd_kernel" else "bwd"
    abytes = algorithmic_bytes(d, io_bytes, direction) if dominant in ("ssm_fwd_kernel",
                                                                       "ssm_bwd_chunk") else 0
    achieved = abytes / (kms * 1e-3) / 1e9
    traffic = measured_traffic(dominant, workload, mode)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dominant, "algorithmic_bytes_per_launch": abytes,
                "avg_launch_ms": round(kms, 4)}
    fwd_ms = kern_ms["ssm_fwd_kernel"]
    fwd_bytes = algorithmic_bytes(d, io_bytes, "fwd")
    fwd_ach = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    roofline_fwd = {"bound": "hbm", "achieved": round(fwd_ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(fwd_ach / HBM_PEAK_GBS, 4),
                    "kernel": "forward scan (every forward launch)" +
                              (", writing the chunk-boundary states" if mode == "fwdbwd" else ""),
                    "algorithmic_bytes_per_launch": fwd_bytes, "median_launch_ms": round(fwd_ms, 4)}
    bwd_ms = sum(v for k, v in kern_ms.items() if k.startswith("ssm_bwd"))

    cpu_line = None
    if cpu:
        cpu_line = cpu_baseline(prob, mode)
        cpu_line["cpu_model"] = cpu_model()

    return {
        "metric": METRIC, "value": round(value, 3), "unit": "Mtokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if io == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": workload, "batch": d["batch"], "seq_len": d["seqlen"],
                   "nheads": d["nheads"], "headdim": d["headdim"], "dstate": d["dstate"],
                   "rank": d["rank_in"], "decay": d["decay_mode"], "n_real": d["n_real"],
                   "n_pairs": d["n_pairs"], "two_endpoint": d["two_endpoint"],
                   "chunk": ssm.chunk_tokens(desc),
                   "step": "forward + reverse" if mode == "fwdbwd" else "forward"},
        "timing": {"statistic": "median over the timed steps", "flush_bytes_between_steps":
                   FLUSH_BYTES if flush else 0,
                   "step_ms_p10": round(pct(step_ms, 10), 4),
                   "step_ms_p50": round(ms_per_step, 4),
                   "step_ms_p90": round(pct(step_ms, 90), 4),
                   "step_ms_mean": round(float(np.mean(step_ms)), 4),
                   "warm_cache_step_ms_median": round(float(np.median(warm_steps)), 4),
                   "wall_s": round(wall, 3)},
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
        "cpu_baseline": cpu_line,
        # M3: saved-for-backward bytes against the peak device allocation of the step
        "memory": {"saved_for_backward_bytes": saved_bytes,
                   "workspace_bytes": {"fwd": ws_f, "bwd": ws_b},
                   "input_bytes": input_bytes,
                   "peak_allocated_bytes": int(peak_bytes)},
        # per-kernel medians from the untimed pass with events around every kernel
        "breakdown": {"kernel_ms": {k: round(v, 4) for k, v in kern_ms.items()},
                      "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                      "fwd_mtok_s": round(tokens / (fwd_ms * 1e-3) / 1e6, 3)},
    }


SUITE = [("ssd_siso", "fwd"), ("ssd_mimo", "fwd"), ("hybrid", "fwd"), ("hybrid_r1", "fwd"),
         ("hybrid_bwd", "fwdbwd"), ("ssd_mimo_bwd", "fwdbwd")]


def run_suite(args):
    """Every workload once, then geometric means over them (the pages aggregate their
    per-workload kernel timings by geometric mean)."""
    lines = []
    for w, m in SUITE:
        o = measure(w, m, args.steps, args.warmup, flush=not args.no_flush, cpu=False)
        lines.append({"workload": w, "step": o["config"]["step"], "mtok_s": o["value"],
                      "ms_per_step": o["ms_per_step"], "fwd_hbm_frac": o["roofline_fwd"]["frac"],
                      "dominant_kernel": o["roofline"]["kernel"],
                      "dominant_hbm_frac": o["roofline"]["frac"]})
        print(json.dumps(lines[-1]), file=sys.stderr, flush=True)
        import torch
        torch.cuda.empty_cache()

    def gmean(k):
        return round(float(np.exp(np.mean([np.log(x[k]) for x in lines]))), 4)

    print(json.dumps({"metric": "geometric mean over the workloads", "workloads": lines,
                      "geomean_mtok_s": gmean("mtok_s"),
                      "geomean_fwd_hbm_frac": gmean("fwd_hbm_frac"),
                      "geomean_dominant_hbm_frac": gmean("dominant_hbm_frac")}), flush=True)


def run_decode(args):
    """Recurrent-step throughput: one step = one token of every (batch, head) slice
    of a serving batch, the fp32 state updated in place in HBM (token 1 of a
    two-token draw, token 0 serving as the previous token of two-endpoint writes)."""
    import torch

    from selective_diagonal_ssm_amd import _lib

    prob = workloads.make_problem(workloads.spec(args.workload, seqlen=2,
                                                 batch=args.decode_batch), seed=0, with_dy=False)
    d = prob["desc"]
    io = prob["dtype"]
    h0 = workloads.make_state(d, seed=1)
    t = workloads.to_device(prob)
    te = d["two_endpoint"]
    tok = {k: t[k][:, 1].contiguous() for k in ("x", "B", "C", "dt")}
    for k in ("beta", "gamma"):
        if t.get(k) is not None:
            tok[k] = t[k][:, 1].contiguous()
    xp = t["x"][:, 0].contiguous() if te else None
    bp = t["B"][:, 0].contiguous() if te else None
    state = torch.from_numpy(h0).cuda()
    dd = dict(d, seqlen=1)
    desc = _lib.make_desc(dd, io, 0)
    y = torch.empty((d["batch"], d["nheads"], d["rank_out"], d["headdim"]), dtype=t["x"].dtype,
                    device=t["x"].device)
    stream = torch.cuda.current_stream()

    def step():
        _lib.decode_step(desc, tok["x"], tok["B"], tok["C"], tok["dt"], t["A"], state, y,
                         omega=t.get("omega"), beta=tok.get("beta"), gamma=tok.get("gamma"),
                         D=t.get("D"), x_prev=xp, B_prev=bp, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # a state of a few hundred MB fits the 256 MB Infinity Cache partly: unless --no-flush,
    # 1 GiB of scratch is written between steps, outside their events
    scratch = (None if args.no_flush else
               torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=state.device))

    def timed(n, flush):
        ev = [[mk(), mk()] for _ in range(n)]
        for k in range(n):
            if flush and scratch is not None:
                scratch.fill_(float(k))
            ev[k][0].record(stream)
            step()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    warm = timed(min(args.steps, 10), False)
    wall0 = time.perf_counter()
    per_step = timed(args.steps, True)
    wall = time.perf_counter() - wall0
    ms_per_step = float(np.median(per_step))
    kms = ms_per_step
    io_bytes = 2 if io == "bf16" else 4
    abytes = decode_bytes(dd, io_bytes)
    achieved = abytes / (kms * 1e-3) / 1e9
    value = d["batch"] / (ms_per_step * 1e-3) / 1e6
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_decode_traffic(args.workload),
                "kernel": "ssm_decode_kernel", "algorithmic_bytes_per_launch": abytes,
                "avg_launch_ms": round(kms, 4)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob, "decode", h0=h0.astype(np.float64))
    out = {
        "metric": "SSM recurrent step Mtokens/s on 1 MI355X", "value": round(value, 3),
        "unit": "Mtokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if io == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload} recurrent step", "batch": d["batch"],
                   "nheads": d["nheads"], "headdim": d["headdim"], "dstate": d["dstate"],
                   "rank": d["rank_in"], "decay": d["decay_mode"], "n_pairs": d["n_pairs"],
                   "two_endpoint": te, "step": "one token per (batch, head) slice"},
        "roofline": roofline, "cpu_baseline": cpu, "breakdown": {"wall_s": round(wall, 3)},
        "timing": {"statistic": "median over the timed steps",
                   "flush_bytes_between_steps": 0 if args.no_flush else FLUSH_BYTES,
                   "step_ms_p10": round(float(np.percentile(per_step, 10)), 5),
                   "step_ms_p90": round(float(np.percentile(per_step, 90)), 5),
                   "warm_cache_step_ms_median": round(float(np.median(warm)), 5),
                   "state_bytes": int(state.numel() * 4)},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
