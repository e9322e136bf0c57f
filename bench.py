#!/usr/bin/env python3
"""Benchmark of the MoE forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_512]

A step is one complete forward pass (route, histogram/scan/schedule,
reorder+gather, fused gate/up SwiGLU GEMM, down GEMM, weighted combination)
over one batch of seeded synthetic inputs already resident in HBM.  W
untimed steps, then K timed steps between two device synchronisations.
Prints ONE JSON line.

``value`` = tokens/s of the whole job.  ``roofline`` covers the dominant
kernel (the fused gate/up GEMM): its algorithmic bytes per launch divided by
its mean duration, measured with HIP events recorded on the stream the
library launches on, against 8 TB/s.  ``cpu_baseline`` times the CPU oracle
(test infrastructure, imported only for this leg) on a bounded sample of the
same workload on this host's cores.

Other modes (not used by the default run):
  --profile            few steps, no CPU baseline (for rocprofv3 runs)
  --copy-bytes N       also run one plain N-byte device copy per step (the
                       calibration kernel of the HBM byte counters)
  --traffic FETCH_DIR WRITE_DIR
                       turn two `rocprofv3 --pmc FETCH_SIZE` / `--pmc
                       WRITE_SIZE` output folders into profiles/traffic_*.json
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE fwd tokens/s + TFLOP/s, HBM GB/s (% roofline) at T=128-512, 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DOMINANT = "grouped_gemm_kernel<...SWIGLU>"   # K4, the fused gate/up SwiGLU GEMM
GEMM_SRC = os.path.join(ROOT, "expert_dispatch_router_amd", "csrc", "grouped_gemm.hip")
STAGES = ["route", "hist_scan_schedule", "reorder_gather", "gate_up_swiglu", "down", "combine"]


def source_sha(path=GEMM_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def algorithmic(cfg, counts):
    """Algorithmic work of one forward pass (what the method must move and
    compute, not what an implementation happens to re-read).
      FLOP  = 6 * A * F * d        (gate, up and down products)
      bytes = 6*F*d per active expert (bf16 weights, read once)
              + 2*T*d (x) + 4*T*E (logits) + 2*T*d (out)
              + 4*A*F (h, bf16, written once and read once)
    The fused gate/up kernel alone: 4*F*d per active expert + 2*A*d (its
    activation rows) + 2*A*F (h written)."""
    T, d, F, E, k = cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k
    A = T * k
    e_act = int((counts > 0).sum())
    flop = 6.0 * A * F * d
    bytes_all = e_act * 6.0 * F * d + 2.0 * T * d + 4.0 * T * E + 2.0 * T * d + 4.0 * A * F
    bytes_k4 = e_act * 4.0 * F * d + 2.0 * A * d + 2.0 * A * F
    flop_k4 = 4.0 * A * F * d
    return dict(A=A, e_act=e_act, flop=flop, bytes=bytes_all, bytes_k4=bytes_k4, flop_k4=flop_k4)


def router_gemm(cfg, x, seed, steps, stream):
    """The router scores x . W_r^T (moe_router_logits), the step upstream of
    the timed path, timed on its own: mean kernel time over ``steps`` calls
    bracketed by events on the launch stream, against its algorithmic bytes
    (x, W_r and the scores, each moved once)."""
    import torch

    import expert_dispatch_router_amd as moe
    from expert_dispatch_router_amd import synth

    wr = synth.make_router_weight(cfg, seed, x.device)
    lg = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=x.device)
    for _ in range(3):
        moe.moe_router_logits(x, wr, out=lg, stream=stream)
    ev = [(moe.Timer(), moe.Timer()) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        moe.moe_router_logits(x, wr, out=lg, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_ms(b) for a, b in ev) / steps
    nbytes = 2.0 * cfg.T * cfg.d + 2.0 * cfg.E * cfg.d + 4.0 * cfg.T * cfg.E
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "router_logits (moe_router_logits, upstream of the timed step)",
            "mean_launch_ms": ms, "alg_bytes_per_launch": nbytes, "achieved": gbs,
            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}


def graph_replay(step, steps, T):
    """The same pass captured once in a HIP graph and replayed `steps`
    times (no host launch work per pass): ms per pass and tokens/s."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(strm=side)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(strm=torch.cuda.current_stream())
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3)}


def traffic_for(cfg_name):
    """Counter-derived HBM bytes per launch of the fused kernel, if the
    stored measurement was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_gate_up_swiglu_{cfg_name}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("source_sha256_16") != source_sha():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(cfg, x, logits, wgu, wd, target_s=10.0):
    """The oracle as it stands, timed on this host on a bounded sample:
    routing of all T tokens plus the expert FFN of the first n tokens,
    n chosen from a one-token-per-thread calibration run to take ~target_s."""
    import numpy as np
    import oracle
    from expert_dispatch_router_amd.synth import bf16_bits

    lg = logits.detach().cpu().numpy()
    xb = bf16_bits(x)
    ids, w = oracle.route(lg, cfg.top_k, cfg.score, cfg.renormalize)
    used = sorted(set(int(e) for e in ids.reshape(-1)))
    gu = [None] * cfg.E
    dn = [None] * cfg.E
    for e in used:
        gu[e] = bf16_bits(wgu[e])
        dn[e] = bf16_bits(wd[e])
    threads = oracle.max_threads()
    n0 = min(cfg.T, threads)
    t0 = time.perf_counter()
    oracle.ffn(xb, ids, w, gu, dn, cfg.ffn, tokens=np.arange(n0, dtype=np.int32))
    cal = time.perf_counter() - t0
    per_round = max(cal, 1e-6)
    rounds = max(1, int(target_s / per_round))
    n = min(cfg.T, n0 * rounds)
    toks = np.arange(n, dtype=np.int32)
    t0 = time.perf_counter()
    ids2, w2 = oracle.route(lg, cfg.top_k, cfg.score, cfg.renormalize)
    counts, offsets = oracle.counts_offsets(ids2, cfg.E)
    perm, inv = oracle.permute(ids2, cfg.E, offsets)
    oracle.ffn(xb, ids2, w2, gu, dn, cfg.ffn, tokens=toks)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"routing of all {cfg.T} tokens + expert FFN and combination of the "
                      f"first {n} of {cfg.T} tokens ({dt:.1f} s)"}


_SINGLE_THREAD_TINY = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import oracle
from expert_dispatch_router_amd import synth
oracle.set_threads(1)
cfg = synth.CONFIGS["tiny"]
x, lg, wgu, wd = synth.make_inputs(cfg, 0, "cpu")
xb, lgn = synth.bf16_bits(x), lg.numpy()
gu, dn = synth.bf16_bits(wgu), synth.bf16_bits(wd)
passes, t0 = 0, time.perf_counter()
while time.perf_counter() - t0 < 2.0:
    oracle.forward(xb, lgn, gu, dn, cfg.top_k, cfg.renormalize, cfg.score, cfg.ffn)
    passes += 1
dt = time.perf_counter() - t0
print(json.dumps({"value": cfg.T * passes / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
                  "kind": "oracle", "sample": f"{passes} whole tiny passes (T={cfg.T}) in {dt:.1f} s"}))
"""


def cpu_single_thread_tiny():
    """The oracle on the whole tiny workload with one OpenMP thread asked
    for, in a child process (so the parent's oracle keeps all its threads);
    ``cores`` reports the threads OpenMP actually granted, which an
    environment may hold above one."""
    import subprocess

    r = subprocess.run([sys.executable, "-c", _SINGLE_THREAD_TINY, ROOT],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1:] or ["failed"]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def run(args):
    import numpy as np
    import torch

    import expert_dispatch_router_amd as moe
    from expert_dispatch_router_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, logits, wgu, wd = synth.make_inputs(cfg, args.seed, dev)
    unfused = 1 if args.unfused else 0
    bm, split, fused_down = moe.moe_plan(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k,
                                         unfused_swiglu=unfused, with_fusion=True)
    out = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.moe_workspace_size(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k,
                                            unfused_swiglu=unfused),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    copy_src = copy_dst = None
    if args.copy_bytes:
        copy_src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
        copy_dst = torch.empty_like(copy_src)

    routing = moe.moe_route(logits, cfg.top_k, cfg.renormalize, cfg.score)
    counts = routing["counts"].cpu().numpy()
    alg = algorithmic(cfg, counts)
    if fused_down:
        # one kernel streams the gate/up and the down weights
        alg["bytes_k4"] = alg["e_act"] * 6.0 * cfg.ffn * cfg.d + 2.0 * alg["A"] * cfg.d

    def step(events=None, strm=None):
        moe.moe_forward(x, logits, wgu, wd, cfg.top_k, cfg.renormalize, out=out, score=cfg.score,
                        workspace=ws, stream=strm or stream, stage_events=events,
                        unfused_swiglu=unfused)
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    for _ in range(args.warmup):
        step()
    # Timed region: the fused gate/up GEMM (the dominant kernel) is bracketed
    # by two events on the library's stream in every step (stage points 3, 4).
    k4_timers = [(moe.Timer(), moe.Timer()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        a, b = k4_timers[i]
        step([None, None, None, a.handle, b.handle, None, None])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_step = elapsed * 1e3 / args.steps
    k4_each = np.array([a.elapsed_ms(b) for a, b in k4_timers])
    k4_ms = float(k4_each.mean())
    # Stage breakdown: a second, separately run set of steps with all seven
    # stage events (each event adds a little time of its own).
    timers = [[moe.Timer() for _ in range(7)] for _ in range(args.steps)]
    for i in range(args.steps):
        step([t.handle for t in timers[i]])
    torch.cuda.synchronize()
    stage_ms = np.zeros(6)
    for i in range(args.steps):
        for s in range(6):
            stage_ms[s] += timers[i][s].elapsed_ms(timers[i][s + 1])
    stage_ms /= args.steps
    pass_each = np.array([timers[i][0].elapsed_ms(timers[i][6]) for i in range(args.steps)])
    pct = lambda v: {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
                     "p90": float(np.percentile(v, 90))}

    t_step = elapsed / args.steps
    t_roof = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9), alg["flop"] / (BF16_PEAK_TFLOPS * 1e12))
    k4_s = k4_ms * 1e-3
    achieved = alg["bytes_k4"] / k4_s / 1e9
    k4_flop = alg["flop"] if fused_down else alg["flop_k4"]
    res = {
        "metric": METRIC,
        "value": cfg.T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: MoE layer T={cfg.T} d={cfg.d} ffn={cfg.ffn} "
                               f"E={cfg.E} top-{cfg.top_k} "
                               f"{'sigmoid' if cfg.score else 'softmax'}"
                               f"{' renormalised' if cfg.renormalize else ''}",
                   "tokens": cfg.T, "hidden": cfg.d, "ffn": cfg.ffn, "experts": cfg.E,
                   "top_k": cfg.top_k, "block_rows": bm, "split_k": split,
                   "active_experts": alg["e_act"], "seed": args.seed,
                   "swiglu": "unfused ablation" if unfused else "fused",
                   "down_projection": "in the gate/up GEMM" if fused_down else "own GEMM"},
        "tflops": alg["flop"] / t_step / 1e12,
        "hbm_gbs": alg["bytes"] / t_step / 1e9,
        "roofline_frac_step": t_roof / t_step,
        "stage_ms": {n: round(float(v), 5) for n, v in zip(STAGES, stage_ms)},
        # distributions: the fused kernel over the timed steps; the whole
        # pass (first to last stage event) over the stage-breakdown steps
        "k4_ms_pct": pct(k4_each),
        "pass_ms_pct": pct(pass_each),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if (unfused or fused_down) else traffic_for(cfg.name),
                     "kernel": ("gate/up stage of the unfused ablation (gate GEMM + up GEMM + "
                                "activation)") if unfused else
                               ("gate_up_swiglu_down (fused gate/up SwiGLU grouped GEMM with "
                                "the down projection in its epilogue)") if fused_down else
                               "gate_up_swiglu (fused gate/up SwiGLU grouped GEMM)",
                     "alg_bytes_per_launch": alg["bytes_k4"],
                     "mean_launch_ms": float(k4_ms)},
        # the same kernel against the bf16 dense MFMA peak (its FLOPs over its
        # mean duration): the hot experts of skewed routing are locally
        # MFMA-bound even where the launch as a whole is HBM-bound
        "k4_mfma": {"achieved": k4_flop / k4_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": k4_flop / k4_s / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    res["router_gemm"] = router_gemm(cfg, x, args.seed, args.steps, stream)
    if args.graph:
        res["graph"] = graph_replay(step, args.steps, cfg.T)
    if not args.profile and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, x, logits, wgu, wd, args.cpu_seconds)
        res["cpu_baseline"]["tiny_one_thread_requested"] = cpu_single_thread_tiny()
    print(json.dumps(res), flush=True)


def summarize_traffic(fetch_dir, write_dir, workload, copy_bytes,
                      out_dir=os.path.join(ROOT, "profiles")):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMM-stage kernels,
    scaled by what the same counters read for the plain copy of copy_bytes
    bytes (reads copy_bytes, writes copy_bytes).  Writes
    profiles/traffic_gate_up_swiglu_<workload>.json for the fused kernel, or
    profiles/traffic_unfused_swiglu_<workload>.json when the run used the
    unfused ablation (gate GEMM, up GEMM, activation kernel)."""
    import csv
    import re

    def load(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        if not rows:
            raise SystemExit(f"no {counter} rows under {d}")
        return rows

    def mode(name):  # output mode of a grouped GEMM instantiation (its fifth template argument)
        m = re.search(r"(?:grouped_gemm_kernel|gemm_lds_kernel)<((?:\d+, )*\d+)>", name)
        if not m:
            return None
        args = [int(a) for a in m.group(1).split(", ")]
        return args[4] if len(args) > 4 else None

    classes = {
        "gate_up_swiglu": lambda n: mode(n) == 0,
        "down": lambda n: mode(n) in (1, 4),   # fp32 parts: 32 or 64 columns per wave
        "proj_bf16": lambda n: mode(n) == 2,
        "swiglu_act": lambda n: "swiglu_act_kernel" in n,
    }
    is_copy = lambda n: "copyBuffer" in n
    f = load(fetch_dir, "FETCH_SIZE")
    w = load(write_dir, "WRITE_SIZE")

    # the calibration copies are the copyBuffer dispatches of copy_bytes: the
    # largest ones (other copies of a run move a few KiB)
    def big_copies(rows):
        vals = sorted((v for n, v in rows if is_copy(n)), reverse=True)
        top = [v for v in vals if v >= 0.25 * vals[0]]
        return sum(top) / len(top), len(top)
    fcp, ncf = big_copies(f)
    wcp, ncw = big_copies(w)
    f_scale = copy_bytes / (fcp * 1024.0)
    w_scale = copy_bytes / (wcp * 1024.0)
    per = {}
    for cname, pred in classes.items():
        fv = [v for n, v in f if pred(n)]
        wv = [v for n, v in w if pred(n)]
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        per[cname] = {"fetch_kib_per_launch": fk, "write_kib_per_launch": wk,
                      "launches": [len(fv), len(wv)],
                      "bytes_per_launch": fk * 1024.0 * f_scale + wk * 1024.0 * w_scale}
    unfused = "proj_bf16" in per
    out = {"workload": workload, "source_sha256_16": source_sha(), "copy_bytes": copy_bytes,
           "copy_fetch_kib": fcp, "copy_write_kib": wcp, "copies": [ncf, ncw],
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": per}
    if unfused:
        # per forward pass: two projections and one activation kernel
        out["kernel"] = "unfused_swiglu (gate GEMM + up GEMM + activation)"
        out["bytes_per_forward"] = 2 * per["proj_bf16"]["bytes_per_launch"] + \
            per["swiglu_act"]["bytes_per_launch"]
        path = os.path.join(out_dir, f"traffic_unfused_swiglu_{workload}.json")
    else:
        out["kernel"] = "gate_up_swiglu"
        out["bytes_per_launch"] = per["gate_up_swiglu"]["bytes_per_launch"]
        path = os.path.join(out_dir, f"traffic_gate_up_swiglu_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks settle within ~20 forward passes of sustained load
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="mixtral_512")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--graph", action="store_true",
                    help="also time the pass captured in a HIP graph and replayed")
    ap.add_argument("--unfused", action="store_true",
                    help="SwiGLU ablation: gate GEMM, up GEMM and activation kernel")
    args = ap.parse_args()
    if args.traffic:
        summarize_traffic(args.traffic[0], args.traffic[1], args.workload,
                          args.copy_bytes or (1 << 30))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        raise SystemExit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("1", ""):
        raise SystemExit("one GPU only: run without torch.distributed")
    run(args)


if __name__ == "__main__":
    main()
