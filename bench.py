#!/usr/bin/env python3
"""Benchmark of the MoE forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_512]

A step is one complete forward pass (route, histogram/scan/schedule,
reorder+gather, fused gate/up SwiGLU GEMM, down GEMM, weighted combination)
over one batch of seeded synthetic inputs already resident in HBM.  The
inputs are generated on the GPU and the W untimed warm-up steps follow at
once; then K timed steps between two device synchronisations.  Prints ONE
JSON line.

``value`` = tokens/s of the whole job.  ``roofline`` covers the dominant
kernel (the fused gate/up GEMM): its algorithmic bytes per launch divided by
its mean duration over the timed steps, measured with two HIP events the
library records on its own stream right before and after that kernel,
against 8 TB/s.  After the timed region: the routing counts (for the
algorithmic work), a separate set of K steps with all seven stage events
(the per-stage breakdown and the down GEMM), rep-by-rep passes after a
1 GiB cache-flush write for workloads whose active weights would fit the
caches, the router scores kernel on its own, other workloads asked for with
``--also`` (by default DeepSeek-V3-shaped T=512 beside the default
Mixtral-shaped T=512), and ``cpu_baseline``: the CPU oracle (test
infrastructure, imported only for this leg) on a bounded sample of the same
workload on this host's cores, with the CPU model, input hashes and a
one-core figure on the tiny workload.

Other modes (not used by the default run):
  --profile            no CPU baseline, no other workloads, no cache-flushed or
                       hot-expert passes (for rocprofv3 runs)
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
GEMM_SRC = os.path.join(ROOT, "expert_dispatch_router_amd", "csrc", "grouped_gemm.hip")
DEFAULT_WORKLOAD = "mixtral_512"


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def input_hashes(x, logits, wgu, wd):
    """sha256 of the bytes of every input, taken from host copies of the
    device tensors the timed passes read (the same copies feed the oracle);
    weights hashed one expert at a time, experts in order."""
    from expert_dispatch_router_amd import synth

    def weights(w):
        h = hashlib.sha256()
        for e in range(w.shape[0]):
            h.update(synth.bf16_bits(w[e]).tobytes())
        return h.hexdigest()
    return {"x": synth.sha256(x), "router_logits": synth.sha256(logits),
            "W_gate_up": weights(wgu), "W_down": weights(wd)}


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
                      f"first {n} of {cfg.T} tokens ({dt:.1f} s)",
            "cpu_model": cpu_model(),
            "cores_available": len(os.sched_getaffinity(0))}


_SINGLE_CORE_TINY = r"""
import os, sys
# one core before anything starts threads: OpenMP then sees one CPU
os.sched_setaffinity(0, {int(sys.argv[2])})
import json, time
sys.path.insert(0, sys.argv[1])
import oracle
from expert_dispatch_router_amd import synth
cfg = synth.CONFIGS["tiny"]
x, lg, wgu, wd = synth.make_inputs(cfg, 0, "cpu")
xb, lgn = synth.bf16_bits(x), lg.numpy()
gu, dn = synth.bf16_bits(wgu), synth.bf16_bits(wd)
# after torch's CPU ops: torch sets the OpenMP thread count when it starts
# its own pool (from MKL_NUM_THREADS, if set, before OMP_NUM_THREADS)
oracle.set_threads(1)
passes, t0 = 0, time.perf_counter()
while time.perf_counter() - t0 < 2.0:
    oracle.forward(xb, lgn, gu, dn, cfg.top_k, cfg.renormalize, cfg.score, cfg.ffn)
    passes += 1
dt = time.perf_counter() - t0
print(json.dumps({"value": cfg.T * passes / dt, "unit": "tokens/s",
                  "cores": len(os.sched_getaffinity(0)), "omp_threads": oracle.max_threads(),
                  "kind": "oracle",
                  "sample": f"{passes} whole tiny passes (T={cfg.T}) in {dt:.1f} s, "
                            f"pinned to CPU {sys.argv[2]}"}))
"""


def cpu_single_core_tiny():
    """The oracle on the whole tiny workload in a child process pinned to
    one CPU (sched_setaffinity before OpenMP starts) with OMP_NUM_THREADS and
    MKL_NUM_THREADS 1 and the oracle's thread count set to 1 after the
    inputs are made: a one-core, one-thread figure whatever thread counts
    the environment sets."""
    import subprocess

    cpu = sorted(os.sched_getaffinity(0))[0]
    env = dict(os.environ, OMP_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _SINGLE_CORE_TINY, ROOT, str(cpu)],
                       capture_output=True, text=True, timeout=300, env=env)
    if r.returncode != 0:
        return {"error": r.stderr.strip().splitlines()[-1:] or ["failed"]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def stage_names(plan):
    """Names of the six intervals between the seven stage events, from the
    launch plan; an interval with no kernel in it measures only the cost of
    two back-to-back event records and is named None."""
    rl = plan["routing_launches"]
    names = ["route_histogram_scan_schedule_reorder" if rl == 1 else "route",
             None if rl == 1 else ("histogram_scan_schedule_reorder" if rl == 2
                                   else "histogram_scan_schedule"),
             "reorder" if rl == 3 else None,
             "gate_up_swiglu_down" if plan["fused_down"] else
             ("gate_up_unfused" if plan["unfused_swiglu"] else "gate_up_swiglu"),
             None if plan["fused_down"] else "down",
             None if plan["fold_combine"] else "combine"]
    if plan["gather_launch"]:
        names[2] = "reorder_gather" if rl == 3 else "gather"
    return names


class Runner:
    """One workload's inputs, workspace and launch plan on the GPU, and the
    timing loops around moe_forward."""

    def __init__(self, cfg, seed, dev, unfused=0, copy_bytes=0):
        import torch

        import expert_dispatch_router_amd as moe
        from expert_dispatch_router_amd import synth

        self.cfg, self.dev, self.unfused = cfg, dev, unfused
        self.x, self.logits, self.wgu, self.wd = synth.make_inputs(cfg, seed, dev)
        self.plan = moe.moe_plan_ex(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k,
                                    unfused_swiglu=unfused)
        self.out = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(moe.moe_workspace_size(cfg.T, cfg.d, cfg.ffn, cfg.E, cfg.top_k,
                                                     unfused_swiglu=unfused),
                              dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.copy_src = self.copy_dst = None
        if copy_bytes:
            self.copy_src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
            self.copy_dst = torch.empty_like(self.copy_src)

    def step(self, stage_events=None, strm=None):
        import expert_dispatch_router_amd as moe

        c = self.cfg
        moe.moe_forward(self.x, self.logits, self.wgu, self.wd, c.top_k, c.renormalize,
                        out=self.out, score=c.score, workspace=self.ws, stream=strm or self.stream,
                        stage_events=stage_events, unfused_swiglu=self.unfused)
        if self.copy_src is not None:
            self.copy_dst.copy_(self.copy_src)

    def timed(self, warmup, steps):
        """warmup untimed passes, then `steps` passes between two device
        synchronisations.  In every timed pass the library records two
        fence-free HIP events on its stream, right before and right after
        the fused gate/up GEMM (stage events 3 and 4; measured at ~1.5 us of
        GPU time each): that kernel's duration over the timed region."""
        import numpy as np
        import torch

        import expert_dispatch_router_amd as moe

        # the events are made before the warm-up passes, so that nothing but
        # the synchronisation separates the last warm-up pass from the timed ones
        ev = [(moe.Timer(), moe.Timer()) for _ in range(steps)]
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            a, b = ev[i]
            self.step(stage_events=[None, None, None, a.handle, b.handle, None, None])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        return elapsed, np.array([a.elapsed_ms(b) for a, b in ev])

    def stages(self, steps):
        """A separate run of `steps` passes with the seven stage events
        (each record adds a few microseconds of its own)."""
        import numpy as np
        import torch

        import expert_dispatch_router_amd as moe

        timers = [[moe.Timer() for _ in range(7)] for _ in range(steps)]
        for i in range(steps):
            self.step(stage_events=[t.handle for t in timers[i]])
        torch.cuda.synchronize()
        ms = np.array([[timers[i][s].elapsed_ms(timers[i][s + 1]) for s in range(6)]
                       for i in range(steps)])
        whole = np.array([timers[i][0].elapsed_ms(timers[i][6]) for i in range(steps)])
        return ms, whole

    def flushed(self, reps, warmup=3, flush_bytes=1 << 30):
        """The pass timed rep by rep with a 1 GiB write between reps, outside
        the timed interval, so that no weight byte is served from the 256 MiB
        MALL or the L2s: (median, p10, p90) ms from the first to the last
        stage event."""
        import numpy as np
        import torch

        import expert_dispatch_router_amd as moe

        buf = torch.empty(flush_bytes, dtype=torch.uint8, device=self.dev)
        for _ in range(warmup):
            self.step()
        vals = []
        for _ in range(reps):
            buf.fill_(7)
            t = [moe.Timer() for _ in range(7)]
            self.step(stage_events=[t[0].handle] + [None] * 5 + [t[6].handle])
            torch.cuda.synchronize()
            vals.append(t[0].elapsed_ms(t[6]))
        del buf
        v = np.array(vals)
        return float(np.median(v)), float(np.percentile(v, 10)), float(np.percentile(v, 90))

    def routing_counts(self):
        import expert_dispatch_router_amd as moe

        c = self.cfg
        r = moe.moe_route(self.logits, c.top_k, c.renormalize, c.score)
        return r["counts"].cpu().numpy()


def hot_experts(r, counts, steps, n_hot=4):
    """The full-tile regime of skewed routing on its own: the same tokens,
    weights and top-k, with every token routed to the n_hot experts the
    workload's routing loads most (each then holds T rows: full blocks).
    The fused gate/up GEMM's FLOPs over its mean duration (two events around
    it, as in the timed passes) against the bf16 dense MFMA peak, over
    128-row blocks (the automatic table: the launch fits one round) and over
    256-row blocks (schedule 3, the tile the workload's hot experts take when
    its routing kernels merge); `active_frac` divides by the peak of the CUs
    that have a workgroup (blocks x column tiles, at most 256)."""
    import numpy as np
    import torch

    import expert_dispatch_router_amd as moe

    cfg = r.cfg
    hot = [int(e) for e in np.argsort(-counts, kind="stable")[:n_hot]]
    lg = r.logits.clone()
    lg[:, hot] += 40.0  # far above the N(0, 1) scores and the skew biases
    k = cfg.top_k
    rows = cfg.T * min(k, n_hot)
    flop = 4.0 * rows * cfg.ffn * cfg.d
    tiles = -(-cfg.ffn // 128)
    res = {"experts": hot, "rows_per_expert": cfg.T}
    for label, sched, bm in (("blocks_128", 1, 128), ("blocks_256", 3, 256)):
        ws = torch.empty(moe.moe_workspace_size(cfg.T, cfg.d, cfg.ffn, cfg.E, k, block_rows=128,
                                                schedule=sched),
                         dtype=torch.uint8, device=r.dev)
        f = lambda se=None: moe.moe_forward(r.x, lg, r.wgu, r.wd, k, cfg.renormalize, out=r.out,
                                            score=cfg.score, workspace=ws, stage_events=se,
                                            block_rows=128, schedule=sched)
        for _ in range(5):
            f()
        ev = [(moe.Timer(), moe.Timer()) for _ in range(steps)]
        for a, b in ev:
            f([None, None, None, a.handle, b.handle, None, None])
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_ms(b) for a, b in ev]))
        tf = flop / (ms * 1e-3) / 1e12
        wgs = min(n_hot * -(-cfg.T // bm) * tiles, 256)
        res[label] = {"gate_up_mean_ms": ms, "gate_up_tflops": tf,
                      "mfma_frac": tf / BF16_PEAK_TFLOPS, "workgroups": wgs,
                      "active_frac": tf / (BF16_PEAK_TFLOPS * wgs / 256)}
        del ws
    # the figures of the automatic table, as before, at the top level
    res.update({"gate_up_mean_ms": res["blocks_128"]["gate_up_mean_ms"],
                "gate_up_tflops": res["blocks_128"]["gate_up_tflops"],
                "mfma_frac": res["blocks_128"]["mfma_frac"],
                "note": f"every token routed to the {n_hot} experts the workload loads most "
                        "(full blocks); gate/up GEMM FLOPs over its mean duration"})
    return res


def pct(v):
    import numpy as np

    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90))}


def workload_label(cfg):
    return (f"{cfg.name}: MoE layer T={cfg.T} d={cfg.d} ffn={cfg.ffn} E={cfg.E} top-{cfg.top_k} "
            f"{'sigmoid' if cfg.score else 'softmax'}{' renormalised' if cfg.renormalize else ''}")


def k4_algorithmic(cfg, alg, plan):
    """(bytes, FLOP) of one launch of the dominant kernel: the fused gate/up
    GEMM (with the down projection when that is fused into it)."""
    if plan["fused_down"]:
        return alg["e_act"] * 6.0 * cfg.ffn * cfg.d + 2.0 * alg["A"] * cfg.d, alg["flop"]
    return alg["bytes_k4"], alg["flop_k4"]


def also_workload(name, seed, dev, warmup, steps):
    """Another workload measured in the same process, same warm-up and step
    counts: ms per pass, tokens/s, pass roofline, and the gate/up kernel's
    mean over the timed region against 8 TB/s."""
    import torch

    from expert_dispatch_router_amd import synth

    cfg = synth.CONFIGS[name]
    r = Runner(cfg, seed, dev)
    elapsed, k4 = r.timed(warmup, steps)
    alg = algorithmic(cfg, r.routing_counts())
    t_step = elapsed / steps
    t_roof = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9), alg["flop"] / (BF16_PEAK_TFLOPS * 1e12))
    kb, _ = k4_algorithmic(cfg, alg, r.plan)
    k4_ms = float(k4.mean())
    res = {"workload": workload_label(cfg), "steps": steps, "warmup": warmup,
           "ms_per_step": t_step * 1e3, "tokens_per_s": cfg.T / t_step,
           "tflops": alg["flop"] / t_step / 1e12, "hbm_gbs": alg["bytes"] / t_step / 1e9,
           "roofline_frac_step": t_roof / t_step, "t_roof_ms": t_roof * 1e3,
           "gate_up": {"mean_launch_ms": k4_ms, "alg_bytes_per_launch": kb,
                       "achieved_gbs": kb / (k4_ms * 1e-3) / 1e9,
                       "frac": kb / (k4_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    del r
    torch.cuda.empty_cache()
    return res


def run(args):
    import numpy as np
    import torch

    from expert_dispatch_router_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    unfused = 1 if args.unfused else 0
    # Inputs are generated on the GPU, and the warm-up passes follow at once:
    # nothing that waits on the host runs between them (the routing counts
    # used for the report are read after the timed region).
    r = Runner(cfg, args.seed, dev, unfused, args.copy_bytes)
    elapsed, k4_each = r.timed(args.warmup, args.steps)
    ms_step = elapsed * 1e3 / args.steps
    plan = r.plan
    alg = algorithmic(cfg, r.routing_counts())
    stage_each, pass_each = r.stages(args.steps)
    stage_mean = stage_each.mean(axis=0)
    k5_each = None if plan["fused_down"] else stage_each[:, 4]

    t_step = elapsed / args.steps
    t_roof = max(alg["bytes"] / (HBM_PEAK_GBS * 1e9), alg["flop"] / (BF16_PEAK_TFLOPS * 1e12))
    k4_ms = float(k4_each.mean())
    k4_s = k4_ms * 1e-3
    k4_bytes, k4_flop = k4_algorithmic(cfg, alg, plan)
    achieved = k4_bytes / k4_s / 1e9
    names = stage_names(plan)
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
        "config": {"workload": workload_label(cfg),
                   "tokens": cfg.T, "hidden": cfg.d, "ffn": cfg.ffn, "experts": cfg.E,
                   "top_k": cfg.top_k, "block_rows": plan["block_rows"], "split_k": plan["split_k"],
                   "active_experts": alg["e_act"], "seed": args.seed,
                   "launches_per_pass": plan["launches"],
                   "swiglu": "unfused ablation" if unfused else "fused",
                   "down_projection": "in the gate/up GEMM" if plan["fused_down"] else "own GEMM",
                   "gate_up_blocks": ("variable: 256 rows for experts past 128 where one round "
                                      "of workgroups needs it (decided on the device)")
                                     if plan["variable_rows"] else "fixed"},
        "tflops": alg["flop"] / t_step / 1e12,
        "hbm_gbs": alg["bytes"] / t_step / 1e9,
        "roofline_frac_step": t_roof / t_step,
        "t_roof_ms": t_roof * 1e3,
        # a second, separately run set of passes with seven stage events;
        # intervals with no kernel (the one-workgroup routing covers three
        # stages, for instance) only measure two back-to-back event records
        "stage_ms": {n: round(float(v), 5) for n, v in zip(names, stage_mean) if n},
        "event_only_intervals_ms": [round(float(v), 5) for n, v in zip(names, stage_mean)
                                    if not n],
        # distributions: the fused gate/up GEMM over the timed passes, the
        # down GEMM and the whole pass (first to last event) over the
        # stage-event passes
        "k4_ms_pct": pct(k4_each),
        "k5_ms_pct": None if k5_each is None else pct(k5_each),
        "pass_ms_pct": pct(pass_each),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if (unfused or plan["fused_down"]) else traffic_for(cfg.name),
                     "kernel": ("gate/up stage of the unfused ablation (gate GEMM + up GEMM + "
                                "activation)") if unfused else
                               ("gate_up_swiglu_down (fused gate/up SwiGLU grouped GEMM with "
                                "the down projection in its epilogue)") if plan["fused_down"] else
                               "gate_up_swiglu (fused gate/up SwiGLU grouped GEMM)",
                     "alg_bytes_per_launch": k4_bytes,
                     "mean_launch_ms": k4_ms,
                     "timing": "two fence-free HIP events on the library's stream around the "
                               "kernel in every timed pass"},
        # the same kernel against the bf16 dense MFMA peak (its FLOPs over its
        # mean duration): the hot experts of skewed routing are locally
        # MFMA-bound even where the launch as a whole is HBM-bound
        "k4_mfma": {"achieved": k4_flop / k4_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": k4_flop / k4_s / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if k5_each is not None:
        dn_bytes = alg["e_act"] * 2.0 * cfg.ffn * cfg.d + alg["A"] * (2.0 * cfg.ffn + 4.0 * cfg.d)
        k5_ms = float(k5_each.mean())
        res["down"] = {"mean_launch_ms": k5_ms, "alg_bytes_per_launch": dn_bytes,
                       "timing": "stage events of the stage-breakdown passes",
                       "achieved_gbs": dn_bytes / (k5_ms * 1e-3) / 1e9,
                       "frac": dn_bytes / (k5_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if args.flush or (args.flush is None and not args.profile and
                      alg["e_act"] * 6.0 * cfg.ffn * cfg.d < (1 << 30)):
        med, p10, p90 = r.flushed(args.steps)
        res["cache_flushed"] = {
            "ms_per_pass_p50": med, "p10": p10, "p90": p90, "roofline_frac": t_roof / (med * 1e-3),
            "protocol": f"{args.steps} reps after 3 warm-ups, a 1 GiB write before each rep "
                        "outside the timed interval (first to last stage event)"}
    if cfg.skew_alpha > 0 and not args.profile:
        res["hot_experts"] = hot_experts(r, r.routing_counts(), args.steps,
                                         n_hot=min(cfg.top_k, 4))
    res["router_gemm"] = router_gemm(cfg, r.x, args.seed, args.steps, r.stream)
    if args.graph:
        res["graph"] = graph_replay(lambda strm=None: r.step(strm=strm), args.steps, cfg.T)
    x, logits, wgu, wd = r.x, r.logits, r.wgu, r.wd
    for name in ([] if args.also is None else [a for a in args.also.split(",") if a]):
        if name == cfg.name:
            continue
        del r
        torch.cuda.empty_cache()
        res.setdefault("also", {})[name] = also_workload(name, args.seed, dev, args.warmup,
                                                         args.steps)
        r = None
    if not args.profile and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, x, logits, wgu, wd, args.cpu_seconds)
        res["cpu_baseline"]["inputs_sha256"] = input_hashes(x, logits, wgu, wd)
        res["cpu_baseline"]["tiny_one_core"] = cpu_single_core_tiny()
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
        # the variable-rows kernel is the same gate/up SwiGLU GEMM
        "gate_up_swiglu": lambda n: mode(n) == 0 or "gemm_lds_var_kernel" in n,
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
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
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
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads also measured in the same process "
                         "(default: dsv3_512 with the default workload, else none)")
    ap.add_argument("--flush", dest="flush", action="store_true", default=None,
                    help="also time passes rep by rep after a 1 GiB cache-flush write "
                         "(default: when the active expert weights are under 1 GiB)")
    ap.add_argument("--no-flush", dest="flush", action="store_false")
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
    if args.also is None and args.workload == DEFAULT_WORKLOAD and not args.profile:
        args.also = "dsv3_512"
    run(args)


if __name__ == "__main__":
    main()
