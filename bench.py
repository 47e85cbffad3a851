"""Benchmark: constrained denoising steps per second on one MI355X.

One step = fa_build_transitions + fa_span_tree + fa_sample + fa_marginals
(q written) over the whole batch of the json-like DFA workload (S=256,
V=151,936, L=256, B=4), inputs resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
METRIC = "constrained denoising steps/sec + per-step µs (L=256, V=151,936); HBM/MFMA % peak"
CSRC = os.path.join(ROOT, "constrained_decoding_diffusion_amd", "csrc")


def src_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("src_hash") != src_hash():
        return None
    return rec


def algorithmic_work(tb, B, L):
    S, Sp, V = tb.info["S"], tb.info["Sp"], tb.info["V"]
    Lpad = 1 << max(0, (L - 1).bit_length())
    K = Lpad.bit_length() - 1
    table_bytes = tb.device_bytes
    p_bytes = B * L * V * 4
    leaves = B * Lpad * Sp * Sp * 4
    internal = B * (Lpad - 1) * Sp * Sp * 4
    return dict(
        a1_bytes=p_bytes + table_bytes + leaves,
        a2_flops=2.0 * Sp ** 3 * B * (Lpad - 1),
        a2_launches=K,
        a4_bytes=p_bytes + p_bytes + leaves + internal + table_bytes,
        S=S, Sp=Sp, V=V, Lpad=Lpad, K=K)


def cpu_baseline(w):
    """The serial fp64 oracle, single thread, on one full step of the same
    workload (all B rows): emission weights, forward-backward, tree-order
    sampling and marginals at every position."""
    import oracle
    orc = oracle.Oracle(w.aut)
    t0 = time.perf_counter()
    for b in range(w.B):
        W = orc.edge_weights(w.p[b])
        fb = orc.forward_backward(W)
        st, tk, _ = orc.sample_tree(w.p[b], W, w.seed, b)
        orc.marginals(w.p[b], fb, None, tk, 0)
    dt = time.perf_counter() - t0
    return dict(value=1.0 / dt, unit="steps/s", cores=1, kind="oracle",
                sample=f"one full step (all {w.B} rows, every position) of the same workload, "
                       f"serial fp64 C, {dt:.2f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=3, help="preset 1..5 (default 3)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run one plain device copy of 1 GiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import constrained_decoding_diffusion_amd as fa
    from synth import configs

    w = configs.make(args.workload)
    tb = fa.Table.from_automaton(w.aut)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    p = torch.from_numpy(w.p).to(dev)
    tb.upload(dev)
    bufs = fa.StepBuffers(tb, w.B, w.L, want_q=True, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if args.copy_calib:
        src_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
    torch.cuda.synchronize()

    def one_step(seed, ev=None):
        bufs.status.zero_()
        if ev: ev[0].record()
        fa.build_transitions(tb, p, bufs, stream)
        if ev: ev[1].record()
        fa.span_tree(tb, bufs, stream)
        if ev: ev[2].record()
        fa.sample(tb, p, bufs, seed, stream)
        if ev: ev[3].record()
        fa.marginals(tb, p, bufs, fa.FA_CONF_PROB, stream, write_q=True)
        if ev: ev[4].record()

    for s in range(args.warmup):
        one_step(w.seed + s)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        one_step(w.seed + args.warmup + s, evs[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    names = ["build_transitions", "span_tree", "sample", "marginals"]
    stage_ms = {n: 0.0 for n in names}
    for ev in evs:
        for k, n in enumerate(names):
            stage_ms[n] += ev[k].elapsed_time(ev[k + 1])
    stage_us = {n: 1000.0 * v / args.steps for n, v in stage_ms.items()}
    ms_per_step = total_ms / args.steps
    status = bufs.status.cpu().numpy()

    work = algorithmic_work(tb, w.B, w.L)
    stages = {
        "build_transitions": dict(us=stage_us["build_transitions"], bound="hbm",
                                  algorithmic_bytes=work["a1_bytes"],
                                  gbs=work["a1_bytes"] / (stage_us["build_transitions"] * 1e3)),
        "span_tree": dict(us=stage_us["span_tree"], bound="mfma", algorithmic_flops=work["a2_flops"],
                          tflops=work["a2_flops"] / (stage_us["span_tree"] * 1e6)),
        "sample": dict(us=stage_us["sample"], bound="latency"),
        "marginals": dict(us=stage_us["marginals"], bound="hbm", algorithmic_bytes=work["a4_bytes"],
                          gbs=work["a4_bytes"] / (stage_us["marginals"] * 1e3)),
    }
    for n in ("build_transitions", "marginals"):
        stages[n]["frac"] = stages[n]["gbs"] / HBM_PEAK_GBS
    stages["span_tree"]["frac"] = stages["span_tree"]["tflops"] / FP32_MFMA_PEAK_TFLOPS
    dominant = max(names, key=lambda n: stage_us[n])
    if dominant == "span_tree":
        # span_gemm launches: K per step; the call adds one fill and one
        # root-reduction launch of a few microseconds
        per_launch_us = stage_us["span_tree"] / work["a2_launches"]
        achieved = work["a2_flops"] / (stage_us["span_tree"] * 1e6)
        tr = traffic_record("span_gemm")
        roof = dict(bound="mfma", kernel="span_gemm", achieved=achieved,
                    peak=FP32_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / FP32_MFMA_PEAK_TFLOPS,
                    traffic=(tr["bytes_per_launch"] if tr else None),
                    avg_launch_us=per_launch_us, launches_per_step=work["a2_launches"])
    else:
        kern = {"build_transitions": "emission", "marginals": "marg_q", "sample": "sample"}[dominant]
        st = stages[dominant]
        tr = traffic_record(kern)
        roof = dict(bound="hbm", kernel=kern, achieved=st.get("gbs", 0.0), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=st.get("frac", 0.0),
                    traffic=(tr["bytes_per_launch"] if tr else None))
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_step": 1000.0 * ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.describe(), "B": w.B, "L": w.L, "S": w.aut.S, "V": w.aut.V,
                   "sequence_steps_per_s": w.B * 1000.0 / ms_per_step},
        "roofline": roof,
        "stages": stages,
        "wall_s": wall,
        "row_status": status.tolist(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
