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
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix
# the span products run on the bf16 matrix cores: each fp32 product is six
# bf16 products of the operands' three-piece split
SPLIT_PRODUCTS = 6
# vector ALU issue: 256 CUs x 64 lanes x 2.4 GHz (fp64 and unpacked fp32 alike)
VALU_FP64_LANE_OPS = 256 * 64 * 2.4e9
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
    """Algorithmic bytes / flops per step and per launch of the measured
    kernels (the method's own data movement and arithmetic, no re-reads)."""
    # the method's own sizes: S trimmed states (the kernels' padded Sp adds
    # work that is not counted)
    S, Sp, V = tb.info["S"], tb.info["Sp"], tb.info["V"]
    Lpad = 1 << max(0, (L - 1).bit_length())
    K = Lpad.bit_length() - 1
    table_bytes = tb.device_bytes
    p_bytes = B * L * V * 4
    mask_bytes = V * 4
    dense_leaves = B * Lpad * S * S * 4
    pair_values = B * L * tb.info["pairs"] * 4
    # a leafless table writes each leaf's pair values, not the dense S*S leaf;
    # a message pass whose leaf level takes the pair values reads those, not
    # the dense leaves (both only when the tree has more than one leaf)
    leafless = bool(tb.info["leafless"]) and K >= 1
    leaf_msg_pairs = bool(tb.info["leaf_msg_pairs"]) and K >= 1
    a1_leaves = pair_values if leafless else dense_leaves
    a4_leaves = pair_values if leaf_msg_pairs else dense_leaves
    internal = B * (Lpad - 1) * S * S * 4
    sparse1 = bool(tb.info["first_sparse"])
    pairs1 = bool(tb.info["first_pairs"])
    sparse2 = sparse1 and bool(tb.info["second_sparse"]) and K >= 2
    npairs, w1 = tb.info["pairs"], tb.info["first_work"]
    npairs2, w2 = tb.info["pairs2"], tb.info["second_work"]
    # first level: dense 2*S^3 per product, or the sparse form's multiply-adds
    # (pairs (a, k), (k, c) sharing k) per product; second level likewise for
    # its L//4 products inside the sequence when it is sparse
    level1_flops = B * (Lpad // 2) * (2.0 * w1 if sparse1 else 2.0 * S ** 3)
    nsp2 = L // 4 if sparse2 else 0
    level2_flops = B * (nsp2 * 2.0 * w2 + (Lpad // 4 - nsp2) * 2.0 * S ** 3) if K >= 2 else 0.0
    upper_flops = 2.0 * S ** 3 * B * max(Lpad // 4 - 1, 0)
    out2 = npairs2 * 4 if sparse2 else 0

    # the tree's roofline, level by level: a dense product reads its two
    # operands and writes its output (3*S^2*4 bytes; a pair-staged first
    # level reads both leaves' pair values instead) and executes 6*2*S^3
    # bf16 flops; its ideal time is the larger of the two at peak.  A sparse
    # level moves its bytes and does its multiply-adds on the vector ALUs.
    def dense_product(in_bytes):
        return dict(bytes=in_bytes + S * S * 4, mfma_flops=SPLIT_PRODUCTS * 2.0 * S ** 3)

    levels = []
    for k in range(1, K + 1):
        nprod = B * (Lpad >> k)
        if k == 1 and sparse1:
            per = dict(bytes=S * S * 4 + 2 * npairs * 4 + out2, mfma_flops=0.0)
        elif k == 1 and pairs1:
            per = dense_product(2 * npairs * 4)
        else:
            per = dense_product(2 * S * S * 4)
        n_dense = nprod - (nsp2 if k == 2 else 0)
        lv = dict(level=k, products=nprod, bytes=nprod * per["bytes"], mfma_flops=n_dense * per["mfma_flops"])
        if k == 2 and nsp2:
            lv["bytes"] += nsp2 * (2 * npairs2 * 4 + S * S * 4 - per["bytes"])
        lv["ideal_us"] = max(lv["bytes"] / (HBM_PEAK_GBS * 1e3), lv["mfma_flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e6))
        levels.append(lv)
    l1 = levels[0] if levels else dict(bytes=0.0, mfma_flops=0.0)
    if sparse1:
        level1 = dict(bound="hbm", work=l1["bytes"], unit="GB/s",
                      per_unit="per product: the dense S*S output write + both leaves' pair values "
                               "(2*pairs*4) + its values on the two-step pattern when the second "
                               "level is sparse (pairs2*4), B*Lpad/2 products")
    elif l1["mfma_flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e6) >= l1["bytes"] / (HBM_PEAK_GBS * 1e3):
        level1 = dict(bound="mfma", work=l1["mfma_flops"], unit="TFLOP/s", peak=BF16_MFMA_PEAK_TFLOPS,
                      per_unit="6*2*S^3 bf16 flops per product (six bf16 products of the three-piece "
                               "split per fp32 product, S trimmed states), B*Lpad/2 products",
                      fp32_equivalent_flops=l1["mfma_flops"] / SPLIT_PRODUCTS)
    else:
        level1 = dict(bound="hbm", work=l1["bytes"], unit="GB/s",
                      per_unit=("per product: both leaves' pair values (2*pairs*4)" if pairs1 else
                                "per product: both dense leaves (2*S*S*4)") +
                               " + the dense S*S output write, B*Lpad/2 products")
    return dict(
        a1_bytes=p_bytes + table_bytes + a1_leaves,
        a1_basis=("p read + table + " + ("each leaf's pair values written (B*L*pairs*4)" if leafless
                                         else "dense leaves written (B*Lpad*S*S*4)")),
        a2_flops=level1_flops + level2_flops + upper_flops,
        tree_levels=levels,
        a4_bytes=p_bytes + p_bytes + a4_leaves + internal + table_bytes,
        a4_basis=("p read + q write + internal nodes read + table + " +
                  ("leaf pair values read (B*L*pairs*4)" if leaf_msg_pairs
                   else "dense leaves read (B*Lpad*S*S*4)")),
        # per launch of the kernels the library can bracket with events
        kernels={
            "emission_dense": dict(bound="hbm", work=p_bytes + mask_bytes, unit="GB/s",
                                   per_unit="p read once (B*L*V*4) + token mask (V*4)"),
            level1_name(tb): level1,
            "marg_q": dict(bound="hbm", work=2 * p_bytes + mask_bytes, unit="GB/s",
                           per_unit="p read + q write (2*B*L*V*4) + token mask (V*4)"),
        },
        S=S, Sp=Sp, V=V, Lpad=Lpad, K=K)


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        ev = self.C.c_void_p()
        if self.hip.hipEventCreate(self.C.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        """Milliseconds between two recorded events, or None when the kernel
        did not run (this workload has no such launch)."""
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), self.C.c_void_p(a), self.C.c_void_p(b)) != 0:
            return None
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(self.C.c_void_p(ev))


def cpu_info():
    """CPU model (from /proc/cpuinfo), logical CPUs, and the CPUs this
    process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return model, os.cpu_count(), affinity


def cpu_baseline(w, reps=3):
    """The serial fp64 oracle, single thread, on one full step of the same
    workload (all B rows): emission weights, forward-backward, tree-order
    sampling and marginals at every position.  Median of `reps` runs."""
    import oracle
    orc = oracle.Oracle(w.aut)
    runs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        for b in range(w.B):
            W = orc.edge_weights(w.p[b])
            fb = orc.forward_backward(W)
            st, tk, _ = orc.sample_tree(w.p[b], W, w.seed, b)
            orc.marginals(w.p[b], fb, None, tk, 0)
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[len(runs) // 2]
    model, nproc, affinity = cpu_info()
    return dict(value=1.0 / dt, unit="steps/s", cores=1, kind="oracle",
                cpu_model=model, nproc=nproc, affinity_cpus=affinity,
                runs_s=runs,
                sample=f"one full step (all {w.B} rows, every position) of the same workload, "
                       f"serial fp64 C on one thread, median of {reps} runs: {dt:.2f} s")


def ceilings(torch, fa, dev, p, reps=7):
    """Bandwidth ceilings measured in the same run with HIP events, median
    of `reps` each: the library's plain read and copy kernels
    (fa_probe_bandwidth) over p and over a 1 GiB buffer, best over a few
    grid sizes; and torch's own device copy of 1 GiB for reference."""
    stream = torch.cuda.current_stream(dev).cuda_stream

    def med(fn):
        ts = []
        for _ in range(reps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1000.0)
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    def rec(us, nbytes, how):
        gbs = nbytes / (us * 1e3)
        return dict(us=us, bytes=nbytes, gbs=gbs, frac=gbs / HBM_PEAK_GBS, how=how)

    grids = (1024, 2048, 4096, 8192)
    part = torch.empty(max(grids), dtype=torch.float32, device=dev)
    pb = p.numel() * 4
    best = min((med(lambda g=g: fa.probe_bandwidth(fa.FA_PROBE_READ, p, part, pb, g, stream)), g)
               for g in grids)
    out = {"read_p": rec(best[0], pb, f"plain read kernel over p, {best[1]} workgroups")}
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    best = min((med(lambda g=g: fa.probe_bandwidth(fa.FA_PROBE_READ, src, part, 1 << 30, g, stream)), g)
               for g in grids)
    out["read_1GiB"] = rec(best[0], 1 << 30, f"plain read kernel, 1 GiB, {best[1]} workgroups")
    best = min((med(lambda g=g: fa.probe_bandwidth(fa.FA_PROBE_COPY, src, dst, 1 << 30, g, stream)), g)
               for g in grids)
    out["copy_1GiB"] = rec(best[0], 2 << 30, f"plain copy kernel, 1 GiB each way, streaming stores, "
                                             f"{best[1]} workgroups of 1024 threads")
    out["torch_copy_1GiB"] = rec(med(lambda: dst.copy_(src)), 2 << 30, "torch copy_ of 1 GiB")
    del src, dst, part
    return out


def stage_fracs(work, stage_us, separate):
    """Per-stage µs with the algorithmic rate and fraction of peak."""
    st = {
        "build_transitions": dict(us=stage_us["build_transitions"], bound="hbm",
                                  algorithmic_bytes=work["a1_bytes"], basis=work["a1_basis"],
                                  gbs=work["a1_bytes"] / (stage_us["build_transitions"] * 1e3)),
        "span_tree": dict(us=stage_us["span_tree"], bound="mfma+hbm",
                          ideal_us=sum(lv["ideal_us"] for lv in work["tree_levels"]),
                          basis=("per level the larger of its HBM bytes at 8 TB/s and its bf16 "
                                 "flops (six per fp32 product) at 2.5 PFLOP/s"),
                          algorithmic_flops=work["a2_flops"],
                          fp32_equivalent_tflops=work["a2_flops"] / (stage_us["span_tree"] * 1e6)),
    }
    if separate:
        st["sample"] = dict(us=stage_us["sample"], bound="latency")
        last = "marginals"
    else:
        last = "sample_marginals"
    st[last] = dict(us=stage_us[last], bound="hbm", algorithmic_bytes=work["a4_bytes"],
                    basis=work["a4_basis"], gbs=work["a4_bytes"] / (stage_us[last] * 1e3))
    for n in ("build_transitions", last):
        st[n]["frac"] = st[n]["gbs"] / HBM_PEAK_GBS
    st["span_tree"]["frac"] = st["span_tree"]["ideal_us"] / st["span_tree"]["us"]
    return st


def time_workload(torch, fa, configs, k, steps, warmup, dev, device_p=False, live=False,
                  chain=True, map_calls=0):
    """µs per step of preset k (joint call form): `steps` steps bracketed by
    two events, then as many with events between the calls for the stage
    split.  live: the table compiled with FA_LIVE_STATES.  map_calls > 0:
    also greedy (MAP) decoding of the whole batch, that many timed calls after
    one untimed call."""
    t_prep = time.perf_counter()
    w = configs.make(k, device=dev if device_p else None)
    tb = fa.Table.from_automaton(w.aut, live_states=live)
    tb.upload(dev)
    p = w.p if device_p else torch.from_numpy(w.p).to(dev)
    bufs = fa.StepBuffers(tb, w.B, w.L, want_q=True, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    prep_s = time.perf_counter() - t_prep
    names = ["build_transitions", "span_tree", "sample_marginals"]

    def step(seed, ev=None):
        bufs.status.zero_()
        if ev: ev[0].record()
        fa.build_transitions(tb, p, bufs, stream)
        if ev: ev[1].record()
        fa.span_tree(tb, bufs, stream)
        if ev: ev[2].record()
        fa.sample_marginals(tb, p, bufs, seed, fa.FA_CONF_PROB, stream, write_q=True)
        if ev: ev[3].record()

    for s in range(warmup):
        step(w.seed + s)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        step(w.seed + warmup + s)
    t1.record()
    torch.cuda.synchronize()
    us = 1000.0 * t0.elapsed_time(t1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for s in range(steps):
        step(w.seed + warmup + s, evs[s])
    torch.cuda.synchronize()
    stage_us = {n: 1000.0 * sum(ev[j].elapsed_time(ev[j + 1]) for ev in evs) / steps
                for j, n in enumerate(names)}
    work = algorithmic_work(tb, w.B, w.L)
    status = bufs.status.cpu().numpy().tolist()
    del bufs
    chain = time_chain_vs_tree(torch, fa, tb, p, w.seed, min(steps, 5), 1, w.aut) if chain else None
    torch.cuda.empty_cache()
    mapd = time_map(torch, fa, tb, p, map_calls, 1) if map_calls else None
    out = dict(workload=w.describe(), B=w.B, L=w.L, S=tb.info["S"], Sp=tb.info["Sp"], V=w.aut.V,
               steps=steps, warmup=warmup, us_per_step=us, steps_per_s=1e6 / us,
               sequence_steps_per_s=w.B * 1e6 / us,
               first_level=first_level_name(tb),
               second_level="sparse" if tb.info["second_sparse"] else "dense",
               leafless=bool(tb.info["leafless"]), live_states=bool(tb.info["live_states"]),
               flops_note=("the tree's flops count every product over all states (a dense-equivalent "
                           "rate: the restricted products execute fewer)") if live else None,
               p_drawn="on the device (same distribution, torch generator)" if device_p
               else "on the host (numpy PCG64)",
               stages=stage_fracs(work, stage_us, False), row_status=status,
               chain_vs_tree=chain, map_decode=mapd, host_prep_s=prep_s)
    del p, tb, w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def time_chain_vs_tree(torch, fa, tb, p, seed, steps, warmup, aut=None):
    """The pages' central trade on this GPU: the sampling half of a step
    (emission reduce, then the draws and log Z) through the log-depth tree
    (fa_span_tree + fa_sample) and through the serial chain
    (fa_chain_sample: L dependent forward launches, then backward sampling);
    then the whole step with q written both ways (fa_span_tree +
    fa_sample_marginals against fa_chain_sample_marginals: L more dependent
    launches for the backward messages).  µs per step each.  The chain reads
    dense leaves: a table that keeps none is compiled again with them
    (FA_FIRST_LEVEL_DENSE, from `aut`) for both sides; None without `aut`."""
    if tb.info["leafless"]:
        if aut is None:
            return None
        tb = fa.Table.from_automaton(aut, first_level="dense")
        tb.upload(p.device)
    B, L, _ = p.shape
    bufs = fa.StepBuffers(tb, B, L, want_q=True, device=p.device)
    stream = torch.cuda.current_stream(p.device).cuda_stream

    def tree_step(s):
        bufs.status.zero_()
        fa.build_transitions(tb, p, bufs, stream)
        fa.span_tree(tb, bufs, stream)
        fa.sample(tb, p, bufs, s, stream)

    def chain_step(s):
        bufs.status.zero_()
        fa.build_transitions(tb, p, bufs, stream)
        fa.chain_sample(tb, p, bufs, s, stream)

    def tree_full(s):
        bufs.status.zero_()
        fa.build_transitions(tb, p, bufs, stream)
        fa.span_tree(tb, bufs, stream)
        fa.sample_marginals(tb, p, bufs, s, fa.FA_CONF_PROB, stream, write_q=True)

    def chain_full(s):
        bufs.status.zero_()
        fa.build_transitions(tb, p, bufs, stream)
        fa.chain_sample_marginals(tb, p, bufs, s, fa.FA_CONF_PROB, stream, write_q=True)

    out = {}
    for name, fn in (("tree", tree_step), ("chain", chain_step), ("tree_full_step", tree_full),
                     ("chain_full_step", chain_full)):
        for s in range(warmup):
            fn(seed + s)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for s in range(steps):
            fn(seed + warmup + s)
        b.record()
        torch.cuda.synchronize()
        out[name + "_us"] = 1000.0 * a.elapsed_time(b) / steps
    out["chain_over_tree"] = out["chain_us"] / out["tree_us"]
    out["chain_over_tree_full_step"] = out["chain_full_step_us"] / out["tree_full_step_us"]
    out["what"] = ("emission reduce + (span tree + top-down sampler) vs emission reduce + "
                   "(serial forward filter, L launches, + backward sampler); both draw tokens. "
                   "full_step: the same plus q and the confidence (tree: message pass; chain: "
                   "backward messages, L launches)")
    out["row_status"] = bufs.status.cpu().numpy().tolist()
    del bufs
    return out


def time_map(torch, fa, tb, p, steps, warmup):
    """Greedy (MAP) decoding of the whole batch, µs per call (fa_map_decode),
    with the max-plus tree's work: one add and one max per term, B (Lpad - 1)
    S^3 terms, against the vector ALUs' fp64 issue rate."""
    bufs = fa.map_decode(tb, p)
    for _ in range(warmup):
        fa.map_decode(tb, p, bufs)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fa.map_decode(tb, p, bufs)
    b.record()
    torch.cuda.synchronize()
    us = 1000.0 * a.elapsed_time(b) / steps
    B, L, _ = p.shape
    S = tb.info["S"]
    Lpad = 1 << max(0, (L - 1).bit_length())
    terms = float(B) * (Lpad - 1) * S ** 3
    out = dict(us_per_call=us, calls_per_s=1e6 / us, steps=steps,
               row_status=bufs.status.cpu().numpy().tolist(),
               logmax=bufs.logmax.cpu().numpy().tolist(),
               tree_terms=terms,
               tree_work_basis="B*(Lpad-1)*S^3 max-plus terms (one fp64 add + one max each)",
               valu_peak_terms_per_s=VALU_FP64_LANE_OPS / 2)
    del bufs
    return out


def generation_sweep(torch, fa, tb, p, seed, bufs, Ts):
    """Synthetic generations of T denoising steps (one constrained step and
    one remasking step each) with the constrained score (Mar) and the
    unconstrained one (Mf), each on a fresh copy of p, timed after one
    untimed run of the same T."""
    out = []
    for mode, label in ((fa.FA_CONF_PROB, "Mar"), (fa.FA_CONF_UNCONSTRAINED, "Mf")):
        for T in Ts:
            p_gen = p.clone()
            fa.generate(tb, p_gen, T, seed, conf_mode=mode, bufs=bufs)
            p_gen.copy_(p)
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record()
            _, committed = fa.generate(tb, p_gen, T, seed, conf_mode=mode, bufs=bufs)
            g1.record()
            torch.cuda.synchronize()
            ms = g0.elapsed_time(g1)
            out.append({"score": label, "T": T, "ms": ms, "ms_per_denoising_step": ms / T,
                        "generations_per_s": 1000.0 / ms,
                        "all_committed": bool((committed == 1).all().item()),
                        "row_status": bufs.status.cpu().numpy().tolist()})
            del p_gen
    return out


# --- rocprofv3 output -> committed summaries ------------------------------

def first_level_name(tb):
    """How the table forms the first span level."""
    if tb.info["first_sparse"]:
        return "sparse"
    return "dense from pair values" if tb.info["first_pairs"] else "dense"


def level1_name(tb):
    """The first tree level's kernel: sparse row combination, dense products
    staged from the pair values, or dense products over dense leaves."""
    if tb.info["first_sparse"]:
        return "span_sparse1"
    return "span_pairs_level1" if tb.info["first_pairs"] else "span_gemm_level1"


# measured kernels: how to find their dispatches in rocprofv3 output
KERNEL_MATCH = {
    "emission_dense": lambda n: "emission_dense<" in n,
    "span_sparse1": lambda n: "span_sparse<" in n,    # first level only (tree_levels)
    "span_gemm_level1": lambda n: "span_gemm" in n,
    "span_pairs_level1": lambda n: "span_pairs256" in n,
    "marg_q": lambda n: "marg_q" in n,
}
LEVEL1_KERNELS = ("span_gemm_level1", "span_sparse1", "span_pairs_level1")


def _tree_product(n):
    return "span_gemm" in n or "span_sparse<" in n or "span_pairs256" in n


def _tree_launch(n):
    return (_tree_product(n) or "span_reduce" in n or "tree_init_rf" in n or "live_reach" in n
            or "live_lists" in n)


def tree_levels(rows):
    """Dispatch id -> "L<k>" for the span tree's launches (level k of the
    step: the k-th product launch of one span tree, which starts with its
    first launch (the row-exponent initialization, the live-state lists or
    the first product) and ends at log Z; a split-K reduce takes its
    product's level), so that levels of one launch shape stay apart in the
    summaries."""
    out, level = {}, None
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        n = r["Kernel_Name"]
        if "tree_logz" in n:
            level = None
            continue
        if level is None and _tree_launch(n):
            level = 0
        if level is None:
            continue
        if _tree_product(n):
            level += 1
            out[r["Dispatch_Id"]] = f"L{level}"
        elif "span_reduce" in n and level:
            out[r["Dispatch_Id"]] = f"L{level}"
    return out


def _select(rows, name):
    """Dispatches of one measured kernel, in dispatch order; for the tree
    products only the first level's launches."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    match = KERNEL_MATCH[name]
    if name not in LEVEL1_KERNELS:
        return [r for r in rows if match(r["Kernel_Name"])]
    lv = tree_levels(rows)
    return [r for r in rows if lv.get(r["Dispatch_Id"]) == "L1" and match(r["Kernel_Name"])]


def summarize_counters(fetch_dir, write_dir, command):
    """profiles/traffic_<kernel>.json and profiles/counters_json_like_dfa.md
    from one FETCH_SIZE and one WRITE_SIZE pass (each with --copy-calib)."""
    import csv
    rows = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        path = os.path.join(d, "run_counter_collection.csv")
        rows[tag] = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == tag]
    # calibration: the 1 GiB device copy moves 2^30 bytes each way
    calib = {}
    for tag, rs in rows.items():
        kib = max(float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"])
        calib[tag] = (1 << 30) / (kib * 1024.0)
    lines = ["# HBM bytes per launch from rocprofv3 counters (json-like DFA, B=4, L=256, V=151,936)",
             "", "Command (one pass per counter, from the repository root; the 1 GiB device copy of",
             "`--copy-calib` calibrates each counter):", "", "```", command, "```", "",
             f"Calibration: FETCH_SIZE x {calib['FETCH_SIZE']:.3f}, WRITE_SIZE x {calib['WRITE_SIZE']:.3f}"
             " (bytes = counter KiB x 1024 x factor).", "",
             "| kernel | dispatch | fetch MB | write MB | traffic MB |", "|---|---|---|---|---|"]
    h = src_hash()
    for name in KERNEL_MATCH:
        mean = lambda rs: sum(float(r["Counter_Value"]) for r in rs) / len(rs)
        fsel, wsel = _select(rows["FETCH_SIZE"], name), _select(rows["WRITE_SIZE"], name)
        if not fsel or not wsel:
            continue
        kname, grid = fsel[0]["Kernel_Name"], int(fsel[0]["Grid_Size"])
        fk, wk = mean(fsel), mean(wsel)
        fb = fk * 1024.0 * calib["FETCH_SIZE"]
        wb = wk * 1024.0 * calib["WRITE_SIZE"]
        rec = dict(kernel=name, dispatch=kname[:120], grid_threads=grid, fetch_bytes=fb,
                   write_bytes=wb, bytes_per_launch=fb + wb, src_hash=h,
                   calibration=calib, command=command)
        with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        lines.append(f"| {name} | `{kname[:60]}` grid {grid} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                     f"{(fb + wb) / 1e6:.1f} |")
    with open(os.path.join(ROOT, "profiles", "counters_json_like_dfa.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


TRACE_NAMES = {
    3: ("json_like_dfa", "json-like DFA, B=4, L=256, V=151,936"),
    4: ("range_dfa", "range DFA, S=1024, B=16, L=512, V=151,936"),
    5: ("random_nfa", "random NFA, S=10,000, E=100,000, B=1, L=64, V=151,936"),
}


def summarize_trace(trace_dir, command, workload=3):
    """profiles/step_<workload>_kernel_trace.md from a --kernel-trace
    --stats run: per-kernel totals and per-launch-shape averages."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    short = lambda n: n.replace("fa::(anonymous namespace)::", "").split("(fa::")[0][:60]
    stem, title = TRACE_NAMES[workload]
    lines = [f"# Kernel trace of the constrained step ({title})", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    groups = {}
    lv = tree_levels(trace)
    for r in trace:
        k = (short(r["Kernel_Name"]), lv.get(r["Dispatch_Id"], ""), r["Grid_Size_X"], r["Grid_Size_Y"])
        groups.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Per launch shape (grid in threads; tree level of the step for the span tree's launches):", "",
              "| kernel | level | grid x | grid y | calls | avg us |", "|---|---|---|---|---|---|"]
    for k, v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:30]:
        lines.append(f"| `{k[0]}` | {k[1]} | {k[2]} | {k[3]} | {len(v)} | {sum(v) / len(v):.1f} |")
    with open(os.path.join(ROOT, "profiles", f"step_{stem}_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def summarize_mfma(pmc_dir, command, workload=3):
    """profiles/mfma_<workload>.md from one rocprofv3 --pmc pass of MfmaUtil
    (MFMA busy cycles over active cycles and SIMDs) and the executed MFMA
    operations (SQ_INSTS_VALU_MFMA_MOPS_* x 512 flops): per kernel launch shape."""
    import csv
    from collections import defaultdict
    rows = list(csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))))
    short = lambda n: n.replace("fa::(anonymous namespace)::", "").split("(fa::")[0][:60]
    agg = defaultdict(lambda: defaultdict(list))
    lv = tree_levels({r["Dispatch_Id"]: r for r in rows}.values())
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg[(short(r["Kernel_Name"]), int(r["Grid_Size"]), lv.get(r["Dispatch_Id"], ""))][r["Counter_Name"]].append(
            (float(r["Counter_Value"]), d))
    stem, title = TRACE_NAMES[workload]
    lines = [f"# MFMA utilization of the constrained step ({title})", "",
             "Command (from the repository root):", "", "```", command, "```", "",
             "MfmaUtil is rocprofv3's derived counter (summed SQ_VALU_MFMA_BUSY_CYCLES over "
             "GRBM_GUI_ACTIVE x SIMDs); the executed flops are SQ_INSTS_VALU_MFMA_MOPS_* x 512. "
             "Durations are under the counter pass.  The span products run as six bf16 products per "
             "fp32 product (the operands' three-piece split): their fp32-equivalent rate is the bf16 "
             "rate / 6.", "",
             "| kernel | level | grid threads | launches | MfmaUtil % | fp32 MFMA GFLOP | bf16 MFMA GFLOP | avg us | "
             "bf16 TFLOP/s | fp32 TFLOP/s |", "|---|---|---|---|---|---|---|---|---|---|"]
    mean = lambda xs: sum(x[0] for x in xs) / len(xs) if xs else 0.0
    for (name, grid, level), c in sorted(agg.items(), key=lambda kv: -mean(kv[1].get(
            "SQ_INSTS_VALU_MFMA_MOPS_F32", [])) - mean(kv[1].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", []))):
        mu = c.get("MfmaUtil", [])
        f32 = mean(c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", [])) * 512
        bf = mean(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [])) * 512
        if not mu or (f32 == 0 and bf == 0):
            continue
        us = sum(x[1] for x in mu) / len(mu)
        lines.append(f"| `{name}` | {level} | {grid} | {len(mu)} | {mean(mu):.1f} | {f32 / 1e9:.3f} | {bf / 1e9:.3f} | "
                     f"{us:.1f} | {bf / (us * 1e6):.1f} | {f32 / (us * 1e6):.1f} |")
    with open(os.path.join(ROOT, "profiles", f"mfma_{stem}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=3, help="preset 1..5 (default 3)")
    ap.add_argument("--first-level", choices=["auto", "sparse", "dense", "pairs"], default="auto",
                    help="form of the first span level (default: the library's choice)")
    ap.add_argument("--separate", action="store_true",
                    help="fa_sample then fa_marginals instead of fa_sample_marginals")
    ap.add_argument("--gen-steps", default="16,64,256",
                    help="denoising steps T of the timed synthetic generations, comma separated, "
                         "each with the constrained and the unconstrained score (empty: none)")
    ap.add_argument("--other-configs", default="2,4,5",
                    help="other presets timed after the headline (joint calls; empty: none)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other call form and the stage split (profiling runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run one plain device copy of 1 GiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_*.json from two rocprofv3 --pmc passes, then exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-trace summary under profiles/ from a rocprofv3 run, then exit")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="write profiles/mfma_<workload>.md from a --pmc MfmaUtil pass and exit")
    ap.add_argument("--command", default="", help="the command recorded in a summary")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.command, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(batch rows would shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    import constrained_decoding_diffusion_amd as fa
    from synth import configs

    w = configs.make(args.workload)
    tb = fa.Table.from_automaton(w.aut, first_level=args.first_level)
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

    # the library brackets one kernel per step with HIP events on its own
    # stream; the timed steps rotate over the three measured kernels
    prof_ids = [("emission_dense", fa.FA_PROF_EMISSION_DENSE),
                (level1_name(tb), fa.FA_PROF_TREE_LEVEL1),
                ("marg_q", fa.FA_PROF_MARG_Q)]
    hev = HipEvents()

    # sampling and marginals: one fa_sample_marginals call (default), or
    # fa_sample then fa_marginals (--separate); the outputs are the same, and
    # the other form is timed too, after the headline steps
    names_of = {True: ["build_transitions", "span_tree", "sample", "marginals"],
                False: ["build_transitions", "span_tree", "sample_marginals"]}
    names = names_of[args.separate]

    def one_step(seed, ev=None, kev=None, separate=args.separate):
        bufs.status.zero_()
        if kev:
            fa.profile_kernel(kev[0], kev[1], kev[2])
        if ev: ev[0].record()
        fa.build_transitions(tb, p, bufs, stream)
        if ev: ev[1].record()
        fa.span_tree(tb, bufs, stream)
        if ev: ev[2].record()
        if separate:
            fa.sample(tb, p, bufs, seed, stream)
            if ev: ev[3].record()
            fa.marginals(tb, p, bufs, fa.FA_CONF_PROB, stream, write_q=True)
        else:
            fa.sample_marginals(tb, p, bufs, seed, fa.FA_CONF_PROB, stream, write_q=True)
        if ev: ev[len(names_of[separate])].record()

    def stage_split(separate):
        """Mean µs per call over args.steps untimed steps with events
        between the calls (the events cost about 20 us per step, so they
        stay out of the timed steps)."""
        nm = names_of[separate]
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(nm) + 1)]
               for _ in range(args.steps)]
        for s in range(args.steps):
            one_step(w.seed + args.warmup + s, evs[s], separate=separate)
        torch.cuda.synchronize()
        acc = {n: 0.0 for n in nm}
        for ev in evs:
            for k, n in enumerate(nm):
                acc[n] += ev[k].elapsed_time(ev[k + 1])
        return {n: 1000.0 * v / args.steps for n, v in acc.items()}

    def timed(separate, kevs=None):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        t0.record()
        for s in range(args.steps):
            one_step(w.seed + args.warmup + s, None, kevs[s][:3] if kevs else None, separate)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), time.perf_counter() - c0

    for s in range(args.warmup):
        one_step(w.seed + s)
        if not args.headline_only:
            one_step(w.seed + s, separate=not args.separate)
    torch.cuda.synchronize()
    kevs = []
    for s in range(args.steps):
        name, pid = prof_ids[s % len(prof_ids)]
        kevs.append((pid, hev.create(), hev.create(), name))
    # the timed steps carry only the library's kernel-bracketing events,
    # which cost nothing measurable
    total_ms, wall = timed(args.separate, kevs)
    fa.profile_kernel(fa.FA_PROF_NONE)
    if args.headline_only:
        other_ms, stage_us, other_stage_us = None, None, None
    else:
        other_ms, _ = timed(not args.separate)
        stage_us = stage_split(args.separate)
        other_stage_us = stage_split(not args.separate)
    gen = None
    if not args.headline_only and args.gen_steps:
        Ts = [int(t) for t in args.gen_steps.split(",") if int(t) > 0]
        gen = {"positions_per_step": f"ceil(masked / steps left), all {w.L} after T",
               "runs": generation_sweep(torch, fa, tb, p, w.seed, bufs, Ts)}
    kern_us = {}
    for pid, a, b, name in kevs:
        ms = hev.elapsed_ms(a, b)
        if ms is not None:
            kern_us.setdefault(name, []).append(1000.0 * ms)
        hev.destroy(a)
        hev.destroy(b)
    kern_us = {k: sum(v) / len(v) for k, v in kern_us.items()}
    ms_per_step = total_ms / args.steps
    status = bufs.status.cpu().numpy()

    work = algorithmic_work(tb, w.B, w.L)
    stages = None if stage_us is None else stage_fracs(work, stage_us, args.separate)
    kernels = {}
    for name, us in kern_us.items():
        kw = work["kernels"][name]
        if kw["bound"] == "hbm":
            achieved, peak = kw["work"] / (us * 1e3), HBM_PEAK_GBS
        else:
            achieved, peak = kw["work"] / (us * 1e6), kw.get("peak", FP32_MFMA_PEAK_TFLOPS)
        tr = traffic_record(name)
        kernels[name] = dict(bound=kw["bound"], achieved=achieved, peak=peak, unit=kw["unit"],
                             frac=achieved / peak, avg_launch_us=us, work_per_launch=kw["work"],
                             work_basis=kw["per_unit"],
                             traffic=(tr["bytes_per_launch"] if tr else None))
    dominant = max(kernels, key=lambda k: kernels[k]["avg_launch_us"])
    roof = dict(kernels[dominant], kernel=dominant)
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
                   "calls": "separate" if args.separate else "joint",
                   "first_level": first_level_name(tb),
                   "sequence_steps_per_s": w.B * 1000.0 / ms_per_step},
        "roofline": roof,
        "kernels": kernels,
        "stages": stages,
        "generation": gen,
        "other_form": None if other_ms is None else {
            "calls": "joint" if args.separate else "separate",
            "us_per_step": 1000.0 * other_ms / args.steps,
            "steps_per_s": 1000.0 * args.steps / other_ms,
            "stages_us": other_stage_us},
        "wall_s": wall,
        "row_status": status.tolist(),
    }
    if not args.headline_only:
        out["ceiling"] = ceilings(torch, fa, dev, p)
        Lpad = 1 << max(0, (w.L - 1).bit_length())
        if w.B * (Lpad - 1) * tb.info["S"] ** 3 <= 1e12:  # at most 1e12 max-plus terms (the batch DFA: with its preset)
            out["map_decode"] = time_map(torch, fa, tb, p, args.steps, args.warmup)
        out["chain_vs_tree"] = time_chain_vs_tree(torch, fa, tb, p, w.seed, args.steps, args.warmup,
                                                  w.aut)
    del bufs, p
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.headline_only and args.other_configs:
        others = {}
        for k in [int(x) for x in args.other_configs.split(",")]:
            if k == args.workload:
                continue
            # the large presets take fewer steps; the batch DFA draws p on the device
            n = args.steps if k <= 3 else 5
            # greedy decoding over the batch DFA's range labels: two calls
            # (about a second each: B (Lpad - 1) S^3 = 8.8e12 max-plus terms)
            others[f"preset{k}"] = time_workload(torch, fa, configs, k, n, 3 if k > 3 else args.warmup,
                                                 dev, device_p=(k == 4), map_calls=2 if k == 4 else 0)
            if k == 4:
                # its committed positions leave about a third of the states
                # live per boundary: the same preset with FA_LIVE_STATES
                others["preset4_live_states"] = time_workload(torch, fa, configs, k, n, 3, dev,
                                                              device_p=True, live=True, chain=False)
        out["configs"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
