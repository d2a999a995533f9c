"""Benchmark: forward pass of one LLaMA-MoE-3.5B (2/8) MoE layer on one MI355X.

Workload: T = 4096 tokens (batch 1 x sequence 4096), hidden 4096, LLaMA-2-7B
intermediate 11008 split into 8 experts of 1376, top-2 Mixtral routing,
dropless, output rescaled by N/k = 4; bf16 activations and expert weights,
fp32 router. Seeded synthetic inputs (no checkpoint or dataset), resident in
HBM before timing. A step is one moe_forward call (router, KeepTopK and gates,
permutation, both grouped expert GEMMs, combine). Steps rotate over several
copies of the layer's inputs so the 256 MB last-level cache cannot keep a
step's weights from the previous step.

Prints one JSON line (rank 0). `value` is tokens/s of the whole job; the
`roofline` object covers the dominant kernel (the fused gate/up GEMM with the
SwiGLU epilogue), timed with HIP events on its launch stream inside the timed
region; `cpu_baseline` is the CPU oracle timed on this host on a sample of the
same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec and % of bf16 MFMA peak, LLaMA-MoE-3.5B 2/8 shape"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "experts_fused_C2_counters.txt")
GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_05_amd", "csrc", "gemm_mfma.hip")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--ramp-ms", type=float, default=150.0,
                    help="untimed steps for at least this long before the warmup steps (clock ramp)")
    ap.add_argument("--copies", type=int, default=3, help="input copies the steps rotate over")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain 512 MiB device copy first (counter calibration under rocprofv3)")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--config", default="C2",
                    help="workload: C2 (the headline LLaMA-MoE-3.5B 2/8 layer) or one of the other layer shapes")
    return ap.parse_args()


def counters_traffic():
    """HBM bytes per launch of the fused expert kernel from the committed rocprofv3 counter summary,
    or None if there is none or the kernel source changed since it was taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    txt = open(COUNTERS_FILE).read()
    kv = dict(re.findall(r"^([a-z_0-9]+):\s*(\S+)\s*$", txt, flags=re.M))
    src_hash = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


WORKLOADS = {
    "C1": ("tiny fp32 MoE layer: T=256, hidden 256, 688 split into 8 experts of 86, top-2 Mixtral, dropless",
           lambda synth: synth.c1()),
    "C2": ("LLaMA-MoE-3.5B (2/8) MoE layer forward: T=4096 tokens, hidden 4096, 11008 split into 8 experts of "
           "1376, top-2 Mixtral, dropless, s=N/k=4, bf16 experts, fp32 router", lambda synth: synth.c2()),
    "C3": ("LLaMA-MoE-3.5B (4/16) MoE layer forward: T=4096, hidden 4096, 11008 split into 16 experts of 688, "
           "top-4 noisy gate with stats, dropless, s=4", lambda synth: synth.c3()),
    "C4cf4": ("Llama-3-8B upcycled E8T2 layer: T=8192, hidden 4096, 8 experts of 14336, top-2 Mixtral, "
              "capacity factor 4 (C=4096)", lambda synth: synth.c4("cf4")),
    "C4cf1": ("Llama-3-8B upcycled E8T2 layer: T=8192, 8 experts of 14336, top-2, capacity factor 1 (C=1024)",
              lambda synth: synth.c4("cf1")),
    "C4dropless": ("Llama-3-8B upcycled E8T2 layer: T=8192, 8 experts of 14336, top-2, dropless",
                   lambda synth: synth.c4("dropless")),
    "C4cf1_assign": ("Llama-3-8B upcycled E8T2 layer: T=8192, 8 experts of 14336, top-2, capacity factor 1 "
                     "counted per assignment (C=2048)", lambda synth: synth.c4("cf1_assign")),
    "C2res": ("LLaMA-MoE-3.5B-shape residual (shared-neuron Inter mode) layer: T=4096, hidden 4096, 11008 neurons = "
              "1376 shared + 7 routed experts of 1376, top-2 Mixtral, dropless, s=1",
              lambda synth: synth.make_residual("C2res", 1007, 4096, 4096, 11008, 1376, 7, 2, out_scale=1.0)),
    "C2train": ("LLaMA-MoE-3.5B (2/8) MoE layer training step (forward that keeps its activations, then the "
                "backward: dx, router and expert weight gradients, balance-loss gradient 0.01): T=4096, hidden "
                "4096, 8 experts of 1376, top-2 Mixtral, dropless, s=4", lambda synth: synth.c2()),
    "C3train": ("LLaMA-MoE-3.5B (4/16) MoE layer training step: T=4096, 16 experts of 688, noisy top-4, stats, "
                "balance-loss gradient 0.01, s=4", lambda synth: synth.c3()),
    "C5": ("decode-shaped E8T2 layer: T=64 tokens, hidden 4096, 8 experts of 14336, top-2, half the tokens "
           "steered to expert 0, dropless", lambda synth: synth.c5()),
}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the MoE layer runs on a single MI355X and there is no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.config not in WORKLOADS:
        print(f"unknown --config {args.config}; one of {', '.join(WORKLOADS)}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from sparse_mixture_experts_05_amd import abi

    torch.cuda.set_device(0)
    abi.load_library()
    dev_name = torch.cuda.get_device_name(0)

    if args.calib_copy:
        n = 512 * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    headline = args.config == "C2"
    desc, make = WORKLOADS[args.config]
    w = make(synth)
    T, H, F, N, k = w.T, w.H, w.F, w.N, w.k
    cfg = abi.MoEConfig(T=T, H=H, F=F, N=N, k=k, capacity=w.capacity, order=w.order, noisy=w.noisy,
                        want_stats=w.want_stats, out_scale=w.out_scale, act=w.act, wt=w.wt)
    bf16 = w.act == "bf16"

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    base = dict(x=dev(w.x), Wg=dev(w.Wg), Wn=dev(w.Wn), eps=dev(w.eps), Wgate=dev(w.Wgate), Wup=dev(w.Wup),
                Wdown=dev(w.Wdown))
    copies = [base] + [{k_: (v.clone() if v is not None else None) for k_, v in base.items()}
                       for _ in range(max(0, args.copies - 1))]
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    kept = torch.zeros(N, dtype=torch.int32, device="cuda")
    stats = dict(load=torch.empty(N, dtype=torch.int32, device="cuda"),
                 importance=torch.empty(N, dtype=torch.float32, device="cuda"),
                 P=torch.empty(N, dtype=torch.float32, device="cuda"),
                 balance=torch.empty(1, dtype=torch.float32, device="cuda")) if w.want_stats else {}
    Fs = w.shared[0].shape[0] if w.shared is not None else 0
    train = args.config.endswith("train")
    if Fs:
        shared = [tuple(dev(a) for a in w.shared) for _ in range(len(copies))]
        ws = torch.empty(abi.moe_residual_workspace_bytes(cfg, Fs), dtype=torch.uint8, device="cuda")
    elif train:
        ws = torch.empty(abi.moe_train_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        dy = dev(synth.normal_f32(w.meta["seed"], 40, (T, H), 1.0))
        grads = dict(dx=torch.empty(T, H, device="cuda"), dWg=torch.empty(H, N, device="cuda"),
                     dWn=torch.empty(H, N, device="cuda") if w.noisy else None,
                     dWgate=torch.empty(N, F, H, device="cuda"), dWup=torch.empty(N, F, H, device="cuda"),
                     dWdown=torch.empty(N, H, F, device="cuda"))
    else:
        ws = abi.workspace(cfg)
    stream = torch.cuda.current_stream()

    def step(i, d=None):
        j = i % len(copies)
        d = d if d is not None else copies[j]
        if train:
            abi.moe_forward_train(cfg, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"], y,
                                  kept=kept, ws=ws, stream=stream, **stats)
            abi.moe_backward(cfg, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"], dy, 0.01,
                             grads["dx"], grads["dWg"], grads["dWn"], grads["dWgate"], grads["dWup"],
                             grads["dWdown"], ws=ws, stream=stream)
        elif Fs:
            abi.moe_forward_residual(cfg, Fs, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"],
                                     *shared[j], y, kept=kept, ws=ws, stream=stream, **stats)
        else:
            abi.moe_forward(cfg, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"], y,
                            kept=kept, ws=ws, stream=stream, **stats)

    # one step first: the kept counts, and whether the library runs the
    # expert GEMMs as one persistent launch (the dominant kernel) or as two
    # launches (then the gate/up GEMM with the SwiGLU epilogue dominates)
    abi.moe_profile_select(abi.MOE_KERNEL_EXPERTS)
    abi.moe_profile_read()
    step(0)
    torch.cuda.synchronize()
    fused = abi.moe_profile_read()[1] > 0
    dom_id = abi.MOE_KERNEL_EXPERTS if fused else abi.MOE_KERNEL_GEMM1
    if train:
        # a training step runs three expert-GEMM kernels: the forward's experts
        # (6*A*H*F flops), the backward's input-gradient launch with dWdown
        # (8*A*H*F) and the launch of dWgate and dWup (4*A*H*F): the
        # dominant one is the slowest of them per step
        per_step = {}
        for kid in (abi.MOE_KERNEL_EXPERTS, abi.MOE_KERNEL_BWD_DGRAD, abi.MOE_KERNEL_BWD_WGRAD):
            abi.moe_profile_select(kid)
            abi.moe_profile_read()
            for i in range(4):
                step(i)
            torch.cuda.synchronize()
            per_step[kid] = abi.moe_profile_read()[0] / 4
        dom_id = max(per_step, key=per_step.get)
    abi.moe_profile_select(-1)
    kept_h = kept.cpu().numpy().astype(np.int64)
    A = int(kept_h.sum())                    # kept (token, expert) rows
    active = int((kept_h > 0).sum())          # experts with at least one row

    # the GPU reaches its steady clock only after tens of milliseconds of
    # load: run untimed steps (same rotating inputs) for args.ramp_ms first,
    # then the warmup steps, then the timed steps right after
    t_ramp = time.perf_counter()
    i = 0
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)

    # timed region; the dominant kernel bracketed by HIP events on the launch stream
    # (per-step durations from events recorded between the steps on the
    # launch stream, for the median and the 10th/90th percentiles)
    abi.moe_profile_select(dom_id)
    abi.moe_profile_read()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step(i)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    abi.moe_profile_select(-1)
    dom_ms, dom_n = abi.moe_profile_read()
    step_ms = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    t_layer = elapsed / args.steps
    # the residual layer launches the expert kernel twice a step (shared
    # slice, then the routed experts): its roofline covers both launches
    dom_avg_s = dom_ms / 1e3 / max(1, dom_n) * (2 if Fs else 1)
    if train:  # per step: the dgrad kernel launches twice, the weight-gradient kernel three times
        dom_avg_s = dom_ms / 1e3 / args.steps

    # layer roofline over the kept assignments: expert flops on the matrix
    # cores plus the fp32 router, or the bytes of reading x, the router
    # weights, the active experts' weights once, the routing outputs, and
    # writing fp32 y once, whichever takes longer
    eb = 2 if bf16 else 4
    f_expert = (18.0 if train else 6.0) * A * H * F + 6.0 * T * H * Fs
    f_router = 2.0 * T * H * N * (2 if w.noisy else 1)
    b_alg = (T * H * eb + H * N * 4 * (2 if w.noisy else 1) + (T * N * 4 if w.noisy else 0)
             + active * 3 * F * H * eb + 3 * Fs * H * eb + T * k * 8 + T * H * 4)
    if train:  # the backward reads dy and the weights again and writes dx and every gradient in fp32
        b_alg += T * H * 4 + active * 3 * F * H * eb + T * H * 4 + active * 3 * F * H * 4 + H * N * 4 * (2 if w.noisy else 1)
    peak_expert = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    t_compute = f_expert / (peak_expert * 1e12) + f_router / (PEAK_FP32_TFLOPS * 1e12)
    t_mem = b_alg / (PEAK_HBM_GBS * 1e9)
    t_roof = max(t_compute, t_mem)

    # dominant kernel's algorithmic work per launch: the fused launch does
    # 6*A*H*F flops and reads the active experts' three matrices; the gate/up
    # GEMM alone does 4*A*H*F and reads two of them
    if train:
        dom_name = {abi.MOE_KERNEL_EXPERTS: "experts_fused_forward",
                    abi.MOE_KERNEL_BWD_DGRAD: "backward_input_gradients_and_dWdown",
                    abi.MOE_KERNEL_BWD_WGRAD: "backward_dWgate_dWup"}[dom_id]
        # per launch
        dom_flops = {abi.MOE_KERNEL_EXPERTS: 6.0, abi.MOE_KERNEL_BWD_DGRAD: 8.0,
                     abi.MOE_KERNEL_BWD_WGRAD: 4.0}[dom_id] * A * H * F
        dom_bytes = {abi.MOE_KERNEL_EXPERTS: 3, abi.MOE_KERNEL_BWD_DGRAD: 3,
                     abi.MOE_KERNEL_BWD_WGRAD: 0}[dom_id] * active * F * H * eb + A * H * eb
    elif fused:
        dom_name = "experts_gate_up_swiglu_down"
        dom_flops = 6.0 * A * H * F + 6.0 * T * H * Fs
        dom_bytes = active * 3 * F * H * eb + A * H * eb + A * H * 4 + 3 * Fs * H * eb + T * H * eb + T * H * 4
    else:
        dom_name = "gemm1_gate_up_swiglu"
        dom_flops = 4.0 * A * H * F
        dom_bytes = active * 2 * F * H * eb + A * H * eb + A * F * eb
    if t_mem > t_compute:
        achieved = dom_bytes / dom_avg_s / 1e9
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None, "bytes_per_launch": dom_bytes}
    else:
        achieved = dom_flops / dom_avg_s / 1e12
        roof = {"bound": "mfma" if bf16 else "alu", "kernel": dom_name, "achieved": round(achieved, 1),
                "peak": peak_expert, "unit": "TFLOP/s", "frac": round(achieved / peak_expert, 4),
                "traffic": counters_traffic() if headline else None, "flops_per_launch": dom_flops}
    roof.update(launches_timed=dom_n, avg_launch_us=round(dom_avg_s * 1e6, 2))

    detail = None
    if not args.no_detail:
        per_kernel = {}
        names = {abi.MOE_KERNEL_ROUTER: "router_topk", abi.MOE_KERNEL_STATS: "router_stats",
                 abi.MOE_KERNEL_SCATTER: "permute_scatter", abi.MOE_KERNEL_GEMM1: "gemm1_gate_up_swiglu",
                 abi.MOE_KERNEL_GEMM2: "gemm2_down", abi.MOE_KERNEL_EXPERTS: "experts_fused",
                 abi.MOE_KERNEL_COMBINE: "combine", abi.MOE_KERNEL_BWD_GATE: "bwd_gate",
                 abi.MOE_KERNEL_BWD_DGRAD: "bwd_dgrad",
                 abi.MOE_KERNEL_BWD_DX: "bwd_dx", abi.MOE_KERNEL_BWD_WGRAD: "bwd_wgrad",
                 abi.MOE_KERNEL_BWD_ROUTER: "bwd_router_wgrad"}
        for kid, name in names.items():
            abi.moe_profile_select(kid)
            for i in range(10):
                step(i)
            torch.cuda.synchronize()
            ms, n = abi.moe_profile_read()
            if n:
                per_kernel[name] = round(ms * 1e3 / (10 if train else n), 2)  # train: per step
        abi.moe_profile_select(-1)
        # same data every step: weights can stay in the last-level cache
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            step(i, copies[0])
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        g2 = per_kernel.get("gemm2_down")
        # per-step HBM rates of the data-movement steps from their own bytes:
        # the combine reads every kept fp32 y_perm row and the routing and
        # writes fp32 y; the scatter reads topk_idx and the per-block
        # histogram and writes slot and row_token (the x rows are gathered
        # inside the gate/up GEMM, so no x_perm is written)
        comb_b = A * H * 4 + T * k * 8 + T * H * 4
        scat_b = T * k * 4 + ((T + 15) // 16) * N * 4 + T * k * 4 + A * 4
        step_gbs = {name: round(b / (per_kernel[name] * 1e-6) / 1e9, 1)
                    for name, b in (("combine", comb_b), ("permute_scatter", scat_b)) if per_kernel.get(name)}
        detail = dict(device=dev_name, kept_rows=A, active_experts=active, kept_per_expert=kept_h.tolist(),
                      kernel_avg_us=per_kernel, layer_us=round(t_layer * 1e6, 2),
                      layer_tflops=round((f_expert + f_router) / t_layer / 1e12, 1),
                      layer_hbm_gbs=round(b_alg / t_layer / 1e9, 1),
                      layer_roofline_us=round(t_roof * 1e6, 2), layer_bound="hbm" if t_mem > t_compute else "compute",
                      layer_frac_of_roofline=round(t_roof / t_layer, 4),
                      gemm2_tflops=round(2.0 * A * F * H / (g2 * 1e-6) / 1e12, 1) if g2 else None,
                      step_bytes={"combine": comb_b, "permute_scatter": scat_b}, step_gbs=step_gbs,
                      same_inputs_every_step_ms=round(warm_ms, 4), input_copies=len(copies))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no checkpoint)",
        "config": {"workload": desc, "T": T, "H": H, "F": F, "N": N, "k": k, "capacity": w.capacity,
                   "out_scale": w.out_scale},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if detail is not None:
        out["detail"] = detail
    print(json.dumps(out), flush=True)


def cpu_baseline(w, target_s: float):
    """The CPU oracle, as it is, on the first S tokens of the workload (same
    weights): routing, capacity and the expert FFNs of those tokens, with the
    token loop on this host's cores. S is sized for about target_s seconds."""
    import oracle
    import synth

    # threads: this process's CPU share (its affinity mask), at most 16, the
    # share of one GPU on a shared host; the host's own count is reported too
    host_cpus = os.cpu_count() or 1
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = host_cpus
    cores = max(1, min(16, share))

    def sample(S):
        return synth.Workload(w.name, S, w.H, w.F, w.N, w.k, w.capacity, w.order, w.noisy, False, w.out_scale,
                              w.act, w.wt, w.x[:S].copy(), w.Wg, w.Wn, None if w.eps is None else w.eps[:S].copy(),
                              w.Wgate, w.Wup, w.Wdown, shared=w.shared)

    def run(v, nthreads):
        if v.shared is not None:
            return oracle.residual_forward(v, nthreads=nthreads)
        return oracle.forward(v, nthreads=nthreads)

    S0 = max(cores, 16)
    t0 = time.perf_counter()
    run(sample(S0), cores)
    dt0 = time.perf_counter() - t0
    S = int(min(w.T, max(S0, S0 * target_s / max(dt0, 1e-3))))
    S = max(cores, S // cores * cores)
    t1 = time.perf_counter()
    run(sample(S), cores)
    dt = time.perf_counter() - t1
    # the same oracle on one thread, on a sample a core count smaller
    S1 = max(1, S // cores)
    t2 = time.perf_counter()
    run(sample(S1), 1)
    dt1 = time.perf_counter() - t2
    return {"value": round(S / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host_cpus": host_cpus, "affinity_cpus": share,
            "sample": f"first {S} of {w.T} tokens of the same layer (routing, capacity and experts of those "
                      f"tokens), fp64 accumulation, {dt:.1f} s",
            "single_thread": {"value": round(S1 / dt1, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"first {S1} tokens, {dt1:.1f} s"}}


if __name__ == "__main__":
    main()
