"""Benchmark of the TQP routed-expert layer on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
route -> permute -> expert FFNs -> combine -> adapter-only backward, at
T=8192 tokens, d=2048, E=460 experts, top-12, d_ff=768, int4 group-128 base,
rank-16 adapters, bf16 activations (the 8K-context, 460-expert, top-12
setting of "Reversible Foundations: Training a 120B Sparse MoE through
State-Preserving Scaling", abstract; hidden sizes are this library's).

Prints one JSON line.  `value` is tokens/s of the timed steps with every input
already resident in device memory.  `roofline` reports the longest of the four
int4 expert-GEMM stages per step (each stage is one launch at this batch size,
timed with HIP events on the launch stream) against the bf16 matrix-core
peak; `stages` lists all four, and `traffic` comes from the committed
FETCH_SIZE/WRITE_SIZE summary of that stage while the kernel sources match.  `decode` measures the
T=64 forward (the weight-streaming shape) against HBM bandwidth, with the
device caches scrubbed before every timed forward; `decode_int8` the same
with an int8 base (twice the weight bytes).  `cpu_baseline` times the
fp64 oracle on a bounded sample of the workload on this host's cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-extras] [--no-decode]
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

from sparse_moe_expert_fp32_amd import configs, inputs  # noqa: E402

PEAK_BF16 = 2.5e15      # dense bf16 matrix-core FLOP/s of MI355X
PEAK_HBM = 8.0e12       # HBM3E bytes/s
METRIC = "TQP MoE-layer tokens/s, E=460 top-12, T=8192; % of MFMA/HBM roofline"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The four int4 expert-GEMM stages: (timer tag, name, algorithmic FLOPs per
# routed slot).  The adapter term's second factor is counted where it is
# fused (the rank-r product into the same accumulator); the adapter
# projections X A^T and the adapter gradients run in their own kernels.
def gemm_stages(cfg, train: bool):
    d, f, r = cfg.d, cfg.f, cfg.r
    st = [("gateup", "gate/up expert GEMM + SwiGLU (grouped_gemm_kernel<0,...>)", 4.0 * f * (d + r)),
          ("down", "down expert GEMM (grouped_gemm_kernel<1,...>)", 2.0 * d * (f + r))]
    if train:
        st += [("bwd_down", "backward dH + SwiGLU backward (grouped_gemm_t_kernel<0,...>)",
                2.0 * f * (d + r)),
               ("bwd_gateup", "backward dX_perm (grouped_gemm_t_kernel<1,...>)", 4.0 * d * (f + r))]
    return st


def layer_flops(cfg, train: bool) -> float:
    S = cfg.T * cfg.k
    fwd = S * (6.0 * cfg.d * cfg.f + 6.0 * cfg.r * (cfg.d + cfg.f))
    if not train:
        return fwd
    return fwd + S * (6.0 * cfg.d * cfg.f + 12.0 * cfg.r * (cfg.d + cfg.f))


def kernel_sources_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_expert_fp32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; None otherwise."""
    path = os.path.join(PROFILES, f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_hash") != kernel_sources_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, inp, target_s: float, gpu_idx=None):
    """The fp64 oracle (as it stands) on a bounded sample of the workload,
    extrapolated to the whole step: the routing of every token (timed whole),
    the expert work (dequantisation, forward and, for a training step, the
    adapter backward) of whole experts in a seeded random order until about
    target_s seconds, scaled by all slots over the slots done, and the
    combine and gate path of 1024 tokens, scaled by T / 1024.  Whole experts
    keep the per-expert dequantisation amortised over that expert's real
    load, as in the full step.  Also reports the routing check: near-tie
    tokens of the fp64 logits, and tokens where the GPU's selection differs
    outside them."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    lam, k = cfg.lora_scale, cfg.k
    with threadpool_limits(cores):
        t0 = time.perf_counter()
        R = oracle.route(inp, k)
        t_route = time.perf_counter() - t0
        order = np.random.default_rng(0).permutation(cfg.E)
        done_slots, n_exp, t_exp = 0, 0, 0.0
        for e in order:
            if R["counts"][e] == 0:
                continue
            t0 = time.perf_counter()
            oracle.expert_rows(inp, R, int(e), k, cfg.group, lam, backward=cfg.train)
            t_exp += time.perf_counter() - t0
            done_slots += int(R["counts"][e])
            n_exp += 1
            if t_exp >= target_s:
                break
        Tc = min(cfg.T, 1024)
        O = np.zeros((Tc * k, cfg.d))
        sp = np.arange(Tc * k, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.combine(R["gates"][:Tc], O, sp)
        if cfg.train:
            oracle.gate_backward(inp["dy"][:Tc], O, R["gates"][:Tc], R["topk_idx"][:Tc], sp,
                                 inp["w_router"])
        t_tok = (time.perf_counter() - t0) * cfg.T / Tc
    S = cfg.T * k
    total = t_route + t_exp * S / done_slots + t_tok
    rec = {"value": cfg.T / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"fp64 oracle, {'forward + adapter backward' if cfg.train else 'forward'}: "
                     f"routing of all {cfg.T} tokens {t_route:.1f} s; all slots of {n_exp} of "
                     f"{cfg.E} experts ({done_slots} of {S} slots) {t_exp:.1f} s, scaled by "
                     f"{S / done_slots:.1f}; combine/gate path of {Tc} tokens scaled by "
                     f"{cfg.T / Tc:.0f}; whole step {total:.0f} s extrapolated"}
    b, o = oracle.near_ties(R["logits"], k)
    routing = {"near_ties": int((b | o).sum())}
    if gpu_idx is not None:
        diff = ~np.all(gpu_idx == R["topk_idx"], axis=1)
        routing["gpu_differs"] = int(diff.sum())
        routing["gpu_differs_outside_near_ties"] = int((diff & ~(b | o)).sum())
    return rec, routing


def decode_hbm(args, B, DeviceLayer, to_numpy, bits=4):
    """The T=64 decode shape (E=460, top-12, unbiased router): forward only,
    each timed forward preceded (outside its events) by a read of 1 GiB, four
    times the 256 MB last-level cache, so the expert weights stream from HBM.
    (A write of the same size leaves the cache full of dirty lines that the
    forward's first reads must write back, 256 MB of traffic that is not the
    forward's; that time is reported beside it, and so is the int4 forward
    run over three weight sets in turn with no scrub at all.)  Bytes are
    algorithmic: the
    int4 (or int8) base, bf16 group scales and adapters of the experts the
    seeded routing touches, plus the router, x and y."""
    import torch
    cfg = configs.C4 if bits == 4 else configs.C4.with_(name=configs.C4.name + "_int8", bits=8)
    inp = inputs.generate(cfg, args.seed)
    L = DeviceLayer(cfg, inp, device="cuda:0", with_backward=False)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        L.forward()
    torch.cuda.synchronize()
    scrub = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    n = max(10, args.steps)

    def timed(write_scrub):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        sink = torch.zeros(n, dtype=torch.int64, device="cuda:0")
        for i, (a, b) in enumerate(ev):
            if write_scrub:
                scrub.fill_(1)
            else:
                sink[i] = scrub.sum()
            a.record(stream)
            L.forward()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev), ev

    cold, ev = timed(False)
    cold_w, _ = timed(True)
    # (int4) the same routing over three sets of expert weights in turn, no
    # scrub: each forward reads weights the other two sets have evicted
    rotated = None
    if bits == 4:
        sets = [L]
        for i in (1, 2):
            other = inputs.generate(cfg, args.seed + 1000 + i)
            mixed = {key: (other[key] if key.split("_")[0] in ("q", "s", "A", "B") else v)
                     for key, v in inp.items()}
            sets.append(DeviceLayer(cfg, mixed, device="cuda:0", with_backward=False))
        for S_ in sets:
            S_.forward()
        torch.cuda.synchronize()
        evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(3 * n)]
        for i, (a, b) in enumerate(evr):
            a.record(stream)
            sets[i % 3].forward()
            b.record(stream)
        torch.cuda.synchronize()
        rt = sorted(a.elapsed_time(b) for a, b in evr)
        rotated = rt[len(rt) // 2]
        del sets
    a, b = ev[0]
    a.record(stream)
    for _ in range(n):
        L.forward()
    b.record(stream)
    torch.cuda.synchronize()
    warm = a.elapsed_time(b) / n
    counts = to_numpy(L.counts)
    touched = int((counts > 0).sum())
    d, f, r, g = cfg.d, cfg.f, cfg.r, cfg.group
    per_expert = 3 * d * f * bits // 8 + 3 * (d * f // g) * 2 + 3 * r * (d + f) * 2
    nbytes = touched * per_expert + d * cfg.E * 4 + 2 * cfg.T * d * 2
    med = cold[len(cold) // 2]
    del scrub, L
    return {"workload": f"{cfg.name} forward (T={cfg.T}, E={cfg.E}, top-{cfg.k}, "
                        f"unbiased router, int{bits} base)",
            "ms": med, "ms_p10": cold[len(cold) // 10], "ms_p90": cold[(9 * len(cold)) // 10],
            "ms_warm_cache": warm, "ms_after_write_scrub": cold_w[len(cold_w) // 2],
            "ms_three_weight_sets_in_turn": rotated,
            "tokens_per_s": cfg.T / (med / 1e3),
            "experts_touched": touched, "bytes": nbytes, "bytes_per_expert": per_expert,
            "GB_s": nbytes / (med / 1e3) / 1e9, "frac_hbm": nbytes / (med / 1e3) / PEAK_HBM,
            "scrub": "1 GiB read before each timed forward, outside its events"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=configs.C5.name, choices=sorted(configs.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the reversible-replay and growth measurements (kernel "
                         "profiles of the layer step alone)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the T=64 decode-shape HBM measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic that calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "built and measured on a single MI355X and has no multi-GPU path.", flush=True)
        sys.exit(2)

    import torch
    from sparse_moe_expert_fp32_amd import binding as B
    from sparse_moe_expert_fp32_amd.layer import DeviceLayer, grow_inputs, to_numpy

    cfg = configs.CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = inputs.generate(cfg, args.seed)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    L = DeviceLayer(cfg, inp, device="cuda:0")
    step = L.train_step if cfg.train else L.forward
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    # timed region: K steps between two events on the launch stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms = total_ms / args.steps
    tokens_per_s = cfg.T / (ms / 1e3)
    log(f"{ms:.3f} ms/step, {tokens_per_s:.4g} tokens/s")

    # each int4 expert-GEMM stage timed on its own pass over K more steps:
    # the library brackets the stage (one launch) with a pair of HIP events
    stages = []
    for tag, name, flops_slot in gemm_stages(cfg, cfg.train):
        B.moe_timer_start(tag)
        for _ in range(args.steps):
            step()
        k_ms, n = B.moe_timer_stop()
        per = k_ms / max(1, n)
        flops = flops_slot * cfg.T * cfg.k
        stages.append({"stage": tag, "kernel": name, "ms": per, "flops": flops,
                       "tflops": flops / (per / 1e3) / 1e12,
                       "frac": flops / (per / 1e3) / PEAK_BF16, "spans_per_step": n / args.steps})
        log(f"stage {tag}: {per:.3f} ms, {stages[-1]['frac']:.3f} of bf16 peak")
    dom = max(stages, key=lambda x: x["ms"])

    # forward-only rate of the same inputs (context)
    ev0.record(stream)
    for _ in range(args.steps):
        L.forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = ev0.elapsed_time(ev1) / args.steps

    # adapter optimizer step (AdamW over the six adapters through
    # moe_adamw_step), timed on its own after the layer steps
    adamw = None
    if cfg.train:
        L.init_optimizer()
        for _ in range(2):
            L.optimizer_step()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            L.optimizer_step()
        ev1.record(stream)
        torch.cuda.synchronize()
        opt_ms = ev0.elapsed_time(ev1) / args.steps
        n_par = sum(t[0].numel() for t in L.opt.values())
        nbytes = n_par * (16 + 12 + 2)   # read p, g, m, v; write p, m, v and the bf16 copy
        adamw = {"ms": opt_ms, "params": n_par, "bytes": nbytes,
                 "GB_s": nbytes / (opt_ms / 1e3) / 1e9, "frac_hbm": nbytes / (opt_ms / 1e3) / PEAK_HBM}
        log(f"adamw {opt_ms:.3f} ms for {n_par} adapter parameters")

    # reversible residual block around the layer: the backward's replay
    # x2 = y2 - MoE(y1), i.e. the layer forward recomputed from y1 and the
    # coupling (moe_rev_couple), timed on its own; the reconstruction error
    # is against the x2 the forward coupling started from
    reversible = growth = None
    if not args.no_extras:
        act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        gen = torch.Generator().manual_seed(7)
        x2 = torch.randn(cfg.T, cfg.d, generator=gen).to(L.dev).to(act)
        y2, back = torch.empty_like(x2), torch.empty_like(x2)
        L.rev_forward(x2, y2)
        L.rev_inverse(y2, back)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            L.rev_inverse(y2, back)
        ev1.record(stream)
        torch.cuda.synchronize()
        rev_ms = ev0.elapsed_time(ev1) / args.steps
        rerr = (back.float() - x2.float()).abs()
        reversible = {"replay_ms": rev_ms, "x2_max_abs_err": float(rerr.max()),
                      "x2_exact_fraction": float((rerr == 0).float().mean())}
        log(f"reversible replay {rev_ms:.3f} ms, x2 max abs error {float(rerr.max()):.3e}")

        # few -> many growth (moe_grow_copy, moe_grow_router): the transform of
        # this layer to twice the experts, timed, and the grown layer's forward
        # (twice k, unperturbed router) against the original output
        ev0.record(stream)
        cfg2, g2 = grow_inputs(L.t, cfg, 2)
        ev1.record(stream)
        torch.cuda.synchronize()
        grow_ms = ev0.elapsed_time(ev1)
        y_orig = L.y.float().clone()
        L2 = DeviceLayer(cfg2, g2, device=L.dev, with_backward=False)
        L2.forward()
        torch.cuda.synchronize()
        growth = {"factor": 2, "experts": cfg2.E, "top_k": cfg2.k, "transform_ms": grow_ms,
                  "forward_rel_l2_vs_original": float((L2.y.float() - y_orig).norm() / y_orig.norm())}
        log(f"growth x2: {grow_ms:.3f} ms, grown forward rel L2 vs original "
            f"{growth['forward_rel_l2_vs_original']:.2e}")
        del L2, g2

    traffic = measured_traffic(dom["stage"])
    counts = to_numpy(L.counts)
    gpu_idx = to_numpy(L.topk_idx)
    decode = decode8 = None
    if not args.no_decode:
        for bits in (4, 8):
            t0 = time.perf_counter()
            dec = decode_hbm(args, B, DeviceLayer, to_numpy, bits)
            log(f"decode T=64 int{bits}: {dec['ms']:.3f} ms, {dec['GB_s']:.0f} GB/s = "
                f"{dec['frac_hbm']:.3f} of HBM ({time.perf_counter() - t0:.1f} s)")
            if bits == 4:
                decode = dec
            else:
                decode8 = dec
    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded; int4 base quantised from N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name + (" (forward + adapter-only backward)" if cfg.train
                                           else " (forward)"),
                   "T": cfg.T, "d_model": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.f, "rank": cfg.r, "group": cfg.group, "act": cfg.act,
                   "router_bias_var": cfg.router_bias_var},
        "roofline": {"bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": dom["frac"], "traffic": traffic,
                     "kernel": dom["kernel"] + ", the longest stage per step",
                     "kernel_ms": dom["ms"],
                     "launches_per_step": 1,
                     "timed_as": "one HIP event pair on the launch stream around the stage's "
                                 "launch, once per step, averaged over the steps",
                     "flops_per_launch": dom["flops"]},
        "stages": stages,
        "decode": decode,
        "decode_int8": decode8,
        "layer_tflops": layer_flops(cfg, cfg.train) / (ms / 1e3) / 1e12,
        "layer_frac_of_bf16_peak": layer_flops(cfg, cfg.train) / (ms / 1e3) / PEAK_BF16,
        "forward_ms": fwd_ms,
        # the frozen int4 base is re-laid out once at setup (moe_pack_base_f
        # for the forward, moe_pack_base_t for the backward), like its
        # quantisation; the timed steps run every per-step kernel
        "base_packed_for_forward": bool(getattr(L, "packed_f", None)),
        "base_packed_for_backward": bool(getattr(L, "packed", None)),
        "adamw": adamw,
        "reversible": reversible,
        "growth": growth,
        "forward_tokens_per_s": cfg.T / (fwd_ms / 1e3),
        "load": {"max": int(counts.max()), "mean": float(counts.mean()),
                 "empty_experts": int((counts == 0).sum())},
    }
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_probe_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        rec["cpu_baseline"], rec["routing"] = cpu_baseline(cfg, inp, args.cpu_seconds, gpu_idx)
        log(f"cpu baseline took {time.perf_counter() - t0:.1f} s")
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
