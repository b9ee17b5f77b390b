#!/usr/bin/env python3
"""Benchmark of the DoRA module hot path on one MI355X.

A step is one pass of the whole hot path over one synthetic batch: the
factored row norm, the base and adapter products, the fused compose
(dora_forward) and the norm-detached backward (dora_backward), on the
training-shaped module d_in 8192 -> d_out 28672, r 384, 8192 tokens, bf16
(the shape and rank the Scaling-DoRA abstract works at).  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

Printed JSON line (one):
  value        module forward time per step (microseconds, HIP events), the
               first quantity of the metric; ms_per_step covers forward +
               backward, wall clock over the K timed steps;
               *_min_median_max the spread over the timed steps.
  fwd_cached_norm_us  dora_forward with the norm given (n_in), as inference
               with frozen adapters runs it.
  compose_*    dora_compose alone, HBM GB/s with the 256 MB MALL flushed
               before every launch (6 bytes per bf16 element);
               compose_warm_GBps back-to-back launches without the flush.
  norm_*       dora_factored_norm alone: algorithmic flops / time against
               the 2.5 PFLOP/s dense bf16 MFMA peak.
  roofline     the dominant kernel (the base product x W^T, bf16 MFMA),
               timed with HIP events on the launch stream.
  merge_*      dora_merge alone (norm given): the merged inference weight,
               HBM GB/s (read W, write W').
  bwd_through_norm_us  dora_backward_through_norm (the gradient also through
               the row norm) reusing the norm's kept W A^T, back-to-back
               launches; *_recompute_U_us without it.
  group_norm   the factored norms of all 56 adapted projections of an 8-layer,
               8B-class decoder (hidden 4096, key/value 1024, MLP 14336,
               r 384): dora_factored_norm_grouped vs one dora_factored_norm
               per module (host launch cost included in both).
  group_forward_qkv  dora_forward_grouped over the query/key/value siblings
               of one such layer on one x, vs three dora_forward calls.
  cpu_baseline the fp64 oracle forward on the same module on the host cores,
               on a bounded token sample, extrapolated to the full batch.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DoRA module fwd µs + compose HBM GB/s + norm-GEMM MFMA util, r=384 bf16"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "base_gemm_traffic.json")
KERNEL_WARMUP = 10  # untimed launches before each kernel-leg burst (the clock settles)
GROUP_LAYERS = 8   # decoder layers whose 7 projections form the grouped-norm workload


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the GEMM kernel sources: counter readings are only reused for
    the kernel they were taken on."""
    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "gemm_bf16_dma.hpp", "gemm_dma_launch.hpp", "gemm_dma_cfg.hip",
              "epilogue.hpp", "dora_internal.hpp"):
        with open(os.path.join(ROOT, "dora_adapter_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def norm_flops(d_out, d_in, r):
    # U = W A^T, G = A A^T, B G (hi and lo), row sums of W^2, the two row dots
    return 2 * d_out * d_in * r + 2 * r * r * d_in + 2 * 2 * d_out * r * r + 2 * d_out * d_in \
        + 4 * d_out * r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--leg", choices=["all", "step", "kernels", "base", "norm", "compose",
                                      "copy"],
                    default="all",
                    help="'base' launches only the dominant kernel, 'norm' only "
                         "dora_factored_norm, 'compose' only dora_compose (for counter runs); "
                         "'copy' a plain device copy of known size (counter calibration)")
    ap.add_argument("--iters", type=int, default=10, help="launches per kernel-leg timing")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the DoRA module path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import torch
    from dora_adapter_amd import dora as D
    from dora_adapter_amd import synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    shape = synth.TRAIN_R384
    T, d_in, d_out, r, s = shape.T, shape.d_in, shape.d_out, shape.r, shape.s

    if args.leg == "copy":
        nbytes = 1 << 30
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(args.iters):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": args.iters}))
        return

    log("generating", shape.name)
    mod = synth.make_module(shape, seed=0, with_dy=True)
    t = {k: mod[k].to(dev) for k in ("x", "W", "A", "B", "m", "dy")}
    del mod
    torch.cuda.synchronize()

    if args.leg == "base":
        # the same launch sequence the kernel leg times: warm-up, then a burst
        y = torch.empty(T, d_out, dtype=torch.bfloat16, device=dev)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_linear(t["x"], t["W"], y=y)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "base", "launches": KERNEL_WARMUP + args.iters,
                          "flops_per_launch": 2 * T * d_in * d_out}))
        return

    if args.leg == "norm":
        # dora_factored_norm alone on the training module (W A^T with the row
        # sums of squares and row dots, A A^T, B G, the finish)
        n = torch.empty(d_out, dtype=torch.float32, device=dev)
        ws_n = torch.empty(D.dora_norm_workspace(d_out, d_in, r, 1), dtype=torch.uint8,
                           device=dev)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_factored_norm(t["W"], t["A"], t["B"], s, ws=ws_n, n=n)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "norm", "launches": KERNEL_WARMUP + args.iters,
                          "flops_per_launch": norm_flops(d_out, d_in, r)}))
        return

    if args.leg == "compose":
        # dora_compose alone on the training module's [T, d_out] (6 bytes per
        # bf16 element: read base and lora, write y)
        base = torch.randn(T, d_out, device=dev).bfloat16()
        lora = torch.randn(T, d_out, device=dev).bfloat16()
        n = torch.rand(d_out, device=dev) + 0.5
        yc = torch.empty_like(base)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_compose(base, lora, t["m"], n, s, y=yc)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "compose", "launches": KERNEL_WARMUP + args.iters,
                          "bytes_per_launch": 6 * T * d_out + 8 * d_out}))
        return

    # Preallocated outputs and workspaces: nothing is allocated inside the step.
    y = torch.empty(T, d_out, dtype=torch.bfloat16, device=dev)
    n = torch.empty(d_out, dtype=torch.float32, device=dev)
    P = torch.empty(T, r, dtype=torch.bfloat16, device=dev)
    grads = {"dx": torch.empty(T, d_in, dtype=torch.bfloat16, device=dev),
             "dA": torch.empty(r, d_in, dtype=torch.bfloat16, device=dev),
             "dB": torch.empty(d_out, r, dtype=torch.bfloat16, device=dev),
             "dm": torch.empty(d_out, dtype=torch.float32, device=dev)}
    ws_f = torch.empty(D.dora_forward_workspace(T, d_in, d_out, r, 1), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(D.dora_backward_workspace(T, d_in, d_out, r, 1), dtype=torch.uint8,
                       device=dev)

    def fwd():
        D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s, ws=ws_f, y=y, n_out=n, P_out=P)

    def bwd():
        D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y, ws=ws_b,
                        out=grads)

    out = {"metric": METRIC, "unit": "µs", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; W, A ~ N(0, 1/d_in), B ~ N(0, 0.02^2), "
                   "m = ||W_i|| (1 + N(0, 0.01^2)), x, dy ~ N(0, 1))",
           "config": {"workload": shape.name, "d_in": d_in, "d_out": d_out, "r": r,
                      "tokens": T, "s": s,
                      "step": "factored norm + forward + compose + norm-detached backward",
                      "parallelism": "single GPU"}}

    if args.leg in ("all", "step"):
        log(f"warmup {args.warmup}")
        for _ in range(args.warmup):
            fwd()
            bwd()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        log(f"timing {args.steps} steps")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            ev[k][0].record()
            fwd()
            ev[k][1].record()
            bwd()
            ev[k][2].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        fwd_each = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
        bwd_each = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in ev)
        fwd_us = sum(fwd_each) / args.steps
        bwd_us = sum(bwd_each) / args.steps

        def spread(xs):  # min, median, max over the timed steps
            return [round(xs[0], 1), round(xs[len(xs) // 2], 1), round(xs[-1], 1)]
        out.update(value=round(fwd_us, 1), ms_per_step=round((t1 - t0) / args.steps * 1e3, 3),
                   fwd_us=round(fwd_us, 1), bwd_us=round(bwd_us, 1),
                   fwd_us_min_median_max=spread(fwd_each),
                   bwd_us_min_median_max=spread(bwd_each),
                   fwd_tflops=round((2 * T * d_in * d_out + 2 * T * r * (d_in + d_out)
                                     + norm_flops(d_out, d_in, r)) / fwd_us / 1e6, 1),
                   bwd_tflops=round((2 * T * d_out * d_in + 4 * T * d_out * r + 4 * T * r * d_in)
                                    / bwd_us / 1e6, 1))
        log(f"fwd {fwd_us:.1f} us  bwd {bwd_us:.1f} us")

    if args.leg == "kernels":
        # the legs below read y, n, P and the gradients: give them the values
        # a training step gives them (matrix-core power, hence the clock under
        # the power limit, depends on the operand values)
        fwd()
        bwd()
        torch.cuda.synchronize()

    if args.leg in ("all", "kernels"):
        # Launches go back to back (the way a model runs them; the clock
        # settles under sustained load) and are timed with HIP events on the
        # launch stream, after KERNEL_WARMUP untimed ones.  With `pre` (a
        # cache flush) each launch is timed alone, the flush outside.
        def timed(fn, pre=None):
            for _ in range(KERNEL_WARMUP):
                fn()
            if pre is None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(args.iters):
                    fn()
                b.record()
                b.synchronize()
                return a.elapsed_time(b) / args.iters * 1e3
            tot = 0.0
            for _ in range(args.iters):
                pre()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                b.synchronize()
                tot += a.elapsed_time(b)
            return tot / args.iters * 1e3

        # dominant kernel: the base product x W^T (one launch of the bf16 MFMA GEMM)
        y_lin = torch.empty_like(y)
        base_us = timed(lambda: D.dora_linear(t["x"], t["W"], y=y_lin))
        flops = 2 * T * d_in * d_out
        ach = flops / base_us / 1e6
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as fh:
                tr = json.load(fh)
            if tr.get("kernel_source_hash") == kernel_source_hash():
                traffic = tr.get("hbm_bytes_per_launch")
        out["roofline"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic, "kernel": "gemm_bf16 x W^T (dora_linear)",
                           "flops_per_launch": flops, "us_per_launch": round(base_us, 1)}
        log(f"base GEMM {base_us:.1f} us = {ach:.0f} TFLOP/s")

        ws_n = torch.empty(D.dora_norm_workspace(d_out, d_in, r, 1), dtype=torch.uint8,
                           device=dev)
        n2 = torch.empty_like(n)
        norm_us = timed(lambda: D.dora_factored_norm(t["W"], t["A"], t["B"], s, ws=ws_n, n=n2))
        nf = norm_flops(d_out, d_in, r)
        out["norm_us"] = round(norm_us, 1)
        out["norm_mfma_util"] = round(nf / norm_us / 1e6 / PEAK_BF16_TFLOPS, 4)
        log(f"norm {norm_us:.1f} us = {nf / norm_us / 1e6:.0f} TFLOP/s")

        # the forward with the norm cached (n_in: inference with frozen
        # adapters skips the factored norm)
        fwd_n_us = timed(lambda: D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s,
                                                n_in=n2, ws=ws_f, y=y_lin, n_out=n2, P_out=P))
        out["fwd_cached_norm_us"] = round(fwd_n_us, 1)
        log(f"forward with the norm cached {fwd_n_us:.1f} us")

        # merged weight for inference (norm given): read W, write W', 2 x 2 bytes per weight
        w_out = torch.empty_like(t["W"])
        ws_m = torch.empty(D.dora_merge_workspace(d_out, d_in, r, 1), dtype=torch.uint8,
                           device=dev)
        merge_us = timed(lambda: D.dora_merge(t["W"], t["A"], t["B"], t["m"], s, n_in=n2,
                                              out=w_out, ws=ws_m))
        merge_bytes = 2 * d_out * d_in * 2 + (d_out + d_in) * r * 2 + 2 * d_out * 4
        out["merge_us"] = round(merge_us, 1)
        out["merge_GBps"] = round(merge_bytes / merge_us / 1e3, 1)
        log(f"merge {merge_us:.1f} us = {merge_bytes / merge_us / 1e3:.0f} GB/s")
        del w_out, ws_m

        # backward with the gradient through the norm (same outputs as the
        # step's backward plus the norm's term in dA and dB)
        ws_t = torch.empty(D.dora_backward_through_norm_workspace(T, d_in, d_out, r, 1),
                           dtype=torch.uint8, device=dev)
        # with the norm's U = W A^T kept by the forward (U_out), the intended
        # pairing, and with U recomputed
        U = torch.empty(d_out, r, dtype=torch.float32, device=dev)
        D.dora_factored_norm(t["W"], t["A"], t["B"], s, ws=ws_n, n=n2, U_out=U)
        thru_us = timed(lambda: D.dora_backward_through_norm(
            t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y, U=U, ws=ws_t,
            out=grads))
        thru_re_us = timed(lambda: D.dora_backward_through_norm(
            t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y, ws=ws_t, out=grads))
        out["bwd_through_norm_us"] = round(thru_us, 1)
        out["bwd_through_norm_recompute_U_us"] = round(thru_re_us, 1)
        log(f"backward through the norm {thru_us:.1f} us (U kept), {thru_re_us:.1f} us (U recomputed)")
        del ws_t, U

        # many modules: the factored norms of every adapted projection of an
        # 8-layer, 8B-class decoder (56 modules, r = 384) in grouped launches,
        # against the same norms module by module (host launch cost included)
        group = synth.make_group(synth.decoder_layer_shapes() * GROUP_LAYERS, r, seed=5,
                                 device=dev)
        gm = [(g["W"], g["A"], g["B"], g["m"], g["s"]) for g in group]
        ns_g = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in gm]
        ws_g = D._ws(D.dora_factored_norm_grouped_workspace(gm, 1), dev)
        grp_us = timed(lambda: D.dora_factored_norm_grouped(gm, ns=ns_g, ws=ws_g))
        ws_1 = D._ws(max(D.dora_norm_workspace(W.shape[0], W.shape[1], r, 1)
                         for W, *_ in gm), dev)
        one_us = timed(lambda: [D.dora_factored_norm(W, A, B, sg, ws=ws_1, n=nk)
                                for (W, A, B, _, sg), nk in zip(gm, ns_g)])
        gf = sum(norm_flops(W.shape[0], W.shape[1], r) for W, *_ in gm)
        out["group_norm"] = {"modules": len(gm), "grouped_us": round(grp_us, 1),
                             "per_module_us": round(one_us, 1),
                             "grouped_mfma_util": round(gf / grp_us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        log(f"norm of {len(gm)} modules: grouped {grp_us:.1f} us, one by one {one_us:.1f} us")
        # sibling modules on one input: query, key, value of one layer, T tokens
        xs = torch.randn(T, 4096, device=dev).bfloat16()
        qkv = gm[:3]
        ys_g = [torch.empty(T, W.shape[0], dtype=torch.bfloat16, device=dev) for W, *_ in qkv]
        Ps_g = [torch.empty(T, r, dtype=torch.bfloat16, device=dev) for _ in qkv]
        ns_q = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in qkv]
        ws_q = D._ws(D.dora_forward_grouped_workspace(qkv, T, 1, P_out=Ps_g), dev)
        fg_us = timed(lambda: D.dora_forward_grouped(xs, qkv, ws=ws_q, ys=ys_g, ns=ns_q, Ps=Ps_g))
        ws_f1 = D._ws(max(D.dora_forward_workspace(T, 4096, W.shape[0], r, 1) for W, *_ in qkv),
                      dev)
        f1_us = timed(lambda: [D.dora_forward(xs, W, A, B, mq, sq, ws=ws_f1, y=yk, n_out=nk,
                                              P_out=Pk)
                               for (W, A, B, mq, sq), yk, nk, Pk in zip(qkv, ys_g, ns_q, Ps_g)])
        out["group_forward_qkv"] = {"tokens": T, "grouped_us": round(fg_us, 1),
                                    "per_module_us": round(f1_us, 1)}
        log(f"q/k/v forward: grouped {fg_us:.1f} us, one by one {f1_us:.1f} us")
        del group, gm, ns_g, ws_g, ws_1, xs, ys_g, Ps_g, ws_q, ws_f1

        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        lora = torch.randn(T, d_out, device=dev).bfloat16()
        yc = torch.empty_like(y)
        comp_us = timed(lambda: D.dora_compose(y, lora, t["m"], n, s, y=yc),
                        pre=lambda: flush.fill_(1))
        gbps = 6 * T * d_out / comp_us / 1e3
        out["compose_us"] = round(comp_us, 1)
        out["compose_GBps"] = round(gbps, 1)
        out["compose_frac_hbm"] = round(gbps / PEAK_HBM_GBPS, 4)
        log(f"compose {comp_us:.1f} us = {gbps:.0f} GB/s (MALL flushed)")
        warm_us = timed(lambda: D.dora_compose(y, lora, t["m"], n, s, y=yc))
        out["compose_warm_GBps"] = round(6 * T * d_out / warm_us / 1e3, 1)
        log(f"compose back to back {warm_us:.1f} us = {6 * T * d_out / warm_us / 1e3:.0f} GB/s")
        del flush, lora, yc, y_lin

    if args.leg == "all" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(t, shape)

    print(json.dumps(out), flush=True)


def cpu_baseline(t, shape):
    """The fp64 oracle's forward on the same module, on the host cores.  Its
    cost is a per-row part (forming row i of W + sBA: d_in * r) plus a
    per-token part (d_in per row); two token counts give both, and the time
    is extrapolated linearly to the full token count."""
    from oracle import oracle as O
    cpu = {k: t[k].cpu() for k in ("x", "W", "A", "B", "m")}
    times = {}
    for ntok in (8, 1032):
        toks = list(range(ntok))
        log(f"cpu baseline: oracle forward on {ntok} tokens")
        a = time.perf_counter()
        O.forward(cpu["x"], cpu["W"], cpu["A"], cpu["B"], cpu["m"], shape.s, toks=toks)
        times[ntok] = time.perf_counter() - a
    per_tok = (times[1032] - times[8]) / 1024
    fixed = times[8] - 8 * per_tok
    full_s = fixed + per_tok * shape.T
    return {"value": round(full_s * 1e6, 0), "unit": "µs", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": f"oracle forward (fp64, dense W + sBA rows) at the full module shape on "
                      f"8 and 1032 tokens ({times[8]:.1f} s, {times[1032]:.1f} s); fixed + per-token "
                      f"cost extrapolated to {shape.T} tokens"}


if __name__ == "__main__":
    main()
