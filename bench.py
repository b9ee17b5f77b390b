#!/usr/bin/env python3
"""Benchmark of the DoRA module hot path on one MI355X.

A step is one pass of the whole hot path over one synthetic batch.  The
default workload (--config c5) is the training-shaped module d_in 8192 ->
d_out 28672, r 384, 8192 tokens, bf16 (the shape and rank the Scaling-DoRA
abstract works at): the factored row norm, the base and adapter products,
the fused compose (dora_forward) and the norm-detached backward
(dora_backward).  The other workloads are forward only: c2 the square
4096 module at r 64 (its norm HBM-bound), c3 the square 8192 module at
r 384 (the abstract's shape, with the workspace / transient check), c4 the
MLP up 5120 -> 27648 and down 27648 -> 5120 pair at r 384 on 16384 tokens,
back to back.  Inputs are seeded synthetic tensors already resident in HBM
when timing starts; one JSON line per run.

Printed JSON line (one):
  value        module forward time per step (microseconds, HIP events; for
               c4 the up and down forwards together), the first quantity of
               the metric; ms_per_step is the wall clock of a whole step
               (c5: forward + backward) over the K timed steps;
               *_min_median_max the spread over the timed steps.
  roofline     the dominant kernel (the base product x W^T, bf16 MFMA),
               timed with HIP events on the launch stream; traffic is the
               counter-measured HBM bytes per launch (null unless the
               committed counter record matches the kernel sources), and
               traffic_ratio that over the algorithmic bytes.
  norm_*       dora_factored_norm alone: algorithmic flops (U, G, B G once,
               the row sums and dots) / time against the 2.5 PFLOP/s dense
               bf16 peak; norm_kernels_us its kernels from the profiler's
               device trace; norm_U_mfma_util U = W A^T alone.
  fwd_cached_norm_us  dora_forward with the norm given (n_in), as inference
               with frozen adapters runs it.
  compose_*    dora_compose alone on the workload's [T, d_out], HBM GB/s
               with the 256 MB MALL flushed before every launch (6 bytes per
               bf16 element); compose_warm_GBps back to back.
  stream_ceiling  the best rate over the launch shapes of a plain two-in /
               one-out 16-byte non-temporal stream of the same size, MALL
               flushed: the ceiling the compose and dh/dm are held against.
  dh_dm_*      (c5) the backward's dh = g dy and dm: dh_dm_dB_us the dB
               product that forms them on the way (the step's path) and its
               rate over the dy, y, dh streams; dh_dm_us / dh_dm_GBps the
               separate streaming pass (6 bytes per bf16 element), from one
               backward with the planners restricted to another tile shape.
  step_kernels_us  (c5) every kernel of one forward + backward step, in
               launch order, from the profiler's device trace.
  merge_*, bwd_through_norm_*, group_norm, group_forward_qkv  (c5) the
               merged-weight export, the backward through the norm, the 56
               norms of an 8-layer 8B-class decoder grouped vs one by one,
               and the grouped query/key/value forward.
  workspace_*  (c3) the peak-allocation growth around dora_factored_norm
               and dora_forward (their workspaces) against one dense
               [d_out, d_in] bf16 buffer.
  cpu_baseline the fp64 oracle on the same module on the host cores: by
               default on a bounded token sample, extrapolated to the full
               batch; with --cpu-full on the whole problem (c2, c3, c5
               forward; c4 the two norms and the forward extrapolated).
"""
import argparse
import ctypes
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
STREAM_LIB = os.path.join(ROOT, "dora_adapter_amd", "libstreamceil.so")
KERNEL_WARMUP = 10  # untimed launches before each kernel-leg burst (the clock settles)
GROUP_LAYERS = 8   # decoder layers whose 7 projections form the grouped-norm workload
CONFIGS = ("c2", "c3", "c4", "c5")
# The factored norm's kernels, by role: G = A A^T, its finalize into the
# bf16 hi / lo pair, U = W A^T (with G's tiles where they ride in its launch),
# B G, and the finish (absent where B G's epilogue forms n)
NORM_ROLES = ("gram_AAt", "gram_finalize", "U_WAt_rowdot", "BG_rowdot", "finish")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the GEMM kernel sources: counter readings are only reused for
    the kernel they were taken on."""
    h = hashlib.sha256()
    for f in ("gemm_bf16.hip", "gemm_bf16_dma.hpp", "gemm_persistent.hpp", "gemm_dma_launch.hpp",
              "gemm_dma_cfg.hip", "epilogue.hpp", "dora_internal.hpp"):
        with open(os.path.join(ROOT, "dora_adapter_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def norm_flops(d_out, d_in, r):
    """Algorithmic flops of one factored norm: U = W A^T, G = A A^T, B G
    (once: the kernels' hi/lo split of G is an implementation choice), the
    row sums of W^2 and the cross and Gram row dots."""
    return 2 * d_out * d_in * r + 2 * r * r * d_in + 2 * d_out * r * r + 2 * d_out * d_in \
        + 4 * d_out * r


def fwd_flops(T, d_in, d_out, r):
    return 2 * T * d_in * d_out + 2 * T * r * (d_in + d_out) + norm_flops(d_out, d_in, r)


def bwd_flops(T, d_in, d_out, r):
    return 2 * T * d_out * d_in + 4 * T * d_out * r + 4 * T * r * d_in


def workload(cfg):
    """The modules of a workload: [(shape)], the first one's x is the input."""
    from dora_adapter_amd import synth
    return {"c2": [synth.SQUARE_R64], "c3": [synth.SQUARE_R384],
            "c4": [synth.MLP_UP, synth.MLP_DOWN], "c5": [synth.TRAIN_R384]}[cfg]


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", choices=CONFIGS, default="c5",
                    help="workload: c2 square 4096 r64, c3 square 8192 r384, c4 MLP up/down "
                         "pair, c5 training module (default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on the whole problem instead of a token sample")
    ap.add_argument("--leg", choices=["all", "step", "kernels", "base", "norm", "compose",
                                      "stream", "copy", "groupnorm"],
                    default="all",
                    help="'base' launches only the dominant kernel, 'norm' only "
                         "dora_factored_norm, 'compose' only dora_compose, 'stream' only the "
                         "stream-ceiling kernel (for counter runs); 'copy' a plain device copy "
                         "of known size (counter calibration); 'groupnorm' only the grouped "
                         "norm of the 56-module decoder set")
    ap.add_argument("--iters", type=int, default=10, help="launches per kernel-leg timing")
    return ap.parse_args(argv)


class Timer:
    """HIP-event timing on the launch stream (the binding launches on torch's
    current stream, which these events are recorded on)."""

    def __init__(self, torch, iters):
        self.torch, self.iters = torch, iters

    def __call__(self, fn, pre=None, iters=None):
        torch = self.torch
        iters = self.iters if iters is None else iters
        for _ in range(KERNEL_WARMUP):
            if pre is not None:
                pre()
            fn()
        if pre is None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(iters):
                fn()
            b.record()
            b.synchronize()
            return a.elapsed_time(b) / iters * 1e3
        tot = 0.0
        for _ in range(iters):
            pre()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            tot += a.elapsed_time(b)
        return tot / iters * 1e3


def device_kernels(torch, fn, calls=1):
    """(name, microseconds) of every kernel fn launches, in launch order, from
    the profiler's device trace (one warm-up call first)."""
    from torch.profiler import ProfilerActivity, profile
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
    evs = [e for e in prof.events() if e.device_type.name == "CUDA"]
    evs.sort(key=lambda e: e.time_range.start)
    dur = (lambda e: e.device_time) if hasattr(evs[0] if evs else None, "device_time") \
        else (lambda e: e.cuda_time)
    return [(e.name, float(dur(e))) for e in evs]


def short_name(name):
    """A readable kernel name: the function and its tile / layout arguments."""
    n = name.replace("dora::", "").replace("(anonymous namespace)::", "").replace("void ", "")
    if "(" in n:
        n = n[:n.index("(")]
    return n.replace("unsigned short", "bf16")


def norm_roles(names):
    """Role (NORM_ROLES) of each kernel of one factored-norm call, from the
    kernel names in launch order: the finalize and finish kernels by name,
    the products by position (G, U, B G when G has a launch of its own; U,
    B G when G's tiles ride in U's launch).  None for any other form."""
    prods = [i for i, n in enumerate(names) if "finalize" not in n and "norm_finish" not in n]
    roles = {}
    for i, n in enumerate(names):
        if "finalize" in n:
            roles[i] = "gram_finalize"
        elif "norm_finish" in n:
            roles[i] = "finish"
    if len(prods) == 3:
        roles.update(zip(prods, ("gram_AAt", "U_WAt_rowdot", "BG_rowdot")))
    elif len(prods) == 2:
        roles.update(zip(prods, ("U_WAt_rowdot", "BG_rowdot")))
    else:
        return None
    return [roles[i] for i in range(len(names))]


def norm_split(torch, fn, calls=5):
    """The factored norm's kernels averaged over `calls` calls, keyed by role
    (norm_roles).  None if the trace does not split into equal calls of a
    known form."""
    ks = device_kernels(torch, fn, calls)
    if not ks or len(ks) % calls:
        return None
    k = len(ks) // calls
    per = [ks[c * k:(c + 1) * k] for c in range(calls)]
    names = [n for n, _ in per[0]]
    roles = norm_roles(names)
    if roles is None or any([n for n, _ in p] != names for p in per):
        return None
    return {roles[i]: round(sum(p[i][1] for p in per) / calls, 1) for i in range(k)}


class StreamCeiling:
    """The plain two-in / one-out stream of libstreamceil.so."""

    VARIANTS = [(v, th) for v in range(4) for th in (1 << 18, 1 << 19, 1 << 20, 1 << 21)] + \
               [(4, th) for th in (1 << 19, 1 << 20, 1 << 21)]

    def __init__(self, torch, nbytes, row_bytes, dev):
        self.L = ctypes.CDLL(STREAM_LIB)
        self.L.stream_ceiling_launch.restype = ctypes.c_int
        self.L.stream_ceiling_launch.argtypes = [ctypes.c_void_p] * 3 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        self.torch, self.nbytes, self.row_bytes = torch, nbytes, row_bytes
        self.a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        self.b = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(2)
        self.c = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream

    def launch(self, variant, threads):
        rc = self.L.stream_ceiling_launch(self.a.data_ptr(), self.b.data_ptr(), self.c.data_ptr(),
                                          self.nbytes, self.row_bytes, variant, threads,
                                          self.stream)
        if rc != 0:
            raise RuntimeError(f"stream_ceiling_launch: hip error {rc}")

    def sweep(self, timer, flush):
        best = None
        for v, th in self.VARIANTS:
            us = timer(lambda: self.launch(v, th), pre=flush, iters=5)
            if best is None or us < best[0]:
                best = (us, v, th)
        us, v, th = best
        return {"GBps": round(3 * self.nbytes / us / 1e3, 1), "us": round(us, 1),
                "variant": ["grid-stride x1", "grid-stride x2", "grid-stride x4",
                            "grid-stride x8", "row runs (compose order)"][v],
                "threads": th, "bytes": 3 * self.nbytes}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the DoRA module path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import torch
    from dora_adapter_amd import dora as D
    from dora_adapter_amd import synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    shapes = workload(args.config)
    sh0 = shapes[0]
    T = sh0.T
    timer = Timer(torch, args.iters)

    if args.leg == "groupnorm":
        r = sh0.r
        group = synth.make_group(synth.decoder_layer_shapes() * GROUP_LAYERS, r, seed=5,
                                 device=dev)
        gm = [(g["W"], g["A"], g["B"], g["m"], g["s"]) for g in group]
        ns_g = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in gm]
        ws_g = D._ws(D.dora_factored_norm_grouped_workspace(gm, 1), dev)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_factored_norm_grouped(gm, ns=ns_g, ws=ws_g)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "groupnorm", "modules": len(gm),
                          "launches": KERNEL_WARMUP + args.iters,
                          "flops_per_launch": sum(norm_flops(W.shape[0], W.shape[1], r)
                                                  for W, *_ in gm)}))
        return

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

    if args.leg == "stream":
        sc = StreamCeiling(torch, T * sh0.d_out * 2, sh0.d_out * 2, dev)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        best = sc.sweep(timer, lambda: flush.fill_(1))
        v = ["grid-stride x1", "grid-stride x2", "grid-stride x4", "grid-stride x8",
             "row runs (compose order)"].index(best["variant"])
        for _ in range(KERNEL_WARMUP + args.iters):
            flush.fill_(1)
            sc.launch(v, best["threads"])
        torch.cuda.synchronize()
        print(json.dumps({"leg": "stream", "launches": KERNEL_WARMUP + args.iters, **best}))
        return

    log("generating", args.config, [s.name for s in shapes])
    if args.config == "c4":
        up, down, x = synth.make_mlp_pair(seed=0)
        mods = [{k: v.to(dev) if torch.is_tensor(v) else v for k, v in md.items()}
                for md in (up, down)]
        x = x.to(dev)
    else:
        m0 = synth.make_module(sh0, seed=0, with_dy=sh0.backward)
        mods = [{k: (m0[k].to(dev)) for k in ("W", "A", "B", "m")} | {"s": m0["s"]}]
        x = m0["x"].to(dev)
        dy = m0["dy"].to(dev) if sh0.backward else None
        del m0
    torch.cuda.synchronize()
    d_in, d_out, r, s = sh0.d_in, sh0.d_out, sh0.r, sh0.s
    md0 = mods[0]

    if args.leg == "base":
        # the same launch sequence the kernel leg times: warm-up, then a burst
        y = torch.empty(T, d_out, dtype=torch.bfloat16, device=dev)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_linear(x, md0["W"], y=y)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "base", "config": args.config,
                          "launches": KERNEL_WARMUP + args.iters,
                          "flops_per_launch": 2 * T * d_in * d_out}))
        return

    if args.leg == "norm":
        n = torch.empty(d_out, dtype=torch.float32, device=dev)
        ws_n = D._ws(D.dora_norm_workspace(d_out, d_in, r, 1), dev)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_factored_norm(md0["W"], md0["A"], md0["B"], s, ws=ws_n, n=n)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "norm", "config": args.config,
                          "launches": KERNEL_WARMUP + args.iters,
                          "flops_per_launch": norm_flops(d_out, d_in, r)}))
        return

    if args.leg == "compose":
        base = torch.randn(T, d_out, device=dev).bfloat16()
        lora = torch.randn(T, d_out, device=dev).bfloat16()
        n = torch.rand(d_out, device=dev) + 0.5
        yc = torch.empty_like(base)
        for _ in range(KERNEL_WARMUP + args.iters):
            D.dora_compose(base, lora, md0["m"], n, s, y=yc)
        torch.cuda.synchronize()
        print(json.dumps({"leg": "compose", "config": args.config,
                          "launches": KERNEL_WARMUP + args.iters,
                          "bytes_per_launch": 6 * T * d_out + 8 * d_out}))
        return

    # Preallocated outputs and workspaces: nothing is allocated inside the step.
    bufs = []
    xin = x
    for sh, md in zip(shapes, mods):
        b = {"y": torch.empty(T, sh.d_out, dtype=torch.bfloat16, device=dev),
             "n": torch.empty(sh.d_out, dtype=torch.float32, device=dev),
             "P": torch.empty(T, sh.r, dtype=torch.bfloat16, device=dev),
             "ws": D._ws(D.dora_forward_workspace(T, sh.d_in, sh.d_out, sh.r, 1), dev),
             "x": xin}
        bufs.append(b)
        xin = b["y"]  # c4: the down module reads the up module's output

    def fwd():
        for md, b in zip(mods, bufs):
            D.dora_forward(b["x"], md["W"], md["A"], md["B"], md["m"], md["s"], ws=b["ws"],
                           y=b["y"], n_out=b["n"], P_out=b["P"])

    bwd = None
    if sh0.backward:
        grads = {"dx": torch.empty(T, d_in, dtype=torch.bfloat16, device=dev),
                 "dA": torch.empty(r, d_in, dtype=torch.bfloat16, device=dev),
                 "dB": torch.empty(d_out, r, dtype=torch.bfloat16, device=dev),
                 "dm": torch.empty(d_out, dtype=torch.float32, device=dev)}
        ws_b = D._ws(D.dora_backward_workspace(T, d_in, d_out, r, 1), dev)
        b0 = bufs[0]

        def bwd():
            D.dora_backward(dy, x, md0["W"], md0["A"], md0["B"], md0["m"], b0["n"], s, b0["P"],
                            b0["y"], ws=ws_b, out=grads)

    what = {"c5": "factored norm + forward + compose + norm-detached backward",
            "c4": "up then down module: factored norm + forward + compose each",
            }.get(args.config, "factored norm + forward + compose")
    cfg = {"workload": sh0.name if len(shapes) == 1 else "mlp_pair_5120_27648_r384_t16384",
           "config": args.config, "d_in": d_in, "d_out": d_out, "r": r, "tokens": T, "s": s,
           "step": what, "parallelism": "single GPU"}
    if len(shapes) > 1:
        cfg["modules"] = [{"d_in": q.d_in, "d_out": q.d_out, "r": q.r} for q in shapes]
    sig_b = sh0.sigma_B
    out = {"metric": METRIC, "unit": "µs", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": f"synthetic (seeded; W, A ~ N(0, 1/d_in), B ~ N(0, {sig_b}^2), "
                   "m = ||W_i|| (1 + N(0, 0.01^2)), x, dy ~ N(0, 1))",
           "config": cfg}

    if args.leg in ("all", "step"):
        log(f"warmup {args.warmup}")
        for _ in range(args.warmup):
            fwd()
            if bwd:
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
            if bwd:
                bwd()
            ev[k][2].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        fwd_each = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in ev)
        fwd_us = sum(fwd_each) / args.steps

        def spread(xs):  # min, median, max over the timed steps
            return [round(xs[0], 1), round(xs[len(xs) // 2], 1), round(xs[-1], 1)]
        ff = sum(fwd_flops(T, q.d_in, q.d_out, q.r) for q in shapes)
        out.update(value=round(fwd_us, 1), ms_per_step=round((t1 - t0) / args.steps * 1e3, 3),
                   fwd_us=round(fwd_us, 1), fwd_us_min_median_max=spread(fwd_each),
                   fwd_tflops=round(ff / fwd_us / 1e6, 1))
        if bwd:
            bwd_each = sorted(e[1].elapsed_time(e[2]) * 1e3 for e in ev)
            bwd_us = sum(bwd_each) / args.steps
            out.update(bwd_us=round(bwd_us, 1), bwd_us_min_median_max=spread(bwd_each),
                       bwd_tflops=round(bwd_flops(T, d_in, d_out, r) / bwd_us / 1e6, 1))
            log(f"fwd {fwd_us:.1f} us  bwd {bwd_us:.1f} us")
        else:
            log(f"fwd {fwd_us:.1f} us")

    if args.leg == "kernels":
        # the legs below read y, n, P and the gradients: give them the values
        # a training step gives them (matrix-core power, hence the clock under
        # the power limit, depends on the operand values)
        fwd()
        if bwd:
            bwd()
        torch.cuda.synchronize()

    if args.leg in ("all", "kernels"):
        kernel_legs(args, out, torch, D, synth, dev, timer, shapes, mods, bufs, fwd, bwd,
                    locals().get("dy"), locals().get("grads"))

    if args.leg == "all" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, shapes, mods, x)

    print(json.dumps(out), flush=True)


def kernel_legs(args, out, torch, D, synth, dev, timer, shapes, mods, bufs, fwd, bwd, dy, grads):
    """Per-kernel timings of the workload (HIP events on the launch stream,
    launches back to back after KERNEL_WARMUP untimed ones; with a cache
    flush each launch is timed alone, the flush outside)."""
    sh0, md0, b0 = shapes[0], mods[0], bufs[0]
    T, d_in, d_out, r, s = sh0.T, sh0.d_in, sh0.d_out, sh0.r, sh0.s
    x = b0["x"]

    # dominant kernel: the base product x W^T (one launch of the bf16 MFMA GEMM)
    def base_roofline(b, sh, md):
        y_lin = torch.empty(T, sh.d_out, dtype=torch.bfloat16, device=dev)
        us = timer(lambda: D.dora_linear(b["x"], md["W"], y=y_lin))
        flops = 2 * T * sh.d_in * sh.d_out
        alg_bytes = 2 * (T * sh.d_in + sh.d_out * sh.d_in + T * sh.d_out)
        traffic = None
        if args.config == "c5" and os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as fh:
                tr = json.load(fh)
            if tr.get("kernel_source_hash") == kernel_source_hash():
                traffic = tr.get("hbm_bytes_per_launch")
        ach = flops / us / 1e6
        log(f"base GEMM {sh.name} {us:.1f} us = {ach:.0f} TFLOP/s")
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_ratio": None if traffic is None else round(traffic / alg_bytes, 2),
                "algorithmic_bytes": alg_bytes,
                "kernel": "gemm_bf16 x W^T (dora_linear)", "flops_per_launch": flops,
                "us_per_launch": round(us, 1)}

    out["roofline"] = base_roofline(b0, sh0, md0)
    if len(shapes) > 1:
        out["roofline_down"] = base_roofline(bufs[1], shapes[1], mods[1])

    # the factored norm alone, and its five kernels
    norms = []
    for sh, md in zip(shapes, mods):
        ws_n = D._ws(D.dora_norm_workspace(sh.d_out, sh.d_in, sh.r, 1), dev)
        n2 = torch.empty(sh.d_out, dtype=torch.float32, device=dev)
        call = lambda md=md, ws_n=ws_n, n2=n2: D.dora_factored_norm(  # noqa: E731
            md["W"], md["A"], md["B"], md["s"], ws=ws_n, n=n2)
        us = timer(call)
        nf = norm_flops(sh.d_out, sh.d_in, sh.r)
        rec = {"us": round(us, 1), "mfma_util": round(nf / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        split = norm_split(torch, call)
        if split:
            rec["kernels_us"] = split
            rec["gram_tiles_in_U_launch"] = "gram_AAt" not in split
            u_flops = 2 * sh.d_out * sh.d_in * sh.r
            rec["U_mfma_util"] = round(u_flops / split["U_WAt_rowdot"] / 1e6 / PEAK_BF16_TFLOPS, 4)
            # the norm's HBM-bound floor: W, A, B read once
            rec["hbm_floor_us"] = round(2 * (sh.d_out * sh.d_in + sh.r * sh.d_in
                                             + sh.d_out * sh.r) / PEAK_HBM_GBPS / 1e3, 1)
        log(f"norm {sh.name} {us:.1f} us = {nf / us / 1e6:.0f} TFLOP/s {split}")
        norms.append((rec, n2, ws_n))
    rec0 = norms[0][0]
    out["norm_us"] = rec0["us"]
    out["norm_mfma_util"] = rec0["mfma_util"]
    out["norm_U_mfma_util"] = rec0.get("U_mfma_util")
    out["norm_kernels_us"] = rec0.get("kernels_us")
    if len(shapes) > 1:
        out["norm_down"] = norms[1][0]

    # the forward with the norm cached (n_in: inference with frozen adapters)
    def fwd_cached():
        for md, b, (_, n2, _) in zip(mods, bufs, norms):
            D.dora_forward(b["x"], md["W"], md["A"], md["B"], md["m"], md["s"], n_in=n2,
                           ws=b["ws"], y=b["y"], n_out=n2, P_out=b["P"])
    out["fwd_cached_norm_us"] = round(timer(fwd_cached), 1)
    log(f"forward with the norm cached {out['fwd_cached_norm_us']:.1f} us")

    if args.config == "c3":
        # transient device memory: the peak-allocation growth around each call
        # (outputs preallocated; the growth is the workspace the binding takes)
        def peak_delta(fn):
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            fn()
            torch.cuda.synchronize()
            return torch.cuda.max_memory_allocated() - base
        nn_ = torch.empty(d_out, dtype=torch.float32, device=dev)
        dn = peak_delta(lambda: D.dora_factored_norm(md0["W"], md0["A"], md0["B"], s, n=nn_))
        df = peak_delta(lambda: D.dora_forward(x, md0["W"], md0["A"], md0["B"], md0["m"], s,
                                               y=b0["y"], n_out=nn_, P_out=b0["P"]))
        out["workspace_MiB"] = {"norm": round(dn / 2 ** 20, 2), "forward": round(df / 2 ** 20, 2),
                                "dense_d_out_x_d_in_bf16": round(d_out * d_in * 2 / 2 ** 20, 2)}
        log(f"transient: {out['workspace_MiB']}")

    if args.config == "c5":
        c5_legs(out, torch, D, synth, dev, timer, sh0, md0, b0, fwd, bwd, dy, grads,
                norms[0][1], norms[0][2])

    # the standalone compose on the workload's [T, d_out] (MALL flushed), and
    # the stream ceiling for the same byte count
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    lora = torch.randn(T, d_out, device=dev).bfloat16()
    yc = torch.empty(T, d_out, dtype=torch.bfloat16, device=dev)
    base = b0["y"]
    comp_us = timer(lambda: D.dora_compose(base, lora, md0["m"], b0["n"], s, y=yc),
                    pre=lambda: flush.fill_(1))
    nbytes = 6 * T * d_out
    out["compose_us"] = round(comp_us, 1)
    out["compose_GBps"] = round(nbytes / comp_us / 1e3, 1)
    out["compose_frac_hbm"] = round(nbytes / comp_us / 1e3 / PEAK_HBM_GBPS, 4)
    log(f"compose {comp_us:.1f} us = {nbytes / comp_us / 1e3:.0f} GB/s (MALL flushed)")
    warm_us = timer(lambda: D.dora_compose(base, lora, md0["m"], b0["n"], s, y=yc))
    out["compose_warm_GBps"] = round(nbytes / warm_us / 1e3, 1)
    del lora, yc
    sc = StreamCeiling(torch, T * d_out * 2, d_out * 2, dev)
    ceil = sc.sweep(timer, lambda: flush.fill_(1))
    del sc
    out["stream_ceiling"] = ceil
    out["compose_frac_of_ceiling"] = round(out["compose_GBps"] / ceil["GBps"], 4)
    if "dh_dm_GBps" in out:
        out["dh_dm_frac_of_ceiling"] = round(out["dh_dm_GBps"] / ceil["GBps"], 4)
    log(f"stream ceiling {ceil}")


def c5_legs(out, torch, D, synth, dev, timer, sh, md, b, fwd, bwd, dy, grads, n2, ws_n):
    T, d_in, d_out, r, s = sh.T, sh.d_in, sh.d_out, sh.r, sh.s
    x = b["x"]
    # every kernel of one step, from the device trace
    ks = device_kernels(torch, lambda: (fwd(), bwd()))
    out["step_kernels_us"] = [[short_name(nm), round(us, 1)] for nm, us in ks]
    # dh = g dy and dm: in the step, formed inside the dB product (the
    # kernel whose last template flag is set); its rate over the dy, y, dh
    # streams (6 bytes per element) beside the separate pass the library
    # runs where that product cannot (timed here by restricting the planners
    # to another tile configuration for one backward)
    fused = [us for nm, us in ks if nm.replace(" ", "").endswith("true>(dora::GemmArgs)")
             and "false,false,false,true" in nm.replace(" ", "")]
    if fused:
        out["dh_dm_dB_us"] = round(fused[0], 1)
        out["dh_dm_dB_stream_GBps"] = round(6 * T * d_out / fused[0] / 1e3, 1)
    os.environ["DORA_TILE_CFG"] = "4"
    try:
        # (that plan's workspace differs: the binding sizes one per call)
        ks2 = device_kernels(torch, lambda: D.dora_backward(
            dy, x, md["W"], md["A"], md["B"], md["m"], b["n"], s, b["P"], b["y"], out=grads))
    finally:
        os.environ.pop("DORA_TILE_CFG", None)
    sep = [us for nm, us in ks2 if "dh_dm" in nm]
    if sep:
        out["dh_dm_us"] = round(sep[0], 1)
        out["dh_dm_GBps"] = round(6 * T * d_out / sep[0] / 1e3, 1)

    # merged weight for inference (norm given): read W, write W', 2 x 2 bytes per weight
    w_out = torch.empty_like(md["W"])
    ws_m = D._ws(D.dora_merge_workspace(d_out, d_in, r, 1), dev)
    merge_us = timer(lambda: D.dora_merge(md["W"], md["A"], md["B"], md["m"], s, n_in=n2,
                                          out=w_out, ws=ws_m))
    merge_bytes = 2 * d_out * d_in * 2 + (d_out + d_in) * r * 2 + 2 * d_out * 4
    out["merge_us"] = round(merge_us, 1)
    out["merge_GBps"] = round(merge_bytes / merge_us / 1e3, 1)
    log(f"merge {merge_us:.1f} us = {merge_bytes / merge_us / 1e3:.0f} GB/s")
    del w_out, ws_m

    # backward with the gradient through the norm, with the norm's kept V A^T
    # (U_out, the intended pairing) and with it recomputed
    ws_t = D._ws(D.dora_backward_through_norm_workspace(T, d_in, d_out, r, 1), dev)
    U = torch.empty(d_out, r, dtype=torch.float32, device=dev)
    D.dora_factored_norm(md["W"], md["A"], md["B"], s, ws=ws_n, n=n2, U_out=U)
    thru_us = timer(lambda: D.dora_backward_through_norm(
        dy, x, md["W"], md["A"], md["B"], md["m"], b["n"], s, b["P"], b["y"], U=U, ws=ws_t,
        out=grads))
    thru_re_us = timer(lambda: D.dora_backward_through_norm(
        dy, x, md["W"], md["A"], md["B"], md["m"], b["n"], s, b["P"], b["y"], ws=ws_t,
        out=grads))
    out["bwd_through_norm_us"] = round(thru_us, 1)
    out["bwd_through_norm_recompute_U_us"] = round(thru_re_us, 1)
    log(f"backward through the norm {thru_us:.1f} us (U kept), {thru_re_us:.1f} us")
    del ws_t, U

    # many modules: the factored norms of every adapted projection of an
    # 8-layer, 8B-class decoder (56 modules, r = 384) in grouped launches,
    # against the same norms module by module (host launch cost included)
    group = synth.make_group(synth.decoder_layer_shapes() * GROUP_LAYERS, r, seed=5, device=dev)
    gm = [(g["W"], g["A"], g["B"], g["m"], g["s"]) for g in group]
    ns_g = [torch.empty(W.shape[0], dtype=torch.float32, device=dev) for W, *_ in gm]
    ws_g = D._ws(D.dora_factored_norm_grouped_workspace(gm, 1), dev)
    grp_us = timer(lambda: D.dora_factored_norm_grouped(gm, ns=ns_g, ws=ws_g))
    ws_1 = D._ws(max(D.dora_norm_workspace(W.shape[0], W.shape[1], r, 1) for W, *_ in gm), dev)
    one_us = timer(lambda: [D.dora_factored_norm(W, A, B, sg, ws=ws_1, n=nk)
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
    fg_us = timer(lambda: D.dora_forward_grouped(xs, qkv, ws=ws_q, ys=ys_g, ns=ns_q, Ps=Ps_g))
    ws_f1 = D._ws(max(D.dora_forward_workspace(T, 4096, W.shape[0], r, 1) for W, *_ in qkv), dev)
    f1_us = timer(lambda: [D.dora_forward(xs, W, A, B, mq, sq, ws=ws_f1, y=yk, n_out=nk,
                                          P_out=Pk)
                           for (W, A, B, mq, sq), yk, nk, Pk in zip(qkv, ys_g, ns_q, Ps_g)])
    out["group_forward_qkv"] = {"tokens": T, "grouped_us": round(fg_us, 1),
                                "per_module_us": round(f1_us, 1)}
    log(f"q/k/v forward: grouped {fg_us:.1f} us, one by one {f1_us:.1f} us")


def cpu_baseline(args, shapes, mods, x):
    """The fp64 oracle on the same module(s), on the host cores.  Its forward
    costs a per-row part (forming row i of W + sBA: d_in * r) plus a
    per-token part (d_in per row).  By default two token counts give both
    and the time is extrapolated linearly to the full token count (about
    10-30 s of CPU work); with --cpu-full the whole problem is timed where it
    finishes in minutes (c2, c3, c5 forward; c4 the two norms, its forward
    still extrapolated)."""
    from oracle import oracle as O
    T = shapes[0].T
    total_s, parts = 0.0, []
    xin = x.cpu()
    for k, (sh, md) in enumerate(zip(shapes, mods)):
        cpu = {q: md[q].cpu() for q in ("W", "A", "B", "m")}
        if k > 0:
            # the down module's input: an input of the same shape and recipe
            # (the oracle's cost does not depend on the values)
            xin = (xin.new_empty(T, sh.d_in).normal_()).to(xin.dtype)
        full = args.cpu_full and args.config in ("c2", "c3", "c5")
        if full:
            log(f"cpu baseline: oracle forward {sh.name} on all {T} tokens")
            a = time.perf_counter()
            O.forward(xin, cpu["W"], cpu["A"], cpu["B"], cpu["m"], sh.s)
            sec = time.perf_counter() - a
            parts.append(f"{sh.name}: full forward {sec:.1f} s")
        else:
            lo, hi = 8, 1032
            times = {}
            for ntok in (lo, hi):
                log(f"cpu baseline: oracle forward {sh.name} on {ntok} tokens")
                a = time.perf_counter()
                O.forward(xin, cpu["W"], cpu["A"], cpu["B"], cpu["m"], sh.s,
                          toks=list(range(ntok)))
                times[ntok] = time.perf_counter() - a
            per_tok = (times[hi] - times[lo]) / (hi - lo)
            sec = times[lo] - lo * per_tok + per_tok * T
            parts.append(f"{sh.name}: forward on {lo} and {hi} tokens ({times[lo]:.1f} s, "
                         f"{times[hi]:.1f} s), fixed + per-token cost extrapolated to {T}")
            if args.cpu_full:
                log(f"cpu baseline: oracle norm {sh.name} (all rows)")
                a = time.perf_counter()
                O.norm(cpu["W"], cpu["A"], cpu["B"], sh.s)
                parts.append(f"{sh.name}: full norm {time.perf_counter() - a:.1f} s")
        total_s += sec
    return {"value": round(total_s * 1e6, 0), "unit": "µs", "cores": O.num_threads(),
            "kind": "oracle", "extrapolated": not (args.cpu_full and args.config != "c4"),
            "sample": "oracle forward (fp64, dense W + sBA rows) at the full module shape; "
                      + "; ".join(parts)}


if __name__ == "__main__":
    main()
