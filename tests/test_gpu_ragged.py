"""GPU parity on bf16 modules of ragged width: d_in, d_out and r need not be
multiples of anything (rows of such widths are not 16-byte aligned, so the
products take the element-masked kernel configuration and the streaming
kernels their element-by-element paths).  Every case is a full comparison
of every output element with the oracle: norm and its three terms, forward
(y, P), both backwards, merge, the grouped norm and forward.

With few tokens (T <= 8) dA and dB may instead lie within the a-priori
rounding bound of the bf16-stored operands they are summed from
(gpu_util.reduction_bound_bf16), as in the random-shape tests."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import U_BF16, check_close, check_norm, gpu, np64, reduction_bound_bf16, say
from oracle import oracle as O
from test_gpu_norm import _terms_ok

pytestmark = pytest.mark.gpu

BF = torch.bfloat16

# (T, d_out, d_in, r, s)
CASES = [
    (129, 1001, 1003, 37, 1.0),    # every width ragged
    (64, 1001, 1024, 64, 2.0),     # only d_out: unaligned output rows
    (65, 1024, 1003, 64, 0.5),     # only d_in: unaligned K-major rows of x, W, A
    (33, 512, 512, 37, 1.0),       # only r: unaligned B, P, Q rows and G
    (1, 9, 13, 3, 1.0),            # tiny: a single partial tile everywhere
    (300, 130, 2051, 5, 0.125),    # long ragged K, split over K by the planner
]


@pytest.mark.parametrize("T,d_out,d_in,r,s", CASES)
def test_ragged_module(T, d_out, d_in, r, s):
    say("ragged module", T, d_out, d_in, r, s)
    mod = synth.custom(d_out, d_in, r, T, "bf16", s, sigma_B=0.03, seed=d_out + d_in + r,
                       with_dy=True)
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    terms = D.dora_factored_norm(t["W"], t["A"], t["B"], s, terms=True)
    y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s)
    det = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y)
    thru = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y,
                           through_norm=True)
    merged = D.dora_merge(t["W"], t["A"], t["B"], t["m"], s)
    torch.cuda.synchronize()

    _terms_ok(terms, O.norm(mod["W"], mod["A"], mod["B"], s), s, BF, "ragged norm")
    ref_y, ref_n = O.forward(mod["x"], mod["W"], mod["A"], mod["B"], mod["m"], s)
    check_norm(n, ref_n, BF, "n")
    check_close(y, ref_y, BF, "y")
    check_close(P, np64(mod["x"]) @ np64(mod["A"]).T, BF, "P")
    ref_det = O.backward_full(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"], mod["m"],
                              ref_n, s)
    ref_thru = O.backward_through_norm(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"],
                                       mod["m"], s)
    bounds = {}
    if T <= 8:
        args = (mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"], mod["m"], ref_n,
                ref_det["dm"], s)
        for path, ref in (("det", ref_det), ("thru", ref_thru)):
            bA, bB = reduction_bound_bf16(*args, path == "thru")
            bounds[path] = {"dA": bA + U_BF16 * np.abs(ref["dA"]),
                            "dB": bB + U_BF16 * np.abs(ref["dB"])}
    for k in ("dx", "dA", "dB", "dm"):
        check_close(det[k], ref_det[k], BF, f"detached {k}",
                    bound=bounds.get("det", {}).get(k))
        check_close(thru[k], ref_thru[k], BF, f"through-norm {k}",
                    bound=bounds.get("thru", {}).get(k))
    check_close(merged, O.merge(mod["W"], mod["A"], mod["B"], mod["m"], s), BF, "merge")


def test_ragged_in_grouped_calls():
    """A ragged module among aligned ones: the grouped norm and forward run
    it on its own path and match the oracle for every module."""
    say("ragged grouped")
    r = 24
    shapes = [("q", 264, 520), ("k", 100, 520), ("v", 264, 520)]
    mods = synth.make_group(shapes, r, seed=31)
    mods[1] = dict(mods[1])
    # module 1 gets a ragged rank: redraw its factors with r = 21
    alt = synth.make_group([("k", 100, 520)], 21, seed=32)[0]
    mods[1].update(A=alt["A"], B=alt["B"])
    g = [(gpu(md["W"]), gpu(md["A"]), gpu(md["B"]), gpu(md["m"]), md["s"]) for md in mods]
    ns = D.dora_factored_norm_grouped(g)
    x = (torch.randn(77, 520, generator=torch.Generator().manual_seed(33))).to(BF)
    ys, ns2, Ps = D.dora_forward_grouped(gpu(x), g)
    torch.cuda.synchronize()
    for i, md in enumerate(mods):
        ref_y, ref_n = O.forward(x, md["W"], md["A"], md["B"], md["m"], md["s"])
        check_norm(ns[i], ref_n, BF, f"grouped n {i}")
        check_norm(ns2[i], ref_n, BF, f"grouped forward n {i}")
        check_close(ys[i], ref_y, BF, f"grouped y {i}")
        check_close(Ps[i], np64(x) @ np64(md["A"]).T, BF, f"grouped P {i}")


def test_ragged_linear():
    say("ragged linear")
    gen = torch.Generator().manual_seed(34)
    x = torch.randn(45, 77, generator=gen).to(BF)
    W = (torch.randn(91, 77, generator=gen) / 9).to(BF)
    y = D.dora_linear(gpu(x), gpu(W))
    torch.cuda.synchronize()
    check_close(y, np64(x) @ np64(W).T, BF, "linear")
