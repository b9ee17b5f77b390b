"""GPU parity on the method's degenerate and extreme cases, each against the
oracle (forward, detached backward, backward through the norm, merge):

  * s = 0: the adapter drops out; n is the plain row norm of W, dA and dB
    are exactly zero;
  * the smallest bf16 module (d_out = d_in = r = 8, one token);
  * a full-rank adapter (r = d_in);
  * a negative scale, and magnitudes of both signs (the stable form and the
    backward hold for any m != 0);
  * a large scale (s = 16): g far from one, the adapter term dominating."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, check_norm, gpu, np64, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _run(mod, s):
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s)
    det = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y)
    thru = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y,
                           through_norm=True)
    Wm = D.dora_merge(t["W"], t["A"], t["B"], t["m"], s)
    torch.cuda.synchronize()
    return y, n, det, thru, Wm


def _check_all(mod, s, tag):
    y, n, det, thru, Wm = _run(mod, s)
    args = (mod["x"], mod["W"], mod["A"], mod["B"], mod["m"])
    n_ref = O.norm(mod["W"], mod["A"], mod["B"], s)["n"]
    y_ref, _ = O.forward(*args, s)
    check_norm(n, n_ref, BF, f"n {tag}")
    check_close(y, y_ref, BF, f"y {tag}")
    det_ref = O.backward_full(mod["dy"], *args, n_ref, s)
    thru_ref = O.backward_through_norm(mod["dy"], *args, s)
    for k in ("dx", "dA", "dB", "dm"):
        check_close(det[k], det_ref[k], BF, f"{k} detached {tag}")
        check_close(thru[k], thru_ref[k], BF, f"{k} through norm {tag}")
    check_close(Wm, O.merge(mod["W"], mod["A"], mod["B"], mod["m"], s), BF, f"merge {tag}")
    return y, n, det, thru


def test_zero_scale():
    """s = 0: n_i = ||W_i|| (the textbook row norm, computed here in fp64 by
    numpy), and no gradient reaches A or B."""
    say("degenerate s = 0")
    mod = synth.custom(520, 1032, 40, 200, "bf16", 0.0, sigma_B=0.05, seed=31, with_dy=True)
    y, n, det, thru = _check_all(mod, 0.0, "s=0")
    check_norm(n, np.linalg.norm(np64(mod["W"]), axis=1), BF, "n = ||W_i||")
    for g in (det, thru):
        assert torch.all(g["dA"] == 0) and torch.all(g["dB"] == 0)


def test_smallest_module():
    say("degenerate 8 x 8, r 8, one token")
    mod = synth.custom(8, 8, 8, 1, "bf16", 2.0, sigma_B=0.1, seed=32, with_dy=True)
    _check_all(mod, 2.0, "8x8 r8 T1")


def test_full_rank_adapter():
    say("degenerate r = d_in")
    mod = synth.custom(264, 64, 64, 96, "bf16", 0.5, sigma_B=0.05, seed=33, with_dy=True)
    _check_all(mod, 0.5, "r = d_in = 64")


def test_negative_scale_and_magnitudes_of_both_signs():
    say("negative s, mixed-sign m")
    mod = synth.custom(600, 1032, 40, 130, "bf16", -1.5, sigma_B=0.02, seed=34, with_dy=True)
    m = mod["m"].clone()
    m[1::3] = -m[1::3]
    mod["m"] = m
    _check_all(mod, -1.5, "s=-1.5, m +/-")


def test_large_scale():
    say("large s")
    mod = synth.custom(520, 1032, 40, 130, "bf16", 16.0, sigma_B=0.02, seed=35, with_dy=True)
    _check_all(mod, 16.0, "s=16")
    g = np64(mod["m"]) / O.norm(mod["W"], mod["A"], mod["B"], 16.0)["n"]
    assert g.max() < 0.9, "the case is meant to leave the near-unity regime"
