"""GPU parity: dora_backward_through_norm (the gradient also flows through the
row norm n = ||W + sBA||) vs the oracle's dense chain rule.

Full comparisons of every gradient element at small and mid sizes (fp32 and
bf16, widths that are not tile multiples, a rank-384 case), dx and dm equal
bit for bit to the detached backward, determinism, the empty-token case,
every gradient at the training module's 28672 rows (64 tokens, d_in 1024),
and at the training module's full shape (d_in 8192 -> d_out 28672, r 384,
8192 tokens) on sampled entries: the detached part against the oracle and
the norm's correction to dB rows against its closed form from oracle
values.  The oracle forms V densely and takes its exact row norm; the GPU
call receives the factored n of its forward, which equals it to a few fp32
ulps."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from dora_adapter_amd import synth
from gpu_util import check_close, gpu, np64, say, sample_ids, sample_pairs
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _fwd(mod):
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], mod["s"])
    return t, y, n, P


def _bwd(t, y, n, P, s, through):
    g = D.dora_backward(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P, y,
                        through_norm=through)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("T,d_out,d_in,r,dtype,s", [
    (16, 64, 128, 8, "f32", 2.0),
    (33, 70, 100, 5, "f32", 0.75),            # fp32, no multiple-of-8 widths
    (300, 264, 520, 24, "bf16", 1.0),
    (200, 1000, 1024, 40, "bf16", 2.0),       # ragged d_out, several tiles
    (129, 512, 1024, 384, "bf16", 0.5),       # full rank 384
])
def test_through_norm_full(T, d_out, d_in, r, dtype, s):
    say("backward through norm", T, d_out, d_in, r, dtype)
    mod = synth.custom(d_out, d_in, r, T, dtype, s, sigma_B=0.02, seed=T + 7, with_dy=True)
    t, y, n, P = _fwd(mod)
    g = _bwd(t, y, n, P, s, True)
    ref = O.backward_through_norm(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"], mod["m"], s)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    for k in ("dx", "dA", "dB", "dm"):
        check_close(g[k], ref[k], tdt, f"{k} {T}x{d_out}x{d_in} r{r}")


def test_through_norm_shares_dx_dm_and_is_deterministic():
    """dx and dm do not depend on the path through n: same bits as the
    detached call.  dA and dB differ from it, and repeat bit for bit."""
    say("through norm vs detached")
    mod = synth.custom(1024, 2048, 128, 600, "bf16", 1.0, sigma_B=0.02, seed=61, with_dy=True)
    t, y, n, P = _fwd(mod)
    det = _bwd(t, y, n, P, 1.0, False)
    g1 = _bwd(t, y, n, P, 1.0, True)
    g2 = _bwd(t, y, n, P, 1.0, True)
    for k in ("dx", "dm"):
        assert torch.equal(g1[k], det[k]), k
    for k in ("dA", "dB"):
        assert not torch.equal(g1[k], det[k]), f"{k} has no norm term"
    for k in g1:
        assert torch.equal(g1[k], g2[k]), f"{k} not deterministic"


def test_through_norm_empty_tokens():
    say("through norm T=0")
    mod = synth.custom(64, 128, 8, 0, "bf16", 1.0, seed=5, with_dy=True)
    t, y, n, P = _fwd(mod)
    g = _bwd(t, y, n, P, 1.0, True)
    assert g["dx"].shape == (0, 128)
    for k in ("dA", "dB", "dm"):
        assert torch.all(g[k] == 0), k


def test_through_norm_full_size_sampled():
    """At the training shape the oracle cannot form every dm (that needs all
    of h = x V^T), so: dx, dm are the detached call's bits; sampled dm and
    the detached parts of dA, dB come from the oracle (with its own n); the
    norm's part of dB rows is its closed form with the coefficient
    cs_i = -s m_i dm_i / n_i^2, dm_i and n_i from the oracle:
      dB[i,k] - dB_det[i,k] = cs_i (V_i . A_k),  V = W + s B A.
    The norm's part of dA sums over every row: it is checked against the
    oracle on the training width at 64 tokens (next test)."""
    shape = synth.TRAIN_R384
    say("backward through norm full size", shape.name)
    mod = synth.make_module(shape, seed=0)
    s = mod["s"]
    t, y, n, P = _fwd(mod)
    det = _bwd(t, y, n, P, s, False)
    g = {k: v.cpu() for k, v in _bwd(t, y, n, P, s, True).items()}
    for k in ("dx", "dm"):
        assert torch.equal(g[k], det[k].cpu()), k
    del t, y, P, det
    torch.cuda.empty_cache()
    d_in, d_out, r = shape.d_in, shape.d_out, shape.r
    n_ref = O.norm(mod["W"], mod["A"], mod["B"], s)["n"]
    rows = sample_ids(11, 12, d_out)
    dB_idx = [(i, k) for i in rows for k in sample_ids(12 + i, 3, r)]
    dA_idx = sample_pairs(13, 12, r, d_in)
    ref = O.backward_sampled(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"], mod["m"],
                             n_ref, s, dA_idx=dA_idx, dB_idx=dB_idx, dm_idx=rows)
    check_close(np64(g["dm"])[rows], ref["dm"], torch.bfloat16, "dm sampled rows")
    W64, A64, B64, m64 = np64(mod["W"]), np64(mod["A"]), np64(mod["B"]), np64(mod["m"])
    cs_row = {i: -s * m64[i] * dmi / (n_ref[i] ** 2) for i, dmi in zip(rows, ref["dm"])}
    exp_dB = np.array([ref["dB"][q] + cs_row[i] * float((W64[i] + s * B64[i] @ A64) @ A64[k])
                       for q, (i, k) in enumerate(dB_idx)])
    got_dB = np.array([float(g["dB"][i, k]) for i, k in dB_idx])
    check_close(got_dB, exp_dB, torch.bfloat16, "dB sampled")


def test_through_norm_training_width_64_tokens():
    """Every gradient against the oracle at the training module's d_out
    (28672 rows, r 384) on 64 tokens and d_in 1024: the norm's part of dA is
    a sum over all 28672 rows (cs B)^T V."""
    say("backward through norm, 28672 rows, 64 tokens")
    mod = synth.custom(28672, 1024, 384, 64, "bf16", 1.0, sigma_B=0.02, seed=65, with_dy=True)
    t, y, n, P = _fwd(mod)
    g = _bwd(t, y, n, P, 1.0, True)
    ref = O.backward_through_norm(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"], mod["m"],
                                  1.0)
    for k in ("dx", "dA", "dB", "dm"):
        check_close(g[k], ref[k], torch.bfloat16, f"{k} 64x28672x1024 r384")


@pytest.mark.parametrize("T,d_out,d_in,r,dtype,s", [
    (300, 264, 520, 24, "bf16", 1.0),
    (129, 512, 1024, 384, "bf16", 0.5),
    (33, 70, 100, 5, "f32", 0.75),
    (64, 28672, 1024, 384, "bf16", 1.0),   # unsplit: V A^T written by the norm's own products
])
def test_through_norm_with_kept_U(T, d_out, d_in, r, dtype, s):
    """The forward keeps V A^T = W A^T + s B A A^T (U_out) and the backward
    through the norm reuses it (U): it matches its definition, the gradients
    match the oracle, and dx, dm are those of the call that forms it anew."""
    say("through norm with kept U", T, d_out, d_in, r, dtype)
    mod = synth.custom(d_out, d_in, r, T, dtype, s, sigma_B=0.02, seed=T + 11, with_dy=True)
    t = {k: gpu(mod[k]) for k in ("x", "W", "A", "B", "m", "dy")}
    U = torch.empty(d_out, r, dtype=torch.float32, device=t["x"].device)
    y, n, P = D.dora_forward(t["x"], t["W"], t["A"], t["B"], t["m"], s, U_out=U)
    kept = _bwd_U(t, y, n, P, s, U)
    fresh = _bwd(t, y, n, P, s, True)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    W64, A64, B64 = np64(mod["W"]), np64(mod["A"]), np64(mod["B"])
    U_ref = (W64 + s * B64 @ A64) @ A64.T   # the definition: V A^T
    # fp32 accumulation, not rounded; the s B G part carries G as a bf16
    # hi / lo pair (about 16 significant bits)
    check_close(U, U_ref, torch.float32, "V A^T", tol=1e-4)
    for k in ("dx", "dm"):
        assert torch.equal(kept[k], fresh[k]), k
    if d_out * d_in * T <= 2e8:
        ref = O.backward_through_norm(mod["dy"], mod["x"], mod["W"], mod["A"], mod["B"],
                                      mod["m"], s)
        for k in ("dA", "dB"):
            check_close(kept[k], ref[k], tdt, f"{k} with kept U")
    for k in ("dA", "dB"):
        check_close(kept[k], np64(fresh[k]), tdt, f"{k} kept U vs recomputed")


def _bwd_U(t, y, n, P, s, U):
    g = D.dora_backward_through_norm(t["dy"], t["x"], t["W"], t["A"], t["B"], t["m"], n, s, P,
                                     y, U=U)
    torch.cuda.synchronize()
    return g
