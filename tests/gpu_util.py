"""Helpers for the GPU parity tests: device transfer and the tolerance rules.

Tolerances (fp64 oracle as reference; rms over the compared set):
  fp32 modules: row norm |n - n_ref| / n_ref <= 1e-5; every element of an
                output or gradient within 1e-5 * max(|ref|, rms(ref)).
  bf16 modules: row norm relative error <= 1e-3; every element within
                2e-2 * max(|ref|, rms(ref)); cosine(out, ref) >= 0.9999
                over the flattened compared set.
  bf16 weight gradients over a handful of tokens (T <= 8): an element may
                instead lie within the a-priori rounding bound of the
                bf16-stored operands it is summed from (reduction_bound_bf16).
"""
import math
import sys

import numpy as np
import torch

DEV = "cuda:0"

NORM_TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-3}
ELEM_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
COS_MIN = 0.9999


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def gpu(t):
    return t.to(DEV, non_blocking=False).contiguous()


def np64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def check_norm(n, n_ref, dtype, what="n", tol=None):
    n, n_ref = np64(n), np64(n_ref)
    tol = NORM_TOL[dtype] if tol is None else tol
    rel = np.abs(n - n_ref) / np.abs(n_ref)
    assert np.all(np.isfinite(n)), f"{what}: non-finite"
    assert rel.max() <= tol, f"{what}: max rel err {rel.max():.3e} > {tol} (row {rel.argmax()})"
    return float(rel.max())


def check_close(got, ref, dtype, what, tol=None, cos=True, bound=None):
    """Every element within tol * max(|ref|, rms(ref)), or, where `bound` (an
    array of ref's shape) is given, within that bound instead if it is larger."""
    g, r = np64(got).reshape(-1), np64(ref).reshape(-1)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    tol = ELEM_TOL[dtype] if tol is None else tol
    if r.size == 0:
        return {}
    rms = math.sqrt(float(np.mean(r * r)))
    lim = tol * np.maximum(np.abs(r), rms)
    if bound is not None:
        lim = np.maximum(lim, np64(bound).reshape(-1))
    err = np.abs(g - r)
    bad = err > lim
    worst = float((err / np.maximum(lim, 1e-300)).max())
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{r.size} elements out of tolerance "
                           f"(worst {worst:.2f}x the limit at {int(np.argmax(err / lim))})")
    out = {"worst_frac_of_limit": worst}
    if cos and dtype == torch.bfloat16 and np.linalg.norm(r) > 0:
        c = float(np.dot(g, r) / (np.linalg.norm(g) * np.linalg.norm(r)))
        assert c >= COS_MIN, f"{what}: cosine {c:.6f} < {COS_MIN}"
        out["cos"] = c
    return out


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits)


def reduction_bound_bf16(dy, x, W, A, B, m, n, dm, s, through_norm):
    """A-priori bound on |dA - dA_exact| and |dB - dB_exact| for bf16 modules,
    from the precision reading: dh = g dy, P = x A^T, Q = s dh B and (through
    the norm) cB = c B, c = -s m dm / n^2, are each rounded once to bf16 (unit
    roundoff u) from fp32 values; V A^T stays fp32 with G as a ~16-bit pair;
    the result is rounded once (the caller adds that u |ref| term).  Each
    stored operand is within u of its own value, so summed over tokens
        dB:  (2u + u^2) |s| |dh|^T |P|
        dA:  (u + u^2) (|Q| + |s| |dh| |B|)^T |x|     (Q inherits dh's error)
    and, through the norm,
        dA: + u (|c| |B|)^T |V|
        dB: + 2^-16 |c| |s| |B| |G|
    with |P|, |Q|, |V|, |G| the magnitudes of the exact values.  Every fp32
    accumulation adds K 2^-23 of its sum of absolute terms (K its length).
    Inputs are float64 arrays or tensors (n and dm the oracle's); returns
    (dA_bound, dB_bound).  When a sum over a few tokens cancels, this bound can
    exceed 2e-2 rms(ref); it is meant for small token counts."""
    dy, x, W, A, B, m, n, dm = (np64(v) for v in (dy, x, W, A, B, m, n, dm))
    T, d_out = dy.shape
    d_in = x.shape[1]
    u, sa = U_BF16, abs(s)
    f32 = (T + d_out + d_in) * 2.0 ** -23
    ax, aW, aA, aB = np.abs(x), np.abs(W), np.abs(A), np.abs(B)
    dh = dy * (m / n)
    adh = np.abs(dh)
    aP, sumP = np.abs(x @ A.T), ax @ aA.T
    aQ, sumQ = np.abs(s * dh @ B), sa * adh @ aB
    bB = (2 * u + u * u + f32) * sa * adh.T @ aP + f32 * sa * adh.T @ sumP
    bA = (u + u * u + f32) * (aQ + sumQ).T @ ax
    if through_norm:
        ac = np.abs(s * m * dm / (n * n))
        acB = ac[:, None] * aB
        V = W + s * B @ A
        sumV = aW + sa * aB @ aA
        bA = bA + (u + f32) * acB.T @ np.abs(V) + f32 * acB.T @ sumV
        aG = np.abs(A @ A.T)
        bB = bB + ac[:, None] * ((2.0 ** -16 + f32) * sa * aB @ aG
                                 + f32 * (sumV @ aA.T))
    return bA, bB


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v)
    a = np.where(a == 0, np.finfo(np.float32).tiny, a)
    e = np.floor(np.log2(a))
    return np.exp2(e - 7)


def sample_pairs(seed, n, b0, b1):
    g = torch.Generator().manual_seed(seed)
    a = torch.randint(0, b0, (n,), generator=g)
    b = torch.randint(0, b1, (n,), generator=g)
    pairs = [(0, 0), (b0 - 1, b1 - 1)] + list(zip(a.tolist(), b.tolist()))
    return pairs


def sample_ids(seed, n, b):
    g = torch.Generator().manual_seed(seed)
    ids = torch.randperm(b, generator=g)[:n].tolist()
    return sorted(set(ids + [0, b - 1]))
