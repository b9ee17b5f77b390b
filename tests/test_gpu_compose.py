"""GPU parity: dora_compose (stable single-pass form) vs the oracle's plain
y = (m/n)(base + s*lora), including the near-unity regime where g = m/n is
within 1e-6 .. 1e-2 of one.

A thread of the compose kernel streams one 8-column group down every R-th
row from its first (the grid sweeps R whole rows at a time: between 2^17 and
2^18 threads, about T / 64 per column group, over the column groups).  The large cases below make R not divide T,
so the last sweep is partial and threads take different row counts (at the
benchmarked 8192 x 28672 output R = 73: 112 or 113 rows per thread), in
place and out of place."""
import numpy as np
import pytest
import torch

from dora_adapter_amd import dora as D
from gpu_util import bf16_ulp, check_close, gpu, np64, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _inputs(T, d_out, dtype, seed, delta=None):
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(T, d_out, generator=g).to(dtype)
    lora = torch.randn(T, d_out, generator=g).to(dtype)
    n = (torch.rand(d_out, generator=g) * 1.5 + 0.5).float()
    if delta is None:
        m = (n.double() * (1 + 1e-3 * torch.randn(d_out, generator=g).double())).float()
    else:
        m = (n.double() * (1 + delta)).float()
    return base, lora, m, n


def _check(y, base, lora, m, n, s, dtype, what):
    ref = O.compose(base, lora, m, n, s)
    got = np64(y)
    # The kernel evaluates y = b + fma(g - 1, b, (g s) l) with g - 1 and g s
    # each rounded once to fp32, then (g s) l, the fma and the final add: with
    # u = 2^-24, |err| <= u |y| + u |(g-1) b + g s l| + u |g-1| |b| + 2u |g s l|
    # <= u |b| (1 + 3 |g-1|) + 4u |g s l| <= 4u (|b| + |g s l|) for |g-1| <= 1,
    # a bound in the operand magnitudes (not |y|: base and s lora may cancel);
    # bf16 output adds at most one bf16 ulp of rounding.
    g = np64(m) / np64(n)
    operand = np.abs(np64(base)) + np.abs(g * s * np64(lora))
    err = np.abs(got - ref)
    bound = 4 * 2.0 ** -24 * operand + 1e-30
    if dtype == torch.bfloat16:
        bound = bound + bf16_ulp(ref)
        exact = torch.tensor(ref).float().bfloat16().double().numpy()
        frac = float(np.mean(got == exact))
        assert frac > 0.95, f"{what}: only {frac:.3f} correctly rounded"
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} beyond bound, worst " \
                                 f"{(err / bound).max():.2f}x"


@pytest.mark.parametrize("T,d_out,dtype", [
    (37, 200, torch.bfloat16), (1000, 4096, torch.bfloat16), (3, 8, torch.bfloat16),
    (37, 201, torch.bfloat16), (5, 3, torch.bfloat16),  # ragged widths: element by element
    (16, 64, torch.float32), (33, 60, torch.float32), (129, 1000, torch.float32),
])
def test_compose_matches_oracle(T, d_out, dtype):
    say("compose", T, d_out, dtype)
    base, lora, m, n = _inputs(T, d_out, dtype, seed=T + d_out)
    s = 1.5
    y = D.dora_compose(gpu(base), gpu(lora), gpu(m), gpu(n), s)
    torch.cuda.synchronize()
    _check(y.cpu(), base, lora, m, n, s, dtype, f"compose {T}x{d_out}")


@pytest.mark.parametrize("delta", [1e-6, -1e-6, 1e-4, -1e-4, 1e-2, -1e-2, 0.0])
def test_compose_near_unity(delta):
    say("compose near-unity", delta)
    dtype = torch.bfloat16
    base, lora, m, n = _inputs(257, 512, dtype, seed=7, delta=delta)
    s = 1.0
    y = D.dora_compose(gpu(base), gpu(lora), gpu(m), gpu(n), s)
    torch.cuda.synchronize()
    _check(y.cpu(), base, lora, m, n, s, dtype, f"near-unity {delta}")


def test_compose_in_place_and_empty():
    say("compose in place")
    dtype = torch.bfloat16
    base, lora, m, n = _inputs(64, 128, dtype, seed=3)
    gb = gpu(base)
    y = D.dora_compose(gb, gpu(lora), gpu(m), gpu(n), 2.0, y=gb)
    torch.cuda.synchronize()
    assert y.data_ptr() == gb.data_ptr()
    _check(y.cpu(), base, lora, m, n, 2.0, dtype, "in place")
    e = torch.empty(0, 128, dtype=dtype, device="cuda:0")
    D.dora_compose(e, e.clone(), gpu(m), gpu(n), 1.0)
    torch.cuda.synchronize()


def test_compose_m_equals_n_is_exact_lora_sum():
    """g = 1 exactly: y = RN(base + s*lora) bit for bit."""
    say("compose m == n")
    base, lora, _, n = _inputs(128, 256, torch.bfloat16, seed=5)
    y = D.dora_compose(gpu(base), gpu(lora), gpu(n), gpu(n), 0.5)
    torch.cuda.synchronize()
    ref = (base.float() + 0.5 * lora.float()).bfloat16()
    assert torch.equal(y.cpu(), ref)


def test_compose_deterministic():
    say("compose determinism")
    base, lora, m, n = _inputs(300, 1024, torch.bfloat16, seed=11)
    a = D.dora_compose(gpu(base), gpu(lora), gpu(m), gpu(n), 1.0)
    b = D.dora_compose(gpu(base), gpu(lora), gpu(m), gpu(n), 1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _sweep_rows(T, d_out):
    """Rows per sweep of the compose launch: gpr T / 64 threads over the gpr
    column groups, within [2^17, 2^18] threads."""
    gpr = (d_out + 7) // 8
    threads = min(max(gpr * T // 64, 1 << 17), 1 << 18)
    return max(min((threads + gpr // 2) // gpr, T), 1)


@pytest.mark.parametrize("T,d_out,dtype,rows", [
    (4100, 8192, torch.bfloat16, 128),    # 32 whole sweeps and 4 rows
    (4100, 16384, torch.float32, 64),     # 64 whole sweeps and 4 rows, fp32
])
@pytest.mark.parametrize("in_place", [False, True])
def test_compose_sweeps_full(T, d_out, dtype, rows, in_place):
    assert _sweep_rows(T, d_out) == rows and T % rows
    say("compose sweeps", T, d_out, dtype, "in place" if in_place else "out of place")
    base, lora, m, n = _inputs(T, d_out, dtype, seed=T + d_out + in_place)
    s = 0.75
    gb = gpu(base)
    y = D.dora_compose(gb, gpu(lora), gpu(m), gpu(n), s, y=gb if in_place else None)
    torch.cuda.synchronize()
    assert (y.data_ptr() == gb.data_ptr()) == in_place
    _check(y.cpu(), base, lora, m, n, s, dtype, f"compose {T}x{d_out}")


@pytest.mark.parametrize("T", [8192, 8191])
@pytest.mark.parametrize("in_place", [False, True])
def test_compose_benchmark_shape_rows(T, in_place):
    """The benchmarked output, 8192 x 28672 bf16 (sweeps of 73 rows, the last
    one partial), and 8191 rows.  Every column of the first 64 rows, the last
    64 rows and 64 sampled rows is compared with the oracle."""
    d_out, dtype = 28672, torch.bfloat16
    assert _sweep_rows(T, d_out) == 73 and T % 73
    say("compose benchmark shape", T, d_out, "in place" if in_place else "out of place")
    base, lora, m, n = _inputs(T, d_out, dtype, seed=T + in_place)
    s = 1.0
    gb = gpu(base)
    y = D.dora_compose(gb, gpu(lora), gpu(m), gpu(n), s, y=gb if in_place else None)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(T)
    rows = sorted(set(range(64)) | set(range(T - 64, T)) |
                  set(torch.randint(64, T - 64, (64,), generator=g).tolist()))
    idx = torch.tensor(rows)
    _check(y[idx.to(y.device)].cpu(), base[idx], lora[idx], m, n, s, dtype,
           f"compose {T}x{d_out} sampled rows")
