"""bench.py's host-side contract, on the CPU: more than one GPU is refused
with a message before any device work, the peaks are the MI355X's published
dense figures, the norm's flop count is the per-module formula written out
term by term, and the stored counter record describes the x W^T launch it
claims to (algorithmic bytes of that shape, write bytes = the bf16 output)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_peaks():
    assert bench.PEAK_BF16_TFLOPS == 2500.0
    assert bench.PEAK_HBM_GBPS == 8000.0


def test_norm_flops_terms():
    """The algorithmic count: B G once (the kernels' split of G into a bf16
    hi/lo pair is an implementation choice, not work the method asks for)."""
    d_out, d_in, r = 28672, 8192, 384
    u = 2 * d_out * d_in * r          # U = W A^T
    g = 2 * r * r * d_in              # G = A A^T
    bg = 2 * d_out * r * r            # B G
    base = 2 * d_out * d_in           # row sums of W^2
    dots = 2 * (2 * d_out * r)        # cross and Gram row dots
    assert bench.norm_flops(d_out, d_in, r) == u + g + bg + base + dots
    # the square and MLP shapes scale the same way
    assert bench.norm_flops(64, 128, 8) == (2 * 64 * 128 * 8 + 2 * 8 * 8 * 128 + 2 * 64 * 8 * 8
                                            + 2 * 64 * 128 + 4 * 64 * 8)


def test_config_choices_and_workloads():
    assert bench.parse_args([]).config == "c5"
    for c in bench.CONFIGS:
        assert bench.parse_args(["--config", c]).config == c
        shapes = bench.workload(c)
        assert all(sh.dtype == "bf16" for sh in shapes)
    up, down = bench.workload("c4")
    assert (up.d_in, up.d_out, down.d_in, down.d_out) == (5120, 27648, 27648, 5120)
    assert up.T == down.T == 16384 and up.r == down.r == 384
    assert bench.workload("c5")[0].backward


def test_traffic_record_describes_the_base_product():
    with open(bench.TRAFFIC_FILE) as fh:
        tr = json.load(fh)
    T, d_in, d_out = 8192, 8192, 28672
    algorithmic = 2 * (T * d_in + d_out * d_in + T * d_out)  # x, W read; y written (bf16)
    assert tr["algorithmic_bytes_per_launch"] == algorithmic
    cal = tr["copy_calibration"]
    # the scaled counters reproduce the stored byte count
    hbm = (tr["fetch_size_kib_per_launch"] * 1024 * cal["bytes"] / 1024 / cal["fetch_size_kib"]
           + tr["write_size_kib_per_launch"] * 1024 * cal["bytes"] / 1024 / cal["write_size_kib"])
    assert abs(hbm - tr["hbm_bytes_per_launch"]) <= 1e-6 * hbm
    # every output byte is written once: WRITE_SIZE scaled equals the bf16 output
    writes = tr["write_size_kib_per_launch"] * 1024 * cal["bytes"] / 1024 / cal["write_size_kib"]
    assert abs(writes - 2 * T * d_out) <= 1e-3 * writes
    assert len(tr["kernel_source_hash"]) == 16


def test_norm_roles_of_each_launch_form():
    """The norm's kernels are told apart by name (finalize, finish) and by
    position (the products): the five-launch form, G's tiles unsplit or
    split in U's launch, and the finish inside B G's epilogue."""
    g = "void dora::dma::gemm_bf16_dma_kernel<128, 384, 2, 4, true, true, false, false>(x)"
    u = "void dora::dma::gemm_bf16_dma_grouped_kernel<128, 384, 2, 4, true, true, true>(x)"
    bg = "void dora::dma::gemm_bf16_dma_kernel<128, 384, 2, 4, true, false, false, false>(x)"
    fz = "dora::(anonymous namespace)::gram_finalize_kernel(float const*, int, long)"
    fn = "dora::(anonymous namespace)::norm_finish_kernel(float const*, int)"
    assert bench.norm_roles([g, fz, u, bg, fn]) == list(bench.NORM_ROLES)
    assert bench.norm_roles([u, bg, fn]) == ["U_WAt_rowdot", "BG_rowdot", "finish"]
    assert bench.norm_roles([u, fz, bg, fn]) == ["U_WAt_rowdot", "gram_finalize", "BG_rowdot",
                                                 "finish"]
    assert bench.norm_roles([u, bg]) == ["U_WAt_rowdot", "BG_rowdot"]
    assert bench.norm_roles([u, fz, bg]) == ["U_WAt_rowdot", "gram_finalize", "BG_rowdot"]
    assert bench.norm_roles([g, fz, u, bg]) == ["gram_AAt", "gram_finalize", "U_WAt_rowdot",
                                                "BG_rowdot"]
    assert bench.norm_roles([u]) is None
