// gemm_dma_launch.hpp - launchers of the pipelined bf16 GEMM (gemm_bf16_dma.hpp),
// one set per tile configuration.  Each configuration's kernels are
// instantiated in their own translation unit (gemm_dma_cfg.hip, compiled once
// per configuration), so that the configurations compile in parallel.
#pragma once

#include "gemm_bf16_dma.hpp"
#include "gemm_persistent.hpp"

#include <atomic>
#include <cstdlib>

namespace dora {
namespace dma {

// The persistent 256 x 256 kernel (gemm_persistent.hpp) serves unsplit bf16
// stores, optionally column-scaled, of whole 16-byte column chunks into an
// output under 2 GiB, with at least two K stages.  DORA_PERSISTENT=0
// (environment) turns it off, so that tests can hold its results against
// the one-tile-per-workgroup launch.
inline bool persistent_ok(const GemmArgs &a)
{
    const char *e = getenv("DORA_PERSISTENT");
    if (e != nullptr && e[0] == '0' && e[1] == '\0')
        return false;
    const int64_t nst = (a.seg[0].K + GEMM_DMA_BK - 1) / GEMM_DMA_BK +
                        (a.nseg > 1 ? (a.seg[1].K + GEMM_DMA_BK - 1) / GEMM_DMA_BK : 0);
    return a.splits == 1 && a.mode == EPI_STORE && !a.out_f32 && !a.out_accum &&
           a.out2 == nullptr && (a.colm == nullptr) == (a.coln == nullptr) && a.N % 8 == 0 &&
           a.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 &&
           a.M * a.ldc * 2 < 0x7fffffffLL && nst >= 2;
}

// Compute units per XCD (8 XCDs) of the current device, looked up once per
// device.
inline int cus_per_xcd()
{
    constexpr int kMaxDev = 64, kDefault = 32;  // MI355X: 256 CUs
    static std::atomic<int> cached[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return kDefault;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            cus < 8)
            cus = 8 * kDefault;
        v = cus / 8;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool RS, bool DH = false>
hipError_t launch_dma(const GemmArgs &a, hipStream_t st)
{
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles == 0 || a.splits == 0)
        return hipSuccess;
    if constexpr (BM == 256 && BN == 256 && AK && !RS && !DH) {
        if (persistent_ok(a)) {
            const int64_t per = std::min<int64_t>(cus_per_xcd(), (tiles + 7) / 8);
            hipLaunchKernelGGL((dma::gemm_bf16_dma_persistent_kernel<BM, BN, WM, WN, BKM>),
                               dim3(static_cast<unsigned>(8 * per)), dim3(WM * WN * 64), 0, st,
                               a);
            return hipGetLastError();
        }
    }
    dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.splits));
    hipLaunchKernelGGL((dma::gemm_bf16_dma_kernel<BM, BN, WM, WN, AK, BKM, RS, DH>), grid,
                       dim3(WM * WN * 64), 0, st, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_dma_layout(const GemmArgs &a, int layout, bool rowsq, hipStream_t st)
{
    switch (layout) {
    case 0:
        if (rowsq) {
            if constexpr (BM == 128 && (BN == 384 || BN == 128))
                return launch_dma<BM, BN, WM, WN, true, true, true>(a, st);
            else
                return hipErrorInvalidValue;
        }
        return launch_dma<BM, BN, WM, WN, true, true, false>(a, st);
    case 1:
        return launch_dma<BM, BN, WM, WN, true, false, false>(a, st);
    case 2:
        return launch_dma<BM, BN, WM, WN, false, false, false>(a, st);
    default:
        return hipErrorInvalidValue;
    }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool RS>
hipError_t launch_dma_group(GemmGroup &g, hipStream_t st)
{
    int64_t total = 0;
    for (int p = 0; p < g.count; ++p) {
        g.tile_start[p] = static_cast<int>(total);
        const GemmArgs &a = g.p[p];
        total += ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splits;
    }
    g.tile_start[g.count] = static_cast<int>(total);
    if (total == 0)
        return hipSuccess;
    if (total > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((dma::gemm_bf16_dma_grouped_kernel<BM, BN, WM, WN, AK, BKM, RS>),
                       dim3(static_cast<unsigned>(total)), dim3(WM * WN * 64), 0, st, g);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_dma_group_layout(GemmGroup &g, int layout, bool rowsq, hipStream_t st)
{
    switch (layout) {
    case 0:
        if (rowsq) {
            if constexpr (BM == 128 && (BN == 384 || BN == 128))
                return launch_dma_group<BM, BN, WM, WN, true, true, true>(g, st);
            else
                return hipErrorInvalidValue;
        }
        return launch_dma_group<BM, BN, WM, WN, true, true, false>(g, st);
    case 1:
        if (rowsq)
            return hipErrorInvalidValue;
        return launch_dma_group<BM, BN, WM, WN, true, false, false>(g, st);
    default:
        return hipErrorInvalidValue;
    }
}


}  // namespace dma

// Per-configuration entry points (layout as in launch_gemm_bf16).
#define DORA_DMA_LAUNCHERS(BM, BN)                                                            \
    hipError_t launch_dma_##BM##x##BN(const GemmArgs &a, int layout, bool rowsq,                \
                                      hipStream_t st);                                          \
    hipError_t launch_dma_group_##BM##x##BN(GemmGroup &g, int layout, bool rowsq, hipStream_t st);
DORA_DMA_LAUNCHERS(256, 256)
DORA_DMA_LAUNCHERS(256, 128)
DORA_DMA_LAUNCHERS(128, 128)
DORA_DMA_LAUNCHERS(128, 384)
DORA_DMA_LAUNCHERS(384, 128)
DORA_DMA_LAUNCHERS(128, 384w8)
#undef DORA_DMA_LAUNCHERS
hipError_t launch_dma_dhdm_128x384w8(const GemmArgs &a, hipStream_t st);

}  // namespace dora
