// gemm_dma_cfg.hip - one tile configuration of the pipelined bf16 GEMM:
// its kernels (single product and grouped launch, every operand layout) and
// their launchers.  Compiled once per configuration with DORA_DMA_CFG = 0..7
// (256 x 256 with its persistent kernels, 256 x 128, 128 x 128, 128 x 384,
// 384 x 128; 5: the 128 x 384 kernels that also sum squares of rows; 6: the
// other grouped 128 x 384 ones; 7: 128 x 384 with eight waves).
#include "gemm_dma_launch.hpp"

#ifndef DORA_DMA_CFG
#error "DORA_DMA_CFG selects the tile configuration"
#endif

namespace dora {

// Explicit instantiations of the kernels: with implicit instantiation from
// the launchers alone, the host compiler emitted launch stubs for only some
// of them.
#define DORA_DMA_CONFIG(BM, BN, WM, WN)                                                         \
    template __global__ void dma::gemm_bf16_dma_kernel<BM, BN, WM, WN, true, true, false>(      \
        GemmArgs);                                                                              \
    template __global__ void dma::gemm_bf16_dma_kernel<BM, BN, WM, WN, true, false, false>(     \
        GemmArgs);                                                                              \
    template __global__ void dma::gemm_bf16_dma_kernel<BM, BN, WM, WN, false, false, false>(    \
        GemmArgs);                                                                              \
    template __global__ void dma::gemm_bf16_dma_grouped_kernel<BM, BN, WM, WN, true, true,      \
                                                               false>(GemmGroup);               \
    template __global__ void dma::gemm_bf16_dma_grouped_kernel<BM, BN, WM, WN, true, false,     \
                                                               false>(GemmGroup);               \
    hipError_t launch_dma_##BM##x##BN(const GemmArgs &a, int layout, bool rowsq, hipStream_t st) \
    {                                                                                           \
        return dma::launch_dma_layout<BM, BN, WM, WN>(a, layout, rowsq, st);                    \
    }                                                                                           \
    hipError_t launch_dma_group_##BM##x##BN(GemmGroup &g, int layout, bool rowsq, hipStream_t st) \
    {                                                                                           \
        return dma::launch_dma_group_layout<BM, BN, WM, WN>(g, layout, rowsq, st);              \
    }

#if DORA_DMA_CFG == 0
DORA_DMA_CONFIG(256, 256, 2, 2)
template __global__ void dma::gemm_bf16_dma_persistent_kernel<256, 256, 2, 2, true>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_persistent_kernel<256, 256, 2, 2, false>(GemmArgs);
#elif DORA_DMA_CFG == 1
DORA_DMA_CONFIG(256, 128, 2, 2)
#elif DORA_DMA_CFG == 2
DORA_DMA_CONFIG(128, 128, 2, 2)
// with the row sums of squares too (the norm's U = W A^T at small rank)
template __global__ void dma::gemm_bf16_dma_kernel<128, 128, 2, 2, true, true, true>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 128, 2, 2, true, true, true>(
    GemmGroup);
#elif DORA_DMA_CFG == 3
// the 1 x 4 layout also sums the squares of A's rows (the norm's base term);
// those two kernels compile in a unit of their own (DORA_DMA_CFG 5)
extern template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 1, 4, true, true, true>(
    GemmArgs);
extern template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, true,
                                                                  true>(GemmGroup);
// and so do its grouped kernels (DORA_DMA_CFG 6)
extern template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, true,
                                                                  false>(GemmGroup);
extern template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, false,
                                                                  false>(GemmGroup);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 1, 4, true, true, false>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 1, 4, true, false, false>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 1, 4, false, false, false>(GemmArgs);
hipError_t launch_dma_128x384(const GemmArgs &a, int layout, bool rowsq, hipStream_t st)
{
    return dma::launch_dma_layout<128, 384, 1, 4>(a, layout, rowsq, st);
}
hipError_t launch_dma_group_128x384(GemmGroup &g, int layout, bool rowsq, hipStream_t st)
{
    return dma::launch_dma_group_layout<128, 384, 1, 4>(g, layout, rowsq, st);
}
#elif DORA_DMA_CFG == 4
DORA_DMA_CONFIG(384, 128, 4, 1)
#elif DORA_DMA_CFG == 5
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 1, 4, true, true, true>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, true, true>(
    GemmGroup);
#elif DORA_DMA_CFG == 6
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, true, false>(
    GemmGroup);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 1, 4, true, false, false>(
    GemmGroup);
#elif DORA_DMA_CFG == 7
// 128 x 384 with eight waves (2 x 4), with and without the row sums of squares
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 2, 4, true, true, true>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 2, 4, true, true, false>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 2, 4, true, false, false>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 2, 4, false, false, false>(GemmArgs);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 2, 4, true, true, true>(
    GemmGroup);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 2, 4, true, true, false>(
    GemmGroup);
template __global__ void dma::gemm_bf16_dma_grouped_kernel<128, 384, 2, 4, true, false, false>(
    GemmGroup);
hipError_t launch_dma_128x384w8(const GemmArgs &a, int layout, bool rowsq, hipStream_t st)
{
    return dma::launch_dma_layout<128, 384, 2, 4>(a, layout, rowsq, st);
}
hipError_t launch_dma_group_128x384w8(GemmGroup &g, int layout, bool rowsq, hipStream_t st)
{
    return dma::launch_dma_group_layout<128, 384, 2, 4>(g, layout, rowsq, st);
}
// dB with dh and the dm sums produced on the way (both operands MN-major)
template __global__ void dma::gemm_bf16_dma_kernel<128, 384, 2, 4, false, false, false, true>(
    GemmArgs);
hipError_t launch_dma_dhdm_128x384w8(const GemmArgs &a, hipStream_t st)
{
    return dma::launch_dma<128, 384, 2, 4, false, false, false, true>(a, st);
}
#else
#error "DORA_DMA_CFG out of range"
#endif

}  // namespace dora
