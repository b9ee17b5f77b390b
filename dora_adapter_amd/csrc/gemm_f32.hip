// gemm_f32.hip - true-fp32 GEMM on the vector ALUs for fp32 DoRA modules.
//
// Same contract as the bf16 MFMA GEMM (GemmArgs: up to two K segments,
// split-K, store / row-dot epilogues, optional row sums of squares of A) so
// that the fp32 module runs the identical factored-norm, forward and
// backward pipeline; no operand is ever rounded below fp32.  64 x 64 tile,
// 256 threads, each thread a 4 x 4 block of outputs, K step 16, operands
// staged in LDS K-major (As[k][m]) for conflict-free broadcast reads.
#include "dora_internal.hpp"
#include "epilogue.hpp"

namespace dora {
namespace {

constexpr int BM = GEMM_F32_BM, BN = GEMM_F32_BN, BK = GEMM_F32_BK, NT = 256;

template <bool KMAJ, int R>
__device__ __forceinline__ void load_tile_f32(float (*S)[R + 4], const float *__restrict__ p,
                                              int64_t ld, int64_t MN, int64_t K, int64_t mn0,
                                              int64_t k0, int tid)
{
#pragma unroll
    for (int i = 0; i < (R * BK) / NT; ++i) {
        const int idx = tid + i * NT;
        int row, kk;
        if constexpr (KMAJ) {
            row = idx / BK;
            kk = idx % BK;
        } else {
            kk = idx / R;
            row = idx % R;
        }
        const int64_t mn = mn0 + row, k = k0 + kk;
        float v = 0.f;
        if (mn < MN && k < K)
            v = KMAJ ? p[mn * ld + k] : p[k * ld + mn];
        S[kk][row] = v;
    }
}

template <bool AK, bool BKM, bool ROWSQ>
__global__ void __launch_bounds__(NT) gemm_f32_kernel(GemmArgs g)
{
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ float Cs[BM * (BN + 4)];

    const int tid = static_cast<int>(threadIdx.x);
    const int tx = tid % 16, ty = tid / 16;
    int tm, tn;
    tile_coords(g.M, g.N, BM, BN, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
    const int z = static_cast<int>(blockIdx.y);

    const int64_t st1 = (g.seg[0].K + BK - 1) / BK;
    const int64_t st_total = st1 + (g.nseg > 1 ? (g.seg[1].K + BK - 1) / BK : 0);
    int64_t s_begin = static_cast<int64_t>(z) * g.steps_per_split;
    if (s_begin > st_total)
        s_begin = st_total;
    int64_t s_end = s_begin + g.steps_per_split;
    if (s_end > st_total)
        s_end = st_total;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.f;
    float sq = 0.f;

    for (int64_t s = s_begin; s < s_end; ++s) {
        const bool first = s < st1;
        const GemmSeg &sg = first ? g.seg[0] : g.seg[1];
        const int64_t k0 = (first ? s : s - st1) * BK;
        load_tile_f32<AK, BM>(As, static_cast<const float *>(sg.a), sg.lda, g.M, sg.K, m0, k0, tid);
        load_tile_f32<BKM, BN>(Bs, static_cast<const float *>(sg.b), sg.ldb, g.N, sg.K, n0, k0,
                               tid);
        __syncthreads();
        if constexpr (ROWSQ) {
            if (tid < BM) {
#pragma unroll
                for (int kk = 0; kk < BK; ++kk)
                    sq += As[kk][tid] * As[kk][tid];
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }

    if constexpr (ROWSQ) {
        if (g.rowsq != nullptr && tn == 0 && tid < BM && m0 + tid < g.M)
            g.rowsq[static_cast<int64_t>(z) * g.M + m0 + tid] = sq;
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            Cs[(ty * 4 + i) * (BN + 4) + tx * 4 + j] = acc[i][j];
    __syncthreads();
    epilogue_rows<BM, BN, BN + 4, NT, float>(Cs, g, m0, n0, z, tn, tid);
}

template <bool AK, bool BKM, bool RS>
hipError_t launch_one(const GemmArgs &a, hipStream_t st)
{
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles == 0 || a.splits == 0)
        return hipSuccess;
    dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.splits));
    hipLaunchKernelGGL((gemm_f32_kernel<AK, BKM, RS>), grid, dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, int layout, bool rowsq, hipStream_t st)
{
    switch (layout) {
    case 0:
        return rowsq ? launch_one<true, true, true>(a, st) : launch_one<true, true, false>(a, st);
    case 1:
        return launch_one<true, false, false>(a, st);
    case 2:
        return launch_one<false, false, false>(a, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dora
