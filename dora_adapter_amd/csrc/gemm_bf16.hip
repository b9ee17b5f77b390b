// gemm_bf16.hip - bf16 GEMM on the gfx950 matrix cores (MFMA), fp32 accumulate.
//
// One kernel template serves every dense contraction of the DoRA module:
//   norm:     U = W A^T (row-dot with B -> cross, row sums of W^2 -> base),
//             G = A A^T (split-K partials), B [G_hi ; G_lo] (row-dot -> gram)
//   forward:  x W^T, x A^T, (x A^T) B^T
//   backward: dh B, [dh | Q] [W ; A], dh^T P, Q^T x
// ("Scaling DoRA" abstract: base, cross and Gram terms through
// O(d_out r + r^2) intermediates; the adapter and base products of the
// forward and backward passes.)
//
// Design (CDNA4, 64-wide wavefronts):
//   * workgroup tile BM x BN, K step 64, 4 wavefronts in a 2 x 2 grid, each
//     owning a (BM/2) x (BN/2) sub-tile of v_mfma_f32_16x16x32_bf16 tiles;
//   * operands staged global -> registers -> LDS, double-buffered, one
//     barrier per K step; the next step's global loads are in flight while
//     the current step's MFMAs run;
//   * LDS rows hold 64 K-values (128 B) as eight 16-byte chunks, chunk c of
//     row r stored at c ^ (r & 7) so that the 16 rows read by one MFMA
//     fragment load hit distinct banks;
//   * MN-major operands (the backward's dh^T, P, W, A, x) are transposed on
//     the way into LDS: each thread loads an 8 (k) x 8 (mn) block with eight
//     16-byte loads and transposes it in registers, so LDS always holds
//     K-contiguous rows and the MFMA fragment reads are the same for every
//     layout;
//   * the epilogue stages fp32 accumulators through LDS for 16-byte
//     coalesced stores or per-row dot products (epilogue.hpp);
//   * XCD-aware tile order (epilogue.hpp, tile_coords).
#include "dora_internal.hpp"
#include "epilogue.hpp"
#include "gemm_dma_launch.hpp"

namespace dora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = GEMM_BK;

// Registers a thread holds for one operand tile of R rows (M or N) x BK.
template <bool KMAJ, int R, int NT>
struct OpRegs {
    // K-major: R*8 chunks of 16 B over NT threads.  MN-major: R 8x8 blocks
    // (BK/8 = 8 block rows times R/8 block columns), one per thread at most
    // ceil(R/NT) times, 8 chunks each.
    static constexpr int PER = KMAJ ? (R * 8) / NT : ((R + NT - 1) / NT) * 8;
};

// Eight consecutive bf16 values p[0 .. 8) with those at or past `live`
// read as zero, loaded one by one (for rows of a ragged width, which need
// not be 16-byte aligned).
__device__ __forceinline__ uint4 load8_masked(const uint16_t *__restrict__ p, int64_t live)
{
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = 2 * q < live ? p[2 * q] : 0u;
        const uint32_t hi = 2 * q + 1 < live ? p[2 * q + 1] : 0u;
        w[q] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// RG (ragged): any K, M, N and leading dimension; every element is loaded
// on its own and masked.  Otherwise K-major operands need K and ld
// multiples of 8, MN-major ones M (or N) and ld multiples of 8, so that
// every 16-byte chunk is aligned and wholly in or wholly out.
template <bool KMAJ, int R, int NT, bool RG, int NV>
__device__ __forceinline__ void load_operand(uint4 (&v)[NV], const uint16_t *__restrict__ p,
                                             int64_t ld, int64_t MN, int64_t K, int64_t mn0,
                                             int64_t k0, int tid)
{
    static_assert(NV == OpRegs<KMAJ, R, NT>::PER, "register count");
    if constexpr (RG && KMAJ) {
#pragma unroll
        for (int i = 0; i < OpRegs<KMAJ, R, NT>::PER; ++i) {
            const int idx = tid + i * NT;
            const int row = idx >> 3, c = idx & 7;
            const int64_t mn = mn0 + row, k = k0 + c * 8;
            v[i] = mn < MN && k < K ? load8_masked(p + mn * ld + k, K - k)
                                    : make_uint4(0, 0, 0, 0);
        }
    } else if constexpr (RG) {
#pragma unroll
        for (int b = 0; b < OpRegs<KMAJ, R, NT>::PER / 8; ++b) {
            const int idx = tid + b * NT;
            const int kb = idx / (R / 8), mb = idx % (R / 8);
            const int64_t mn = mn0 + mb * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t k = k0 + kb * 8 + j;
                v[b * 8 + j] = idx < R && mn < MN && k < K ? load8_masked(p + k * ld + mn, MN - mn)
                                                           : make_uint4(0, 0, 0, 0);
            }
        }
    } else if constexpr (KMAJ) {
        static_assert((R * 8) % NT == 0, "K-major tile must split evenly");
#pragma unroll
        for (int i = 0; i < OpRegs<KMAJ, R, NT>::PER; ++i) {
            const int idx = tid + i * NT;
            const int row = idx >> 3, c = idx & 7;
            const int64_t mn = mn0 + row, k = k0 + c * 8;
            // K is a multiple of 8 for K-major operands: a chunk is all in or all out.
            if (mn < MN && k < K)
                v[i] = *reinterpret_cast<const uint4 *>(p + mn * ld + k);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    } else {
        constexpr int NB = R;  // 8x8 blocks in a BK x R tile
#pragma unroll
        for (int b = 0; b < OpRegs<KMAJ, R, NT>::PER / 8; ++b) {
            const int idx = tid + b * NT;
            const int kb = idx / (R / 8), mb = idx % (R / 8);
            const int64_t mn = mn0 + mb * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t k = k0 + kb * 8 + j;
                // MN is a multiple of 8 for MN-major operands; K may be ragged.
                if (idx < NB && mn < MN && k < K)
                    v[b * 8 + j] = *reinterpret_cast<const uint4 *>(p + k * ld + mn);
                else
                    v[b * 8 + j] = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b)
{
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b)
{
    return (a >> 16) | (b & 0xffff0000u);
}
__device__ __forceinline__ uint32_t word(const uint4 &v, int w)
{
    return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Write one operand tile into LDS as R rows of eight swizzled 16-byte chunks.
template <bool KMAJ, int R, int NT, int NV>
__device__ __forceinline__ void store_operand(uint4 *__restrict__ S, const uint4 (&v)[NV], int tid)
{
    static_assert(NV == OpRegs<KMAJ, R, NT>::PER, "register count");
    if constexpr (KMAJ) {
#pragma unroll
        for (int i = 0; i < OpRegs<KMAJ, R, NT>::PER; ++i) {
            const int idx = tid + i * NT;
            const int row = idx >> 3, c = idx & 7;
            S[row * 8 + (c ^ (row & 7))] = v[i];
        }
    } else {
#pragma unroll
        for (int b = 0; b < OpRegs<KMAJ, R, NT>::PER / 8; ++b) {
            const int idx = tid + b * NT;
            if (idx >= R)
                continue;
            const int kb = idx / (R / 8), mb = idx % (R / 8);
            // v[b*8 + j] holds k = kb*8 + j, mn = mb*8 .. mb*8+7 (two per word).
            // Output q holds mn = mb*8 + q, k = kb*8 .. kb*8+7.
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int w = q >> 1;
                uint4 o;
                if ((q & 1) == 0) {
                    o.x = lo_halves(word(v[b * 8 + 0], w), word(v[b * 8 + 1], w));
                    o.y = lo_halves(word(v[b * 8 + 2], w), word(v[b * 8 + 3], w));
                    o.z = lo_halves(word(v[b * 8 + 4], w), word(v[b * 8 + 5], w));
                    o.w = lo_halves(word(v[b * 8 + 6], w), word(v[b * 8 + 7], w));
                } else {
                    o.x = hi_halves(word(v[b * 8 + 0], w), word(v[b * 8 + 1], w));
                    o.y = hi_halves(word(v[b * 8 + 2], w), word(v[b * 8 + 3], w));
                    o.z = hi_halves(word(v[b * 8 + 4], w), word(v[b * 8 + 5], w));
                    o.w = hi_halves(word(v[b * 8 + 6], w), word(v[b * 8 + 7], w));
                }
                const int row = mb * 8 + q;
                S[row * 8 + (kb ^ (row & 7))] = o;
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
struct Smem {
    static constexpr int NT = WM * WN * 64;
    static constexpr int OPS = 2 * (BM + BN) * BK * 2;  // double-buffered bf16 tiles
    static constexpr int CST = BN + 4;                   // epilogue row stride (floats)
    static constexpr int EPI = (BM / WM) * CST * 4;
    static constexpr int BYTES = OPS > EPI ? OPS : EPI;
};

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool ROWSQ, bool RG>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_kernel(GemmArgs g)
{
    using SM = Smem<BM, BN, WM, WN>;
    constexpr int NT = SM::NT;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int AV = OpRegs<AK, BM, NT>::PER;
    constexpr int BV = OpRegs<BKM, BN, NT>::PER;
    static_assert(!ROWSQ || AK, "row sums of squares need a K-major A");

    __shared__ __align__(16) unsigned char smem[SM::BYTES];
    uint4 *As = reinterpret_cast<uint4 *>(smem);  // [2][BM * 8]
    uint4 *Bs = As + 2 * BM * 8;                   // [2][BN * 8]

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
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

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float sq[ROWSQ ? AV : 1];
#pragma unroll
    for (int i = 0; i < (ROWSQ ? AV : 1); ++i)
        sq[i] = 0.f;

    uint4 ra[AV], rb[BV];

    auto load_step = [&](int64_t s) {
        const bool first = s < st1;
        const GemmSeg &sg = first ? g.seg[0] : g.seg[1];
        const int64_t k0 = (first ? s : s - st1) * BK;
        load_operand<AK, BM, NT, RG>(ra, static_cast<const uint16_t *>(sg.a), sg.lda, g.M, sg.K,
                                     m0, k0, tid);
        load_operand<BKM, BN, NT, RG>(rb, static_cast<const uint16_t *>(sg.b), sg.ldb, g.N, sg.K,
                                      n0, k0, tid);
    };
    auto store_step = [&](int buf) {
        if constexpr (ROWSQ) {
#pragma unroll
            for (int i = 0; i < AV; ++i) {
                const uint32_t w[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __uint_as_float(w[q] << 16);
                    const float hi = __uint_as_float(w[q] & 0xffff0000u);
                    sq[i] += lo * lo;
                    sq[i] += hi * hi;
                }
            }
        }
        store_operand<AK, BM, NT>(As + buf * BM * 8, ra, tid);
        store_operand<BKM, BN, NT>(Bs + buf * BN * 8, rb, tid);
    };
    auto compute = [&](int buf) {
        const uint4 *Ab = As + buf * BM * 8;
        const uint4 *Bb = Bs + buf * BN * 8;
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int chunk = kk * 4 + (lane >> 4);
            bf16x8_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + i * 16 + (lane & 15);
                af[i] = __builtin_bit_cast(bf16x8_t, Ab[row * 8 + (chunk ^ (row & 7))]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + j * 16 + (lane & 15);
                bfr[j] = __builtin_bit_cast(bf16x8_t, Bb[row * 8 + (chunk ^ (row & 7))]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                         0, 0, 0);
        }
    };

    if (s_begin < s_end) {
        load_step(s_begin);
        store_step(0);
        __syncthreads();
        for (int64_t s = s_begin; s < s_end; ++s) {
            const int cur = static_cast<int>((s - s_begin) & 1);
            const bool more = (s + 1) < s_end;
            if (more)
                load_step(s + 1);
            compute(cur);
            if (more)
                store_step(cur ^ 1);
            __syncthreads();
        }
    }

    if constexpr (ROWSQ) {
        if (g.rowsq != nullptr && tn == 0) {
#pragma unroll
            for (int i = 0; i < AV; ++i) {
                float v = sq[i];
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 4);
                const int row = (tid + i * NT) >> 3;
                const int64_t m = m0 + row;
                if ((tid & 7) == 0 && m < g.M)
                    g.rowsq[static_cast<int64_t>(z) * g.M + m] = v;
            }
        }
    }

    // Epilogue: one wave-row band (BM/WM rows) at a time through LDS.
    float *Cs = reinterpret_cast<float *>(smem);
#pragma unroll 1
    for (int h = 0; h < WM; ++h) {
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = i * 16 + (lane >> 4) * 4 + v;
                        const int col = wn * WTN + j * 16 + (lane & 15);
                        Cs[row * SM::CST + col] = acc[i][j][v];
                    }
        }
        __syncthreads();
        epilogue_rows<WTM, BN, SM::CST, NT, uint16_t>(Cs, g, m0 + h * WTM, n0, z, tn, tid);
        __syncthreads();
    }
}

// Tile configurations.  rel_speed scales the planner's per-CU MFMA rate for
// each tile shape: measured throughput of a full tile on the base product
// for the square ones, and, for 128 x 128 and the rank-wide tiles, the
// rate they reach as one wave of tiles on the rank-r products (x A^T,
// dh^T P, Q^T x at the training shape).
// The 128 x 128 register-staged configuration also exists with
// element-masked loads (ragged_ok), for operands of any width.
constexpr TileCfg kCfgs[] = {
    {256, 256, GEMM_BK, false, 0.76f, true, true, false, false, false},
    {256, 128, GEMM_BK, false, 0.68f, true, true, false, false, false},
    {128, 128, GEMM_BK, false, 0.56f, true, true, false, true, false},
    {128, 64, GEMM_BK, false, 0.40f, true, true, false, false, false},
    // 4 waves (2 x 2), 128 x 128 per wave
    {256, 256, GEMM_DMA_BK, true, 1.00f, true, false, false, false, false},
    {256, 128, GEMM_DMA_BK, true, 0.80f, true, false, false, false, false},  // 4 waves (2 x 2)
    // 4 waves (2 x 2), 2 per CU; row sums of squares and row dots from the
    // accumulators (the factored norm at small rank: N = r <= 128 fills the
    // tile, where the rank-384 tiles would stage and multiply zeros)
    {128, 128, GEMM_DMA_BK, true, 0.60f, true, true, true, false, false},
    // 4 waves (1 x 4): a whole rank-384 row block per tile, so the row-dot
    // products of the factored norm read W once, and products with N = r
    // (x A^T, dh B) read their long operand once
    {128, 384, GEMM_DMA_BK, true, 0.77f, true, true, true, false, false},
    // 4 waves (4 x 1): the same with M = r (Q^T x)
    {384, 128, GEMM_DMA_BK, true, 0.77f, true, false, false, false, false},
    // 8 waves (2 x 4, 64 x 96 per wave): the rank-384 row block with two
    // waves per SIMD, which hide each other's waits (measured on the
    // norm's row-dot products against the 4-wave tile: W A^T 231 -> 208 us,
    // B G 42 -> 28 us at d_out 28672, d_in 8192, r 384)
    {128, 384, GEMM_DMA_BK, true, 0.85f, true, true, true, false, true},
};

}  // namespace

namespace {

template <int BM, int BN, bool AK, bool BKM, bool RS, bool RG>
hipError_t launch_one(const GemmArgs &a, hipStream_t st)
{
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles == 0 || a.splits == 0)
        return hipSuccess;
    dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.splits));
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, 2, 2, AK, BKM, RS, RG>), grid, dim3(256), 0, st,
                       a);
    return hipGetLastError();
}

template <int BM, int BN, bool RG = false>
hipError_t launch_cfg(const GemmArgs &a, int layout, bool rowsq, hipStream_t st)
{
    switch (layout) {
    case 0:
        return rowsq ? launch_one<BM, BN, true, true, true, RG>(a, st)
                     : launch_one<BM, BN, true, true, false, RG>(a, st);
    case 1:
        return launch_one<BM, BN, true, false, false, RG>(a, st);
    case 2:
        return launch_one<BM, BN, false, false, false, RG>(a, st);
    default:
        return hipErrorInvalidValue;
    }
}

// Whether a product needs the element-masked loads: a leading dimension or
// base address that leaves rows unaligned to 16 bytes, a K-major operand
// whose K is not a multiple of 8, or an MN-major one whose M (or N) is not.
bool ragged_args(const GemmArgs &a, int layout)
{
    const bool ak = layout < 2, bk = layout == 0;
    for (int q = 0; q < a.nseg; ++q) {
        const GemmSeg &sg = a.seg[q];
        if ((sg.lda % 8) || (sg.ldb % 8) || (reinterpret_cast<uintptr_t>(sg.a) & 15) ||
            (reinterpret_cast<uintptr_t>(sg.b) & 15))
            return true;
        if ((ak && sg.K % 8) || (bk && sg.K % 8) || (!ak && a.M % 8) || (!bk && a.N % 8))
            return true;
    }
    return false;
}

}  // namespace

int gemm_bf16_num_cfgs()
{
    return static_cast<int>(sizeof(kCfgs) / sizeof(kCfgs[0]));
}

TileCfg gemm_bf16_cfg(int cfg)
{
    return kCfgs[cfg];
}

hipError_t launch_gemm_bf16(const GemmArgs &a, int layout, int cfg, bool rowsq, hipStream_t st)
{
    if (rowsq && layout != 0)
        return hipErrorInvalidValue;
    if (cfg < 0 || cfg >= gemm_bf16_num_cfgs() || (a.mode != EPI_ROWDOT && !kCfgs[cfg].store_ok) ||
        (rowsq && !kCfgs[cfg].rowsq_ok))
        return hipErrorInvalidValue;
    if (ragged_args(a, layout)) {
        // only the element-masked configuration takes unaligned operands
        if (!kCfgs[cfg].ragged_ok)
            return hipErrorInvalidValue;
        return launch_cfg<128, 128, true>(a, layout, rowsq, st);
    }
    switch (cfg) {
    case 0:
        return launch_cfg<256, 256>(a, layout, rowsq, st);
    case 1:
        return launch_cfg<256, 128>(a, layout, rowsq, st);
    case 2:
        return launch_cfg<128, 128>(a, layout, rowsq, st);
    case 3:
        return launch_cfg<128, 64>(a, layout, rowsq, st);
    case 4:
        return launch_dma_256x256(a, layout, rowsq, st);
    case 5:
        return launch_dma_256x128(a, layout, rowsq, st);
    case 6:
        return launch_dma_128x128(a, layout, rowsq, st);
    case 7:
        return launch_dma_128x384(a, layout, rowsq, st);
    case 8:
        return launch_dma_384x128(a, layout, rowsq, st);
    case 9:
        return launch_dma_128x384w8(a, layout, rowsq, st);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_bf16_dhdm(const GemmArgs &a, int cfg, hipStream_t st)
{
    if (cfg < 0 || cfg >= gemm_bf16_num_cfgs() || !kCfgs[cfg].dhdm_ok || a.nseg != 1 ||
        a.mode != EPI_STORE || ragged_args(a, 2) || !a.Y || !a.dh_out || !a.dm_part || !a.dh_m ||
        !a.dh_n || a.colm || a.coln)
        return hipErrorInvalidValue;
    switch (cfg) {
    case 9:
        return launch_dma_dhdm_128x384w8(a, st);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_bf16_grouped(GemmGroup &g, int layout, int cfg, bool rowsq, hipStream_t st)
{
    if (g.count < 1 || g.count > kMaxGroup || cfg < 0 || cfg >= gemm_bf16_num_cfgs() ||
        !kCfgs[cfg].dma || (rowsq && !kCfgs[cfg].rowsq_ok))
        return hipErrorInvalidValue;
    for (int p = 0; p < g.count; ++p)
        if ((g.p[p].mode != EPI_ROWDOT && !kCfgs[cfg].store_ok) || g.p[p].splits < 1)
            return hipErrorInvalidValue;
    switch (cfg) {
    case 4:
        return launch_dma_group_256x256(g, layout, rowsq, st);
    case 5:
        return launch_dma_group_256x128(g, layout, rowsq, st);
    case 6:
        return launch_dma_group_128x128(g, layout, rowsq, st);
    case 7:
        return launch_dma_group_128x384(g, layout, rowsq, st);
    case 8:
        return launch_dma_group_384x128(g, layout, rowsq, st);
    case 9:
        return launch_dma_group_128x384w8(g, layout, rowsq, st);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dora
