// epilogue.hpp - GEMM epilogues shared by the bf16 MFMA and fp32 VALU GEMMs.
//
// After the K loop a workgroup stages R rows of its fp32 accumulator tile in
// LDS (Cs, row stride CST floats) and calls epilogue_rows, which either
// stores alpha*C (rounded once to bf16, or fp32) with 16-byte coalesced
// writes, or reduces each row of C (.) E to one partial dot product.  The
// row-dot mode is how the factored norm's cross term (rows of B against
// U = W A^T) and Gram term (rows of B against B G) are formed without U or
// B G ever reaching HBM.
#pragma once

#include "dora_internal.hpp"

namespace dora {

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN): gfx950
// converts in hardware, two values per v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2_cvt_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Eight consecutive elements of E (a row of the row-dot operand), held raw
// until used (bf16: one 16-byte register quad); columns past `cnt` read as
// zero.
template <typename TE>
struct EChunk;
template <>
struct EChunk<uint16_t> {
    uint4 raw;
    __device__ __forceinline__ void load(const uint16_t *p, int cnt)
    {
        if (cnt == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
            raw = *reinterpret_cast<const uint4 *>(p);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = 2 * q < cnt ? p[2 * q] : 0u;
                const uint32_t hi = 2 * q + 1 < cnt ? p[2 * q + 1] : 0u;
                w[q] = lo | (hi << 16);
            }
            raw = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    __device__ __forceinline__ void zero() { raw = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ float get(int q) const
    {
        const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        const uint32_t u = words[q >> 1];
        return __uint_as_float((q & 1) ? (u & 0xffff0000u) : (u << 16));
    }
};
template <>
struct EChunk<float> {
    float v[8];
    __device__ __forceinline__ void load(const float *p, int cnt)
    {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = q < cnt ? p[q] : 0.f;
    }
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = 0.f;
    }
    __device__ __forceinline__ float get(int q) const { return v[q]; }
};

// Store up to 8 consecutive elements v[0 .. cnt) of a row at o, rounded once
// to the element type: one or two 16-byte stores when all 8 are live and o
// is 16-byte aligned (rows of a ragged width need not be), else element by
// element.
__device__ __forceinline__ void store_row8(uint16_t *o, const float (&v)[8], int cnt)
{
    if (cnt == 8 && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
        *reinterpret_cast<uint4 *>(o) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
        for (int q = 0; q < cnt; ++q)
            o[q] = f32_to_bf16(v[q]);
    }
}
__device__ __forceinline__ void store_row8(float *o, const float (&v)[8], int cnt)
{
    if (cnt == 8 && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
        reinterpret_cast<float4 *>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4 *>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        for (int q = 0; q < cnt; ++q)
            o[q] = v[q];
    }
}

// Process rows [mrow0, mrow0 + R) of the tile whose first column is n0.
// Every thread of the workgroup must call this (row-dot uses wave shuffles).
// Thread tid always handles the 8-column chunk tid % (BN / 8), on rows
// tid / (BN / 8) + k * NT / (BN / 8): per-column factors are loaded once, and
// all row-dot operands are loaded before any is used, so their latencies
// overlap.
//
// EPI_MERGE with `pre` set: the thread's ITER chunks of E were loaded before
// (merge_chunk_load, same rows and columns), so no load waits here.
template <int R, int BN, int CST, int NT, typename TE>
__device__ __forceinline__ void epilogue_rows(const float *Cs, const GemmArgs &g, int64_t mrow0,
                                              int64_t n0, int z, int tn, int tid,
                                              const EChunk<TE> *pre = nullptr)
{
    constexpr int CPR = BN / 8;  // 8-column chunks per row
    static_assert(BN % 8 == 0 && 64 % CPR == 0, "row chunks must tile a wavefront");
    static_assert((R * CPR) % NT == 0, "every thread takes the same number of chunks");
    constexpr int ITER = R * CPR / NT;  // chunks per thread
    constexpr int RSTEP = NT / CPR;     // rows between a thread's chunks
    const int64_t M = g.M, N = g.N;
    const int c = tid % CPR, row0 = tid / CPR;
    const int64_t n = n0 + c * 8;
    const int cnt = n >= N ? 0 : ((N - n) < 8 ? static_cast<int>(N - n) : 8);

    if (g.mode == EPI_STORE) {
        // y = h + (g - 1) h with g - 1 = (m - n) / n formed in fp32
        float gm1[8];
        const bool scale = g.colm != nullptr;
        if (scale) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float mi = q < cnt ? g.colm[n + q] : 1.f;
                const float ni = q < cnt ? g.coln[n + q] : 1.f;
                gm1[q] = (mi - ni) / ni;
            }
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int row = row0 + it * RSTEP;
            const int64_t m = mrow0 + row;
            if (m >= M || cnt == 0)
                continue;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                v[q] = g.alpha * Cs[row * CST + c * 8 + q];
                if (scale)
                    v[q] = __fmaf_rn(gm1[q], v[q], v[q]);
            }
            if (g.out_f32) {
                float *o = static_cast<float *>(g.out) + static_cast<int64_t>(z) * M * g.ldc +
                           m * g.ldc + n;
                if (g.out_accum) {
                    for (int q = 0; q < cnt; ++q)
                        o[q] += v[q];
                } else {
                    store_row8(o, v, cnt);
                }
            } else {
                store_row8(static_cast<TE *>(g.out) + m * g.ldc + n, v, cnt);
            }
            if (g.out2 != nullptr) {
                // the second output: alpha2 * C rounded once, or the residual
                // of the first output's rounding
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    v[q] = g.out2_lo ? v[q] - bf16_to_f32(f32_to_bf16(v[q]))
                                     : g.alpha2 * Cs[row * CST + c * 8 + q];
                if (g.out_f32)
                    store_row8(static_cast<float *>(g.out2) + m * g.ldc + n, v, cnt);
                else
                    store_row8(static_cast<TE *>(g.out2) + m * g.ldc + n, v, cnt);
            }
        }
    } else if (g.mode == EPI_MERGE) {
        // W' = W + ((g - 1) W + g s C) by rows, g = m / n, rounded once; all
        // operands of the thread's chunks are loaded before any is stored
        // (W' may be W itself: each element is read, then written, by the
        // same thread)
        const TE *E = static_cast<const TE *>(g.E);
        EChunk<TE> e[ITER];
        float gm1[ITER], gs[ITER];
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int64_t m = mrow0 + row0 + it * RSTEP;
            const bool live = m < M && cnt > 0;
            if (pre != nullptr)
                e[it] = pre[it];
            else if (live)
                e[it].load(E + m * g.lde + n, cnt);
            else
                e[it].zero();
            const float mi = live ? g.colm[m] : 1.f;
            const float ni = live ? g.coln[m] : 1.f;
            gm1[it] = (mi - ni) / ni;
            gs[it] = (mi / ni) * g.alpha;
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int row = row0 + it * RSTEP;
            const int64_t m = mrow0 + row;
            if (m >= M || cnt == 0)
                continue;
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float w = e[it].get(q);
                v[q] = w + __fmaf_rn(gm1[it], w, gs[it] * Cs[row * CST + c * 8 + q]);
            }
            store_row8(static_cast<TE *>(g.out) + m * g.ldc + n, v, cnt);
        }
    } else {  // EPI_ROWDOT
        const int ntn = static_cast<int>((N + BN - 1) / BN);
        const TE *E = static_cast<const TE *>(g.E);
        EChunk<TE> e[ITER];
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int64_t m = mrow0 + row0 + it * RSTEP;
            if (m < M && cnt > 0)
                e[it].load(E + m * g.lde + n, cnt);
            else
                e[it].zero();
        }
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int row = row0 + it * RSTEP;
            const int64_t m = mrow0 + row;
            if (g.out != nullptr && m < M) {
                // the product itself as well (fp32, split z at out + z M ldc;
                // with out_accum, alpha times it added to what out holds)
                float *o = static_cast<float *>(g.out) + static_cast<int64_t>(z) * M * g.ldc +
                           m * g.ldc + n;
                for (int q = 0; q < cnt; ++q)
                    o[q] = g.out_accum ? o[q] + g.alpha * Cs[row * CST + c * 8 + q]
                                       : Cs[row * CST + c * 8 + q];
            }
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                sum += q < cnt ? Cs[row * CST + c * 8 + q] * e[it].get(q) : 0.f;
#pragma unroll
            for (int off = CPR / 2; off >= 1; off >>= 1)
                sum += __shfl_xor(sum, off);
            if (c == 0 && m < M)
                g.rowdot[(static_cast<int64_t>(z) * ntn + tn) * M + m] = sum;
        }
    }
}

// The E chunks epilogue_rows<R, BN, CST, NT> takes for thread tid on rows
// [mrow0, mrow0 + R) from column n0 (EPI_MERGE: W's tile, loaded early).
template <int R, int BN, int NT, typename TE>
__device__ __forceinline__ void merge_chunk_load(EChunk<TE> *e, const GemmArgs &g, int64_t mrow0,
                                                 int64_t n0, int tid)
{
    constexpr int CPR = BN / 8, ITER = R * CPR / NT, RSTEP = NT / CPR;
    const int c = tid % CPR, row0 = tid / CPR;
    const int64_t n = n0 + c * 8;
    const int cnt = n >= g.N ? 0 : ((g.N - n) < 8 ? static_cast<int>(g.N - n) : 8);
    const TE *E = static_cast<const TE *>(g.E);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int64_t m = mrow0 + row0 + it * RSTEP;
        if (m < g.M && cnt > 0)
            e[it].load(E + m * g.lde + n, cnt);
        else
            e[it].zero();
    }
}

// Map the linear workgroup id to a (tile row, tile column).  Consecutive
// hardware workgroup ids go to the 8 XCDs in turn; each XCD is given a
// contiguous run of logical tiles, and logical tiles are ordered in groups
// of 8 tile rows so that the workgroups resident on one XCD at a time share
// A rows and B columns in that XCD's L2.
__device__ __forceinline__ int xcd_linear_id()
{
    const int nb = static_cast<int>(gridDim.x);
    const int b = static_cast<int>(blockIdx.x);
    const int q = nb >> 3, rem = nb & 7;
    const int xcd = b & 7, local = b >> 3;
    return (xcd < rem) ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

// Tile L of an M x N product in groups of 8 tile rows.
__device__ __forceinline__ void tile_in_order(int L, int64_t M, int64_t N, int BM, int BN, int &tm,
                                              int &tn)
{
    const int num_m = static_cast<int>((M + BM - 1) / BM);
    const int num_n = static_cast<int>((N + BN - 1) / BN);
    constexpr int GROUP = 8;
    const int per_group = GROUP * num_n;
    const int group = L / per_group;
    const int first_m = group * GROUP;
    const int gsz = (num_m - first_m) < GROUP ? (num_m - first_m) : GROUP;
    const int in_g = L - group * per_group;
    tm = first_m + in_g % gsz;
    tn = in_g / gsz;
}

__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int BM, int BN, int &tm, int &tn)
{
    tile_in_order(xcd_linear_id(), M, N, BM, BN, tm, tn);
}

// Grouped launch: problem p, its tile (tm, tn) and split z of this workgroup
// (the XCD-aware linear order runs through the problems in turn).
__device__ __forceinline__ void group_coords(const GemmGroup &grp, int BM, int BN, int &p, int &tm,
                                             int &tn, int &z)
{
    const int L = grp.spread ? static_cast<int>(blockIdx.x) : xcd_linear_id();
    p = 0;
    while (p + 1 < grp.count && L >= grp.tile_start[p + 1])
        ++p;
    const int64_t M = grp.p[p].M, N = grp.p[p].N;
    const int tiles = static_cast<int>(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
    const int local = L - grp.tile_start[p];
    z = local / tiles;
    tile_in_order(local - z * tiles, M, N, BM, BN, tm, tn);
}

}  // namespace dora
