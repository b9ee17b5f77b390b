// gemm_bf16_dma.hpp - pipelined bf16 MFMA GEMM for K-major operands (gfx950).
//
// C[M, N] = sum_seg A_seg[M, K] B_seg[N, K]^T with both operands stored
// K-contiguous: the form of x W^T, x A^T, P B^T, W A^T and A A^T.
//
//   * v_mfma_f32_32x32x16_bf16: one wavefront keeps the matrix core busy
//     from only a few independent accumulators (the 16x16x32 shape needs
//     many more chains and several waves per SIMD to reach the same rate).
//   * Operand tiles move global -> LDS with direct-to-LDS buffer loads
//     (buffer_load_dwordx4 ... lds): no VGPR staging, asynchronous, landing in
//     LDS in lane order (lane l writes bytes [16 l, 16 l + 16) of a 1 KiB
//     block).  One wavefront load fills 16 tile rows of 64 bytes (32 bf16 K
//     values); each lane fetches the global 16-byte chunk that belongs at
//     its LDS position.
//   * STAGES steps of BK = 32 are resident: step s + STAGES - 1 is issued
//     right after the barrier of step s.
//   * Fragment prefetch: after the barrier of step s (which also makes step
//     s + 1 visible), each wave issues its LDS reads of step s + 1 and then
//     runs the MFMAs of step s from registers, so LDS latency hides behind
//     the matrix cores.  One barrier per step.
//   * Chunk c (8 K values) of tile row r sits at slot c ^ f(r), f(r) =
//     ((r >> 1) ^ (r >> 3 & 1)) & 3: the 16-byte fragment reads of 8 and of
//     16 consecutive lanes (consecutive rows) hit distinct banks.
//   * Rows beyond M or N load a clamped, valid row (their results are never
//     stored); K must be a multiple of BK (the host checks), so no zero fill.
//   * The epilogue is the shared LDS-staged one (epilogue.hpp).
#pragma once

#include "dora_internal.hpp"
#include "epilogue.hpp"

namespace dora {
namespace dma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 32;          // K values per step (64 bytes per tile row)
constexpr int ROW_BYTES = BK * 2;

// Depends on the low 4 bits of r only, so a 16-row DMA block (whose first row
// is a multiple of 16) can compute it from the row within the block.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r >> 3) & 1)) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) alone (LDS reads issued so far have returned).
__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Workgroup barrier without the release/acquire fences of __syncthreads(),
// which would wait for every outstanding direct-to-LDS load (vmcnt(0)) and
// so drain the pipeline.  Before it each wave waits (wait_vmcnt) for its own
// loads of the step about to be read; its LDS reads of older steps were
// consumed by MFMAs, hence complete.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES>
struct DmaCfg {
    static constexpr int NT = WM * WN * 64;
    static constexpr int NW = WM * WN;
    static constexpr int A_BYTES = BM * ROW_BYTES;
    static constexpr int B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int OPS = STAGES * STAGE_BYTES;
    static constexpr int CST = BN + 4;
    static constexpr int EPI = (BM / WM) * CST * 4;
    static constexpr int SMEM = OPS > EPI ? OPS : EPI;
    // 1 KiB (16-row) blocks per operand tile, and DMA instructions per wave
    static constexpr int A_BLK = BM / 16, B_BLK = BN / 16;
    static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "blocks must split over wavefronts");
    static constexpr int LPW = (A_BLK + B_BLK) / NW;
    static_assert(STAGES >= 3, "fragment prefetch needs at least 3 stages");
};

// Per-lane byte offsets of the DMA sources of one operand tile, relative to
// the (scalar) address of the step's first K value: computed once per tile,
// so a K step only advances one scalar base pointer.  Lane l of a 16-row
// block fetches row (l >> 2) of the block and the logical K chunk that
// belongs at its LDS slot (l & 3).  Rows past the matrix are clamped to the
// last row.  Offsets fit 32 bits: the host checks rows x ld x 2 < 4 GiB.
template <int NBLK, int NW>
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[NBLK / NW], int64_t rows, int64_t ld,
                                            int64_t r0, int wave, int lane)
{
    const int rloc = lane >> 2;
    const int chunk = (lane & 3) ^ swz(rloc);
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) {
        int64_t row = r0 + (i * NW + wave) * 16 + rloc;
        row = row < rows ? row : rows - 1;
        off[i] = static_cast<uint32_t>((row * ld + chunk * 8) * 2);
    }
}

// Buffer descriptor over one operand matrix (raw, byte-addressed; dword 3 =
// 0x00020000 selects plain linear addressing on gfx9-family parts).  Every
// access the kernel makes lies inside [base, base + bytes): rows are
// clamped and K stays below the segment's K.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void *base, int64_t bytes)
{
    const int nrec = bytes < 0x7fffffff ? static_cast<int>(bytes) : 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), nrec,
                                             0x00020000);
}

// Issue the direct-to-LDS loads of one operand tile of a K step:
// buffer_load_dwordx4 ... lds with the per-lane offset in a VGPR and the K
// offset of the step as the scalar offset, so a load needs no address math.
// The offset is picked per load from the two segments' tables (a select, not
// a pointer to either table, which would put them in scratch).
template <int NBLK, int NW>
__device__ __forceinline__ void dma_issue(unsigned char *dst, __amdgpu_buffer_rsrc_t rsrc,
                                          uint32_t koff, bool first,
                                          const uint32_t (&off0)[NBLK / NW],
                                          const uint32_t (&off1)[NBLK / NW], int wave)
{
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) {
        const uint32_t o = first ? off0[i] : off1[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_void *)(dst + (i * NW + wave) * 1024), 16, o, koff, 0, 0);
    }
}

// One step's MFMA operands of a wave: two 16-wide K halves, TM A and TN B
// 32-row fragments each (lane: row lane & 31, K chunk 2 kk + lane >> 5).
template <int TM, int TN>
struct Frags {
    bf16x8_t a[2][TM], b[2][TN];
};

template <int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void read_frags(Frags<TM, TN> &f, const unsigned char *As,
                                           const unsigned char *Bs, int wm, int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int fc = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + (lane & 31);
            f.a[kk][i] = *reinterpret_cast<const bf16x8_t *>(As + row * ROW_BYTES +
                                                             ((fc ^ swz(row)) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WTN + j * 32 + (lane & 31);
            f.b[kk][j] = *reinterpret_cast<const bf16x8_t *>(Bs + row * ROW_BYTES +
                                                             ((fc ^ swz(row)) << 4));
        }
    }
}

template <int TM, int TN>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[TM][TN], const Frags<TM, TN> &f)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j],
                                                                     acc[i][j], 0, 0, 0);
}

template <int BM, int BN, int WM, int WN, int STAGES, bool ROWSQ>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_dma_kernel(GemmArgs g)
{
    using C = DmaCfg<BM, BN, WM, WN, STAGES>;
    constexpr int NT = C::NT;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold 32x32 MFMA tiles");
    static_assert(!ROWSQ || BM <= NT, "one A row per thread for the row sums of squares");

    __shared__ __align__(1024) unsigned char smem[C::SMEM];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    // wave index as a scalar: LDS destinations of the DMA are then SGPR values
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_coords(g.M, g.N, BM, BN, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
    const int z = static_cast<int>(blockIdx.y);

    const int64_t st1 = g.seg[0].K / BK;
    const int64_t st_total = st1 + (g.nseg > 1 ? g.seg[1].K / BK : 0);
    int64_t s_begin = static_cast<int64_t>(z) * g.steps_per_split;
    if (s_begin > st_total)
        s_begin = st_total;
    int64_t s_end = s_begin + g.steps_per_split;
    if (s_end > st_total)
        s_end = st_total;

    constexpr int AP = C::A_BLK / C::NW, BP = C::B_BLK / C::NW;
    uint32_t offa0[AP], offb0[BP], offa1[AP] = {}, offb1[BP] = {};
    dma_offsets<C::A_BLK, C::NW>(offa0, g.M, g.seg[0].lda, m0, wave, lane);
    dma_offsets<C::B_BLK, C::NW>(offb0, g.N, g.seg[0].ldb, n0, wave, lane);
    if (g.nseg > 1) {
        dma_offsets<C::A_BLK, C::NW>(offa1, g.M, g.seg[1].lda, m0, wave, lane);
        dma_offsets<C::B_BLK, C::NW>(offb1, g.N, g.seg[1].ldb, n0, wave, lane);
    }

    auto stage_ptr = [&](int64_t s) {
        return smem + static_cast<int>((s - s_begin) % STAGES) * C::STAGE_BYTES;
    };
    const __amdgpu_buffer_rsrc_t ra0 = operand_rsrc(g.seg[0].a, g.M * g.seg[0].lda * 2);
    const __amdgpu_buffer_rsrc_t rb0 = operand_rsrc(g.seg[0].b, g.N * g.seg[0].ldb * 2);
    const __amdgpu_buffer_rsrc_t ra1 =
        g.nseg > 1 ? operand_rsrc(g.seg[1].a, g.M * g.seg[1].lda * 2) : ra0;
    const __amdgpu_buffer_rsrc_t rb1 =
        g.nseg > 1 ? operand_rsrc(g.seg[1].b, g.N * g.seg[1].ldb * 2) : rb0;
    auto issue = [&](int64_t s) {
        unsigned char *st = stage_ptr(s);
        const bool first = s < st1;
        const uint32_t koff = static_cast<uint32_t>((first ? s : s - st1) * BK * 2);
        dma_issue<C::A_BLK, C::NW>(st, first ? ra0 : ra1, koff, first, offa0, offa1, wave);
        dma_issue<C::B_BLK, C::NW>(st + C::A_BYTES, first ? rb0 : rb1, koff, first, offb0, offb1,
                                   wave);
    };
    // Wait until this wave's loads of step t have landed, given that at most
    // `later` further steps (and none past s_end - 1) have been issued.
    auto wait_step = [&](int64_t t, int later) {
        const int64_t pend = (s_end - 1 - t) < later ? (s_end - 1 - t) : later;
        if (pend >= 2)
            wait_vmcnt<2 * C::LPW>();
        else if (pend == 1)
            wait_vmcnt<C::LPW>();
        else
            wait_vmcnt<0>();
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.f;
    float sq = 0.f;  // ROWSQ: the row of A owned by this thread (tid < BM)
    auto rowsq_step = [&](const unsigned char *As) {
        if (tn == 0 && tid < BM) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 v = *reinterpret_cast<const uint4 *>(As + tid * ROW_BYTES +
                                                                 ((c ^ swz(tid)) << 4));
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __uint_as_float(w[q] << 16);
                    const float hi = __uint_as_float(w[q] & 0xffff0000u);
                    sq += lo * lo;
                    sq += hi * hi;
                }
            }
        }
    };

    // prologue: STAGES-1 steps in flight, then step s_begin visible and read
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
        if (s_begin + p < s_end)
            issue(s_begin + p);

    Frags<TM, TN> fa, fb;
    if (s_begin < s_end) {
        wait_step(s_begin, STAGES - 2);
        stage_barrier();
        read_frags<TM, TN, WTM, WTN>(fa, stage_ptr(s_begin), stage_ptr(s_begin) + C::A_BYTES, wm,
                                     wn, lane);
    }
    // step s: the fragments of s are in `cur`; make s + 1 visible, refill the
    // ring, read s + 1 into `nxt`, run the MFMAs of s.
    auto body = [&](int64_t s, Frags<TM, TN> &cur, Frags<TM, TN> &nxt) {
        const bool more = s + 1 < s_end;
        // the reads of `cur` were issued a whole MFMA phase ago: retire them
        // here, so that no wait lands between the reads of `nxt` and the MFMAs
        wait_lgkm0();
        if (more)
            wait_step(s + 1, STAGES - 3);
        stage_barrier();
        if (s + STAGES - 1 < s_end)
            issue(s + STAGES - 1);
        if constexpr (ROWSQ)
            rowsq_step(stage_ptr(s));
        if (more)
            read_frags<TM, TN, WTM, WTN>(nxt, stage_ptr(s + 1), stage_ptr(s + 1) + C::A_BYTES, wm,
                                         wn, lane);
        mfma_step<TM, TN>(acc, cur);
    };
    int64_t s = s_begin;
    for (; s + 1 < s_end; s += 2) {
        body(s, fa, fb);
        body(s + 1, fb, fa);
    }
    if (s < s_end)
        body(s, fa, fb);
    stage_barrier();  // every wave is done reading the stages before LDS is reused

    if constexpr (ROWSQ) {
        if (g.rowsq != nullptr && tn == 0 && tid < BM && m0 + tid < g.M)
            g.rowsq[static_cast<int64_t>(z) * g.M + m0 + tid] = sq;
    }

    float *Cs = reinterpret_cast<float *>(smem);
#pragma unroll 1
    for (int h = 0; h < WM; ++h) {
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        // 32x32 accumulator: row 8 (v >> 2) + 4 (lane >> 5) + (v & 3),
                        // column lane & 31
                        const int row = i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                        const int col = wn * WTN + j * 32 + (lane & 31);
                        Cs[row * C::CST + col] = acc[i][j][v];
                    }
        }
        __syncthreads();
        epilogue_rows<WTM, BN, C::CST, NT, uint16_t>(Cs, g, m0 + h * WTM, n0, z, tn, tid);
        __syncthreads();
    }
}

}  // namespace dma
}  // namespace dora
