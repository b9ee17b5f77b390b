// gemm_bf16_dma.hpp - pipelined bf16 MFMA GEMM (gfx950).
//
// C[M, N] = sum_seg op(A_seg) op(B_seg), each operand either K-major (K
// contiguous: x, W and A in x W^T, W A^T, A A^T, dh in dh B) or MN-major (M
// or N contiguous: W and A in dh W, dh and P in dh^T P, Q and x in Q^T x).
//
//   * v_mfma_f32_32x32x16_bf16: one wavefront keeps the matrix core busy
//     from only a few independent accumulators (the 16x16x32 shape needs
//     many more chains and several waves per SIMD to reach the same rate).
//   * Operand tiles move global -> LDS with direct-to-LDS buffer loads
//     (buffer_load_dwordx4 ... lds): no VGPR staging, asynchronous, landing
//     in LDS in lane order (lane l writes bytes [16 l, 16 l + 16) of a 1 KiB
//     block); each lane fetches the global 16-byte chunk that belongs at its
//     LDS position.
//   * K-major tiles are rows of 32 K values (64 bytes), chunk c of row r at
//     slot c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3 & 1)) & 3; fragments are read
//     with ds_read_b128 (8 and 16 consecutive rows hit distinct banks).
//   * MN-major tiles are 32 rows (one per K value) of R M or N values; the
//     16-byte chunk c of row k sits at c ^ t(k), t(k) = {0, 6, 10, 12}[k & 3].
//     Fragments are read with two ds_read_b64_tr_b16: within each group of
//     16 lanes, lane j reads 4 consecutive values of row k0 + j / 4 at column
//     c0 + 4 (j % 4), and lane i receives column c0 + i of rows k0 .. k0 + 3,
//     exactly half of an MFMA fragment.  t keeps the 4 rows x 32 bytes of a
//     16-lane group (and the 4 rows x 64 bytes of two groups) on distinct
//     banks.  K rows past the end fall outside the buffer range and load as
//     zeros, so K need not be a multiple of 32 for MN-major operands.
//   * STAGES steps of BK = 32 are resident: step s + STAGES - 1 is issued
//     right after the barrier of step s.  After that barrier (which also
//     makes step s + 1 visible) each wave reads its fragments of step s + 1
//     and then runs the MFMAs of step s from registers.  One barrier per step.
//   * Rows / columns past M or N load clamped, valid data (never stored); the
//     host checks K % 32 for K-major operands and that every operand is under
//     2 GiB (32-bit buffer offsets).
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

// Chunk swizzle of MN-major tiles: t(k) = {0, 6, 10, 12}[k & 3].
__device__ __forceinline__ int swz_mn(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }

// Buffer descriptor over one operand matrix (raw, byte-addressed; dword 3 =
// 0x00020000 selects plain linear addressing on gfx9-family parts).  Loads
// at offsets >= `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void *base, int64_t bytes)
{
    const int nrec = bytes < 0x7fffffff ? static_cast<int>(bytes) : 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), nrec,
                                             0x00020000);
}

// One direct-to-LDS load: lane l's 16 bytes at rsrc + voff + soff land at LDS
// byte lds + 16 l.  Issued from inline asm (no register outputs; it clobbers
// m0 and memory) rather than the builtin: the compiler treats the builtin as
// an LDS store and then drains every such load (vmcnt(0)) before any
// transpose read it cannot prove disjoint, which would empty the pipeline
// each step.  Completion is covered by the kernel's explicit vmcnt waits and
// barriers.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, uint32_t voff,
                                          uint32_t soff)
{
    __asm__ volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :
                     : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
                     : "memory", "m0");
}

// One operand's DMA plan: per-lane byte offsets of the sources of the
// wave's load instructions, computed once per tile.
//   K-major (rows = M or N, ld over K): instruction i fills 16 tile rows;
//   lane l fetches row l >> 2 of the block and the K chunk that belongs at
//   slot l & 3.  A step adds its K offset as the scalar buffer offset.
//   MN-major (rows = K, ld over M or N): instruction i fills 1 KiB of the
//   [32][R] tile; lane l fetches the chunk that belongs at byte 16 l.  A step
//   adds k0 * ld * 2 to the per-lane offset (rows past K are out of range
//   and load as zeros).
template <bool KMAJ, int R, int NW>
struct OperandDma {
    static constexpr int NINST = R / 16;  // 1 KiB load instructions per tile
    static_assert(NINST % NW == 0, "tile loads must split over wavefronts");
    static constexpr int PER = NINST / NW;
    static constexpr int PITCH = R * 2;   // MN-major row bytes
    static_assert(KMAJ || R >= 128, "MN-major tiles need >= 16 chunks per row");
    uint32_t off[PER];

    __device__ __forceinline__ void init(int64_t mn_extent, int64_t ld, int64_t mn0, int wave,
                                         int lane)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = i * NW + wave;
            if constexpr (KMAJ) {
                const int rloc = lane >> 2;
                const int chunk = (lane & 3) ^ swz(rloc);
                int64_t row = mn0 + blk * 16 + rloc;
                row = row < mn_extent ? row : mn_extent - 1;
                off[i] = static_cast<uint32_t>((row * ld + chunk * 8) * 2);
            } else {
                const int b = blk * 1024 + lane * 16;
                const int krow = b / PITCH;
                const int chunk = ((b % PITCH) >> 4) ^ swz_mn(krow);
                int64_t col = mn0 + chunk * 8;
                col = col + 8 <= mn_extent ? col : mn_extent - 8;
                off[i] = static_cast<uint32_t>((krow * ld + col) * 2);
            }
        }
    }

    // Issue the tile's loads of the step whose first K index is k0.
    __device__ __forceinline__ void issue(unsigned char *dst, __amdgpu_buffer_rsrc_t rsrc,
                                          int64_t k0, int64_t ld, int wave) const
    {
        const uint32_t kadd = static_cast<uint32_t>(KMAJ ? k0 * 2 : k0 * ld * 2);
        const uint32_t base = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((lds_void *)(dst + wave * 1024)));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const uint32_t lds = __builtin_amdgcn_readfirstlane(base + i * NW * 1024);
            if constexpr (KMAJ)
                lds_dma16(rsrc, lds, off[i], kadd);
            else
                lds_dma16(rsrc, lds, off[i] + kadd, 0u);
        }
    }
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// The MFMA fragment of 32 M (or N) indices starting at `mn` and the 8 K
// values 16 kk + 8 (lane >> 5) + 0..7 of a step: lane holds index
// mn + (lane & 31).
template <bool KMAJ, int R>
__device__ __forceinline__ bf16x8_t read_frag(const unsigned char *tile, int mn, int kk, int lane)
{
    if constexpr (KMAJ) {
        const int row = mn + (lane & 31);
        const int fc = kk * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8_t *>(tile + row * ROW_BYTES + ((fc ^ swz(row)) << 4));
    } else {
        constexpr int PITCH = R * 2;
        const int grp = lane >> 4, j = lane & 15;
        const int col = mn + 16 * (grp & 1) + 4 * (j & 3);
        const int k = kk * 16 + 8 * (grp >> 1) + (j >> 2);
        const int k2 = k + 4;
        const unsigned char *p0 =
            tile + k * PITCH + (((col >> 3) ^ swz_mn(k)) << 4) + ((col & 7) << 1);
        const unsigned char *p1 =
            tile + k2 * PITCH + (((col >> 3) ^ swz_mn(k2)) << 4) + ((col & 7) << 1);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
        const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, v);
    }
}

// One step's MFMA operands of a wave: two 16-wide K halves, TM A and TN B
// 32-index fragments each.
template <int TM, int TN>
struct Frags {
    bf16x8_t a[2][TM], b[2][TN];
};

template <bool AK, bool BKM, int BM, int BN, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void read_frags(Frags<TM, TN> &f, const unsigned char *As,
                                           const unsigned char *Bs, int wm, int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            f.a[kk][i] = read_frag<AK, BM>(As, wm * WTM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            f.b[kk][j] = read_frag<BKM, BN>(Bs, wn * WTN + j * 32, kk, lane);
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

template <int BM, int BN, int WM, int WN, int STAGES, bool AK, bool BKM, bool ROWSQ>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_dma_kernel(GemmArgs g)
{
    using C = DmaCfg<BM, BN, WM, WN, STAGES>;
    using DA = OperandDma<AK, BM, WM * WN>;
    using DB = OperandDma<BKM, BN, WM * WN>;
    constexpr int NT = C::NT;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold 32x32 MFMA tiles");
    static_assert(!ROWSQ || (AK && BM <= NT), "row sums of squares: K-major A, one row per thread");
    static_assert(DA::PER + DB::PER == C::LPW, "load count");

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

    const int64_t st1 = (g.seg[0].K + BK - 1) / BK;
    const int64_t st_total = st1 + (g.nseg > 1 ? (g.seg[1].K + BK - 1) / BK : 0);
    int64_t s_begin = static_cast<int64_t>(z) * g.steps_per_split;
    if (s_begin > st_total)
        s_begin = st_total;
    int64_t s_end = s_begin + g.steps_per_split;
    if (s_end > st_total)
        s_end = st_total;

    // per-segment load plans and buffer descriptors (a K-major operand spans
    // its M or N rows, an MN-major one its K rows)
    DA da0, da1;
    DB db0, db1;
    da0.init(g.M, g.seg[0].lda, m0, wave, lane);
    db0.init(g.N, g.seg[0].ldb, n0, wave, lane);
    const __amdgpu_buffer_rsrc_t ra0 =
        operand_rsrc(g.seg[0].a, (AK ? g.M : g.seg[0].K) * g.seg[0].lda * 2);
    const __amdgpu_buffer_rsrc_t rb0 =
        operand_rsrc(g.seg[0].b, (BKM ? g.N : g.seg[0].K) * g.seg[0].ldb * 2);
    __amdgpu_buffer_rsrc_t ra1 = ra0, rb1 = rb0;
    if (g.nseg > 1) {
        da1.init(g.M, g.seg[1].lda, m0, wave, lane);
        db1.init(g.N, g.seg[1].ldb, n0, wave, lane);
        ra1 = operand_rsrc(g.seg[1].a, (AK ? g.M : g.seg[1].K) * g.seg[1].lda * 2);
        rb1 = operand_rsrc(g.seg[1].b, (BKM ? g.N : g.seg[1].K) * g.seg[1].ldb * 2);
    } else {
        da1 = da0;
        db1 = db0;
    }

    auto stage_ptr = [&](int64_t s) {
        return smem + static_cast<int>((s - s_begin) % STAGES) * C::STAGE_BYTES;
    };
    auto issue = [&](int64_t s) {
        unsigned char *st = stage_ptr(s);
        if (s < st1) {
            da0.issue(st, ra0, s * BK, g.seg[0].lda, wave);
            db0.issue(st + C::A_BYTES, rb0, s * BK, g.seg[0].ldb, wave);
        } else {
            da1.issue(st, ra1, (s - st1) * BK, g.seg[1].lda, wave);
            db1.issue(st + C::A_BYTES, rb1, (s - st1) * BK, g.seg[1].ldb, wave);
        }
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
    float sq[4] = {0.f, 0.f, 0.f, 0.f};  // ROWSQ: the row of A owned by this thread
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
                    sq[q] = __fmaf_rn(lo, lo, sq[q]);
                    sq[q] = __fmaf_rn(hi, hi, sq[q]);
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
        read_frags<AK, BKM, BM, BN, TM, TN, WTM, WTN>(fa, stage_ptr(s_begin),
                                                      stage_ptr(s_begin) + C::A_BYTES, wm, wn,
                                                      lane);
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
            read_frags<AK, BKM, BM, BN, TM, TN, WTM, WTN>(nxt, stage_ptr(s + 1),
                                                          stage_ptr(s + 1) + C::A_BYTES, wm, wn,
                                                          lane);
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
            g.rowsq[static_cast<int64_t>(z) * g.M + m0 + tid] = (sq[0] + sq[1]) + (sq[2] + sq[3]);
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
