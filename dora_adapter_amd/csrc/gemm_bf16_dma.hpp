// gemm_bf16_dma.hpp - pipelined bf16 MFMA GEMM (gfx950).
//
// C[M, N] = sum_seg op(A_seg) op(B_seg), each operand either K-major (K
// contiguous: x, W and A in x W^T, W A^T, A A^T, dh in dh B) or MN-major (M
// or N contiguous: W and A in dh W, dh and P in dh^T P, Q and x in Q^T x).
//
//   * v_mfma_f32_32x32x16_bf16: one wavefront keeps the matrix core busy
//     from a few independent accumulators, so a workgroup of four waves
//     (one per SIMD) can hold a 128 x 128 wave tile in accumulation
//     registers, which halves LDS fragment traffic per flop against eight
//     waves of 128 x 64.
//   * Operand tiles move global -> LDS with direct-to-LDS buffer loads
//     (buffer_load_dwordx4 ... lds): no VGPR staging, asynchronous, landing
//     in LDS in lane order (lane l writes bytes [16 l, 16 l + 16) of a 1 KiB
//     block); each lane fetches the global 16-byte chunk that belongs at its
//     LDS position.
//   * A stage holds BK = 64 K values.  K-major tile rows are then 128 bytes,
//     one full L2 line per row and load (32-wide rows would issue twice as
//     many 64-byte requests for the same bytes).  Chunk c of row r sits at
//     slot c ^ g(r), g(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7, so that the 16
//     rows of a 16-lane ds_read_b128 phase, and any 8 consecutive rows, hit
//     distinct banks.
//   * MN-major tiles are 64 rows (one per K value) of R M or N values; the
//     16-byte chunk c of row k sits at c ^ t(k), t(k) = {0, 6, 10, 12}[k & 3].
//     Fragments are read with two ds_read_b64_tr_b16: within each group of
//     16 lanes, lane j reads 4 consecutive values of row k0 + j / 4 at column
//     c0 + 4 (j % 4), and lane i receives column c0 + i of rows k0 .. k0 + 3,
//     exactly half of an MFMA fragment.  t keeps the 4 rows x 32 bytes of a
//     16-lane group (and the 4 rows x 64 bytes of two groups) on distinct
//     banks.
//   * K past the end of a segment loads as zeros: an MN-major operand's rows
//     past K fall outside its buffer range; a K-major lane whose chunk lies
//     past K is given an out-of-range offset.  Rows / columns past M or N
//     load clamped, valid data (never stored).  The host checks that every
//     operand is under 2 GiB (32-bit buffer offsets) and that K-major K is a
//     multiple of 8 (whole 16-byte chunks).
//   * Two stage slots (2 x 64 KiB at 256 x 256).  Each stage runs as two
//     32-wide halves: while the MFMAs of one half run from registers, the
//     wave reads the fragments of the next half into the other register
//     set.  Half 1 of stage D starts with the only barrier of the stage: it
//     makes stage D + 1 visible and frees slot D (its fragments are all in
//     registers by then), and the loads of stage D + 2 go there.  A load thus
//     has two halves of MFMA time to land.
//   * The epilogue is the shared LDS-staged one (epilogue.hpp), a wave row
//     (or part of one, where a whole row of 384-wide tiles would not fit)
//     at a time; the row dots of such tiles come straight from the
//     accumulators instead.
#pragma once

#include "dora_internal.hpp"
#include "epilogue.hpp"

#include <type_traits>
#include <utility>

namespace dora {
namespace dma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N - 1>).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

constexpr int BK = GEMM_DMA_BK;  // K values per stage
static_assert(BK == 64, "tile layouts below assume 64 K values per stage");
constexpr int ROW_BYTES = BK * 2;  // K-major tile row

// K-major chunk slot permutation; depends on the low 4 bits of r only.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// Chunk swizzle of MN-major tiles: t(k) = {0, 6, 10, 12}[k & 3].
__device__ __forceinline__ int swz_mn(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }

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
// loads of the stage about to be read; its LDS reads of the slot about to be
// refilled were consumed by MFMAs, hence complete.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// DH: the A operand is produced in the kernel (the backward's dh from dy, see
// gemm_dma_tile); a third tile per stage, of A's shape, holds y.
template <int BM, int BN, int WM, int WN, bool DH = false>
struct DmaCfg {
    static constexpr int NT = WM * WN * 64;
    static constexpr int NW = WM * WN;
    static constexpr int A_BYTES = BM * ROW_BYTES;  // also [BK][BM] for MN-major
    static constexpr int B_BYTES = BN * ROW_BYTES;
    static constexpr int Y_BYTES = DH ? A_BYTES : 0;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + Y_BYTES;
    static constexpr int OPS = 2 * STAGE_BYTES;
    // stored epilogue: fp32 rows of the tile staged in LDS, ER at a time (a
    // wave row's BM / WM rows, or half or a quarter of them where those do
    // not fit), handed to epilogue_rows in column slabs of EB (its 8-column
    // chunks must tile a wavefront: BN / 8 divides 64, else 128-wide slabs)
    static constexpr int CST = BN + 4;
    static constexpr int WTM_ = BM / WM;
    static constexpr int ER = WTM_ * CST * 4 <= 160 * 1024       ? WTM_
                              : (WTM_ / 2) * CST * 4 <= 160 * 1024 ? WTM_ / 2
                                                                   : WTM_ / 4;
    static_assert(ER % 32 == 0 && ER * CST * 4 <= 160 * 1024, "epilogue rows");
    static constexpr int EPI = ER * CST * 4;
    static constexpr int EB = 64 % (BN / 8) == 0 ? BN : 128;
    static_assert(BN % EB == 0, "epilogue column slabs");
    // the staged row-dot epilogue needs whole wave rows and one slab; other
    // tiles form their row dots from the accumulators directly
    // (and 128 x 128 tiles, the small-rank norm's: their row dots then need
    // no LDS pass per wave row)
    static constexpr bool DIRECT_ROWDOT = ER != WTM_ || EB != BN || (BM == 128 && BN == 128);
    // row-dot epilogue: the E tile (bf16, padded rows) and one partial sum
    // per wave column and tile row
    static constexpr int EP = BN * 2 + 16;
    static constexpr int E_BYTES = BM * EP;
    static constexpr int RED_BYTES = E_BYTES + WN * BM * 4;
    static constexpr int max2(int a, int b) { return a > b ? a : b; }
    static constexpr int SMEM = max2(max2(OPS, EPI), RED_BYTES);
    static_assert(SMEM <= 160 * 1024, "LDS");
    // 1 KiB load instructions per operand tile and per wave and stage
    static constexpr int A_INST = A_BYTES / 1024, B_INST = B_BYTES / 1024;
    static_assert(A_INST % NW == 0 && B_INST % NW == 0, "tile loads must split over wavefronts");
    static constexpr int LPS = (A_INST * (DH ? 2 : 1) + B_INST) / NW;
    static_assert(LPS < 64, "vmcnt range");
};

// Byte range of an operand buffer, capped to the 31 bits a descriptor
// range takes here.
__device__ __forceinline__ int range_bytes(int64_t bytes)
{
    return bytes < 0x7fffffff ? static_cast<int>(bytes) : 0x7fffffff;
}

// Loads go out in groups of four whose LDS destinations are consecutive
// 1 KiB blocks: the instruction offset (0, 1024, 2048, 3072) advances the
// LDS address and the global address alike, so m0 is written once per group.
// (An m0 write waits for the previous direct-to-LDS load to take its m0, so
// one write per load stalls the issuing wave, and with it the matrix core.)
// Per-lane offsets are pre-reduced by the instruction offset and raised by
// GROUP_BIAS, and the descriptor base is lowered by GROUP_BIAS, which keeps
// every offset non-negative.
// A tile whose loads per wave are not a multiple of four groups them in
// twos (or ones); the bias stays that of a group of four.
constexpr int GROUP = 4;
constexpr uint32_t GROUP_BIAS = (GROUP - 1) * 1024;
template <int PA, int PB>
constexpr int group_size()
{
    return (PA % 4 == 0 && PB % 4 == 0) ? 4 : (PA % 2 == 0 && PB % 2 == 0) ? 2 : 1;
}

// Buffer descriptor over one operand matrix (raw, byte-addressed; dword 3 =
// 0x00020000 selects plain linear addressing on gfx9-family parts), with its
// base lowered by GROUP_BIAS.  Loads at (biased) offsets past the range
// return zeros; the range check includes the instruction offset.  An empty
// range (`bytes` = 0) makes every load return zeros.  The base and range
// pass through readfirstlane so the descriptor is built in scalar registers
// even where it is chosen per stage.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scalar_rsrc(const void *base, int bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base) - GROUP_BIAS;
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
    const int64_t biased = bytes > 0 ? static_cast<int64_t>(bytes) + GROUP_BIAS : 0;
    const int nrec = __builtin_amdgcn_readfirstlane(
        static_cast<int>(biased < 0x7fffffff ? biased : 0x7fffffff));
    void *q = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, static_cast<short>(0), nrec, 0x00020000);
}

// A group of direct-to-LDS loads: set_m0 sets the group's LDS base, then
// load J moves lane l's 16 bytes at rsrc + v + soff + 1024 J to LDS byte
// lds + 1024 J + 16 l.  Issued from inline asm (no register outputs; memory
// and m0 clobbered) rather than the builtin: the compiler treats the builtin
// as an LDS store and then drains every such load (vmcnt(0)) before any
// transpose read it cannot prove disjoint, which would empty the pipeline
// each step.  Completion is covered by the kernel's explicit vmcnt waits and
// barriers.  The four loads of a group go out one by one between MFMAs
// (issued back to back they stall the wave at issue, and with it the matrix
// core); nothing between them writes m0, which no other instruction of the
// kernel uses.
__device__ __forceinline__ void set_m0(uint32_t lds)
{
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds) : "memory", "m0");
}
template <int J>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t v, uint32_t soff)
{
    __asm__ volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds" ::"v"(v), "s"(rsrc),
                     "s"(soff), "n"(J * 1024)
                     : "memory", "m0");
}

constexpr uint32_t OOB_OFFSET = 0x80000000u;  // beyond every descriptor range

// Load modes of a stage (see dma_prep).
constexpr int LOAD_ANY = 0, LOAD_SEG0 = 1, LOAD_SEG1 = 2, LOAD_NONE = 3;

// One operand's load plan: per-lane byte offsets (biased, see GROUP_BIAS)
// of the sources of the wave's load instructions, computed once per tile.
// Wave w fills the PER consecutive 1 KiB blocks from w * PER.
//   K-major (rows = M or N, ld over K): a block holds 8 tile rows; lane l
//   fetches row l >> 3 of the block and the K chunk that belongs at slot
//   l & 7 (kch[i]: its first K index within the stage).  A stage adds its K
//   offset as the scalar buffer offset.
//   MN-major (rows = K, ld over M or N): a block is 1 KiB of the [64][R]
//   tile; lane l fetches the chunk that belongs at byte 16 l.  A stage adds
//   k0 * ld * 2 to the per-lane offset (rows past K are out of range and
//   load as zeros).
// SW16: the MN-major chunk swizzle of the 16 x 16 x 32 MFMA fragments
// (swz_mn16 in gemm_persistent.hpp).
__device__ __forceinline__ int swz_mn16(int k) { return swz_mn(k) ^ (((k >> 3) & 1) << 1); }

template <bool KMAJ, int R, int NW, int G = GROUP, bool SW16 = false>
struct OperandDma {
    static constexpr int NINST = R * ROW_BYTES / 1024;
    static_assert(NINST % NW == 0, "tile loads must split over wavefronts");
    static constexpr int PER = NINST / NW;
    static_assert(PER % G == 0 && G <= GROUP, "whole load groups per wave");
    static constexpr int PITCH = R * 2;  // MN-major row bytes
    static_assert(KMAJ || R >= 128, "MN-major tiles need >= 16 chunks per row");
    uint32_t off[PER];

    // K-major: the first K index (within the stage) of the chunk lane l of
    // wave `wave` fetches for load i (formed where a stage needs it, not kept)
    __device__ __forceinline__ static uint32_t kchunk(int wave, int i, int lane)
    {
        const int rloc = (wave * PER + i) * 8 + (lane >> 3);
        return static_cast<uint32_t>(((lane & 7) ^ swz(rloc)) * 8);
    }

    __device__ __forceinline__ void init(int64_t mn_extent, int64_t ld, int64_t mn0, int wave,
                                         int lane)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = wave * PER + i;
            const uint32_t bias = GROUP_BIAS - (i % G) * 1024;
            if constexpr (KMAJ) {
                const int rloc = blk * 8 + (lane >> 3);
                const int chunk = (lane & 7) ^ swz(rloc);
                int64_t row = mn0 + rloc;
                row = row < mn_extent ? row : mn_extent - 1;
                off[i] = static_cast<uint32_t>((row * ld + chunk * 8) * 2) + bias;
            } else {
                const int b = blk * 1024 + lane * 16;
                const int krow = b / PITCH;
                const int chunk = ((b % PITCH) >> 4) ^ (SW16 ? swz_mn16(krow) : swz_mn(krow));
                int64_t col = mn0 + chunk * 8;
                col = col + 8 <= mn_extent ? col : mn_extent - 8;
                off[i] = static_cast<uint32_t>((krow * ld + col) * 2) + bias;
            }
        }
    }
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// The MFMA fragment of 32 M (or N) indices starting at `mn` and the 8 K
// values 16 q + 8 (lane >> 5) + 0..7 of a stage (q = 0..3): lane holds
// index mn + (lane & 31).
template <bool KMAJ, int R>
__device__ __forceinline__ bf16x8_t read_frag(const unsigned char *tile, int mn, int q, int lane)
{
    if constexpr (KMAJ) {
        const int row = mn + (lane & 31);
        const int fc = q * 2 + (lane >> 5);
        return *reinterpret_cast<const bf16x8_t *>(tile + row * ROW_BYTES + ((fc ^ swz(row)) << 4));
    } else {
        constexpr int PITCH = R * 2;
        const int grp = lane >> 4, j = lane & 15;
        const int col = mn + 16 * (grp & 1) + 4 * (j & 3);
        const int k = q * 16 + 8 * (grp >> 1) + (j >> 2);
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

// One half stage's MFMA operands of a wave: two 16-wide K slices, TM A and
// TN B 32-index fragments each.
template <int TM, int TN>
struct Frags {
    bf16x8_t a[2][TM], b[2][TN];
};

// Fragment read number o of half `h` (A fragments of K slice 0, B
// fragments of slice 0, then the same for slice 1).
template <bool AK, bool BKM, int BM, int BN, int TM, int TN, int WTM, int WTN, int O>
__device__ __forceinline__ void read_one(Frags<TM, TN> &f, const unsigned char *As,
                                         const unsigned char *Bs, int h, int wm, int wn, int lane)
{
    constexpr int kk = O / (TM + TN), idx = O % (TM + TN);
    if constexpr (idx < TM)
        f.a[kk][idx] = read_frag<AK, BM>(As, wm * WTM + idx * 32, 2 * h + kk, lane);
    else
        f.b[kk][idx - TM] = read_frag<BKM, BN>(Bs, wn * WTN + (idx - TM) * 32, 2 * h + kk, lane);
}

// MFMA number q of a half (q = kk * TM * TN + i * TN + j).
template <int TM, int TN, int Q>
__device__ __forceinline__ void mfma_one(f32x16_t (&acc)[TM][TN], const Frags<TM, TN> &f)
{
    constexpr int kk = Q / (TM * TN), i = (Q / TN) % TM, j = Q % TN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
}

// One output tile (tm, tn) of split z of the product g.
//
// DH (the backward's dB = s dh^T P with dh and dm formed on the way, for A
// = dy [K = T][M = d_out] MN-major, B = P MN-major, one segment): every stage
// also loads the matching tile of y (g.Y, same layout as dy), and once a
// stage has landed each thread turns two 16-byte chunks of the dy tile into
// dh = g dy (g = dh_m / dh_n per column, rounded once to bf16) in place,
// stores them to g.dh_out (from the tiles of the first N block) and adds
// dy * y into its running dm sums; the MFMAs then read dh.  A thread keeps
// one 8-column chunk of the tile for the whole K loop, so its dm sums need
// one fixed-order reduction over the tile's threads at the end, written to
// g.dm_part[z * M + m] (the raw sums over this split's tokens).
template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool ROWSQ, bool DH = false>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs &g, const int tm, const int tn,
                                              const int z)
{
    using C = DmaCfg<BM, BN, WM, WN, DH>;
    static_assert(!DH || (!AK && !BKM && !ROWSQ), "dh/dm production: both operands MN-major");
    constexpr int G = group_size<(BM * ROW_BYTES / 1024) / (WM * WN),
                                 (BN * ROW_BYTES / 1024) / (WM * WN)>();
    using DA = OperandDma<AK, BM, WM * WN, G>;
    using DB = OperandDma<BKM, BN, WM * WN, G>;
    constexpr int NT = C::NT;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold 32x32 MFMA tiles");
    static_assert(!ROWSQ || AK, "row sums of squares: K-major A");
    static_assert(DA::PER * (DH ? 2 : 1) + DB::PER == C::LPS, "load count");

    __shared__ __align__(1024) unsigned char smem[C::SMEM];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    // wave index as a scalar: LDS destinations of the DMA are then SGPR values
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;

    // stages of the concatenated K range, and this split's share
    const int64_t st1 = (g.seg[0].K + BK - 1) / BK;
    const int64_t st_total = st1 + (g.nseg > 1 ? (g.seg[1].K + BK - 1) / BK : 0);
    int64_t s_begin = static_cast<int64_t>(z) * g.steps_per_split;
    if (s_begin > st_total)
        s_begin = st_total;
    int64_t s_end = s_begin + g.steps_per_split;
    if (s_end > st_total)
        s_end = st_total;

    // byte ranges per segment (a K-major operand spans its M or N rows, an
    // MN-major one its K rows), and the load plan of the segment whose
    // stages are being loaded: every loop below loads stages of one segment
    // only, so one plan is kept and rebuilt between loops (use_seg)
    const int na0 = range_bytes((AK ? g.M : g.seg[0].K) * g.seg[0].lda * 2);
    const int nb0 = range_bytes((BKM ? g.N : g.seg[0].K) * g.seg[0].ldb * 2);
    int na1 = na0, nb1 = nb0;
    if (g.nseg > 1) {
        na1 = range_bytes((AK ? g.M : g.seg[1].K) * g.seg[1].lda * 2);
        nb1 = range_bytes((BKM ? g.N : g.seg[1].K) * g.seg[1].ldb * 2);
    }
    DA da;
    DB db;
    int plan_seg = -1;
    auto use_seg = [&](int q) {
        q = q > 0 && g.nseg > 1 ? 1 : 0;
        if (q != plan_seg) {
            da.init(g.M, g.seg[q].lda, m0, wave, lane);
            db.init(g.N, g.seg[q].ldb, n0, wave, lane);
            plan_seg = q;
        }
    };

    auto slot = [&](int64_t s) {
        return smem + static_cast<int>((s - s_begin) & 1) * C::STAGE_BYTES;
    };

    // Load group d of stage sd (A tile groups first).  Stages past the end
    // of this split go through descriptors with an empty range: they fetch
    // nothing and deposit zeros in a slot no later stage reads, so every
    // stage has the same shape (no branches, the same vmcnt bookkeeping).
    constexpr int GA = DA::PER / G, NG = C::LPS / G;
    //
    // MODE (compile-time at each call site) removes the per-lane selects
    // from the common stages: LOAD_SEG0 / LOAD_SEG1 for live stages lying
    // wholly inside K of segment 0 / 1, LOAD_NONE for stages past the
    // split's end (no loads), LOAD_ANY decides per lane (a segment's tail
    // stage, whose chunks past K must load as zeros; any stage of the
    // prologue).  dma_prep sets m0 to the group's LDS base and returns its
    // descriptor and offsets; load J of the group is then issue<J>.
    struct Group {
        __amdgpu_buffer_rsrc_t rs;
        uint32_t soff;
        uint32_t v[G];
    };
    auto dma_prep = [&](int64_t sd, int d, auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        const bool live = MODE == LOAD_ANY ? sd < s_end : true;
        const bool sg1 = MODE == LOAD_ANY ? sd >= st1 : MODE == LOAD_SEG1;
        const int64_t kd = (sg1 ? sd - st1 : sd) * BK;
        const int64_t kseg = sg1 ? g.seg[1].K : g.seg[0].K;
        // groups of the operand whose loads take longer go first and get the
        // most time to land: A (x, dh rows) for a K-major B, B (a weight
        // read MN-major) otherwise (measured both ways on x W^T and dh W)
        constexpr int GB = DB::PER / G;
        // DH: groups past A's load the y tile (A's shape and plan)
        const bool isy = DH && d >= GB + GA;
        const bool isa = BKM ? d < GA : (d >= GB && !isy);
        const int i0 = (isa ? (BKM ? d : d - GB) : isy ? d - GB - GA : (BKM ? d - GA : d)) * G;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((lds_void *)(slot(sd) +
                                                     (isa ? 0 : isy ? C::A_BYTES + C::B_BYTES
                                                                    : C::A_BYTES) +
                                                     (wave * (isa || isy ? DA::PER : DB::PER) +
                                                      i0) *
                                                         1024))));
        Group grp;
        uint32_t *v = grp.v;
        uint32_t soff;
        __amdgpu_buffer_rsrc_t rs;
        if (isa || isy) {
            rs = scalar_rsrc(isy ? g.Y : sg1 ? g.seg[1].a : g.seg[0].a,
                             live ? (sg1 ? na1 : na0) : 0);
            const int64_t ld = sg1 ? g.seg[1].lda : g.seg[0].lda;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t off = da.off[i0 + j];
                if constexpr (AK) {
                    if constexpr (MODE == LOAD_ANY)
                        v[j] = kd + DA::kchunk(wave, i0 + j, lane) < kseg ? off : OOB_OFFSET;
                    else
                        v[j] = off;
                } else {
                    v[j] = off + static_cast<uint32_t>(kd * ld * 2);
                }
            }
            soff = AK ? static_cast<uint32_t>(kd * 2) : 0u;
        } else {
            rs = scalar_rsrc(sg1 ? g.seg[1].b : g.seg[0].b, live ? (sg1 ? nb1 : nb0) : 0);
            const int64_t ld = sg1 ? g.seg[1].ldb : g.seg[0].ldb;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t off = db.off[i0 + j];
                if constexpr (BKM) {
                    if constexpr (MODE == LOAD_ANY)
                        v[j] = kd + DB::kchunk(wave, i0 + j, lane) < kseg ? off : OOB_OFFSET;
                    else
                        v[j] = off;
                } else {
                    v[j] = off + static_cast<uint32_t>(kd * ld * 2);
                }
            }
            soff = BKM ? static_cast<uint32_t>(kd * 2) : 0u;
        }
        grp.rs = rs;
        grp.soff = soff;
        set_m0(lds);
        return grp;
    };
    auto issue = [&](const Group &grp, auto j_c) {
        constexpr int J = decltype(j_c)::value;
        lds_dma16<J>(grp.rs, grp.v[J], grp.soff);
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.f;
    // ROWSQ: sums of squares of A's rows from the A fragments already in
    // registers (every wave of a wave row holds all of that row's WTM tile
    // rows): lane l covers row wm * WTM + i * 32 + (l & 31) of block i and K
    // half l >> 5 of each 16-wide step.  Every wave sums every block of its
    // rows (branch-free, two v_dot2_f32_bf16 chains per block, spread over
    // the first MFMAs of a half) and keeps blocks i = wn, wn + WN, ... at the
    // end.
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    float sq[ROWSQ ? TM : 1][2];
#pragma unroll
    for (int i = 0; i < (ROWSQ ? TM : 1); ++i)
        sq[i][0] = sq[i][1] = 0.f;
    auto rowsq_part = [&](const Frags<TM, TN> &f, auto kk_c) {
        constexpr int kk = decltype(kk_c)::value;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const bf16x8_t v = f.a[kk][i];
            const bf16x2_t p0 = __builtin_shufflevector(v, v, 0, 1);
            const bf16x2_t p1 = __builtin_shufflevector(v, v, 2, 3);
            const bf16x2_t p2 = __builtin_shufflevector(v, v, 4, 5);
            const bf16x2_t p3 = __builtin_shufflevector(v, v, 6, 7);
            sq[i][0] = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, sq[i][0], false);
            sq[i][1] = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, sq[i][1], false);
            sq[i][0] = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, sq[i][0], false);
            sq[i][1] = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, sq[i][1], false);
        }
    };

    // One half stage: the MFMAs of `cur` from registers and, between them,
    // the fragment reads of the next half into `nxt` and (half 1 only) the
    // loads of stage D + 2.  The scheduling barriers pin that interleaving:
    // left to itself the compiler clusters the LDS reads, which stalls the
    // single wave of a SIMD on a full LDS queue while its matrix core idles.
    constexpr int NMF = 2 * TM * TN;    // MFMAs per half
    constexpr int NRD = 2 * (TM + TN);  // fragment reads per half
    using FR = Frags<TM, TN>;
    // DH: dh = g dy in place over the landed A tile of stage sd, dh to
    // g.dh_out, dy * y into the running dm sums.  Thread tid keeps column
    // chunk c = tid % CPC of the tile (8 columns) and rows k = q / CPC of its
    // chunks q = tid + j NT.
    constexpr int CPC = DH ? BM / 8 : 1;          // 16-byte chunks per K row
    constexpr int NCHK = DH ? BK * CPC / NT : 1;  // chunks per thread and stage
    static_assert(!DH || (BK * CPC) % NT == 0, "dy chunks must split over threads");
    float gcol[DH ? 8 : 1], dmacc[DH ? 8 : 1];
    if constexpr (DH) {
        const int64_t col0 = m0 + (tid % CPC) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            gcol[q] = col0 + q < g.M ? g.dh_m[col0 + q] / g.dh_n[col0 + q] : 0.f;
            dmacc[q] = 0.f;
        }
    }
    // The dh chunks of the stage last produced go to g.dh_out as buffer
    // stores issued after that half's loads (flush_dh, which reads them back
    // from the stage's slot, untouched until the next half 1's loads): a
    // wave's memory operations retire in issue order, so the next stage's
    // wait for its loads can leave those NCHK stores in flight
    // (wait_vmcnt<NCHK>) instead of waiting for the writes too.  Lanes with
    // nothing to store (past T, past M, tiles of other N blocks, stages past
    // the split) store to an offset outside the descriptor's range, which the
    // hardware drops, so every wave issues the same NCHK stores each time.
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    uint32_t dh_off[NCHK];
    int64_t dh_sd = 0;  // the stage whose dh chunks flush_dh stores
    __amdgpu_buffer_rsrc_t dh_rs;
    if constexpr (DH) {
        const int64_t dh_bytes = tn == 0 ? g.seg[0].K * g.seg[0].lda * 2 : 0;
        dh_rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(g.dh_out), static_cast<short>(0),
            __builtin_amdgcn_readfirstlane(static_cast<int>(dh_bytes)), 0x00020000);
#pragma unroll
        for (int j = 0; j < NCHK; ++j)
            dh_off[j] = OOB_OFFSET;
    }
    auto produce_dh = [&](int64_t sd) {
        if constexpr (DH) {
            unsigned char *At = slot(sd);
            const unsigned char *Yt = At + C::A_BYTES + C::B_BYTES;
            const int c = tid % CPC;
            const int64_t col = m0 + c * 8;
#pragma unroll
            for (int j = 0; j < NCHK; ++j) {
                const int k = (tid + j * NT) / CPC;
                const int off = k * (BM * 2) + ((c ^ swz_mn(k)) << 4);
                const uint4 dv = *reinterpret_cast<const uint4 *>(At + off);
                const uint4 yv = *reinterpret_cast<const uint4 *>(Yt + off);
                const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
                const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
                float h[8];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float d0 = __uint_as_float(dw[w] << 16);
                    const float d1 = __uint_as_float(dw[w] & 0xffff0000u);
                    const float y0 = __uint_as_float(yw[w] << 16);
                    const float y1 = __uint_as_float(yw[w] & 0xffff0000u);
                    dmacc[2 * w] = __fmaf_rn(d0, y0, dmacc[2 * w]);
                    dmacc[2 * w + 1] = __fmaf_rn(d1, y1, dmacc[2 * w + 1]);
                    h[2 * w] = gcol[2 * w] * d0;
                    h[2 * w + 1] = gcol[2 * w + 1] * d1;
                }
                const uint4 hv = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]),
                                            pack_bf16x2(h[4], h[5]), pack_bf16x2(h[6], h[7]));
                *reinterpret_cast<uint4 *>(At + off) = hv;
                const int64_t t = sd * BK + k;
                dh_off[j] = t < g.seg[0].K && col < g.M
                                ? static_cast<uint32_t>((t * g.seg[0].lda + col) * 2)
                                : OOB_OFFSET;
            }
            dh_sd = sd;
            // the dh chunks are in LDS before any wave reads fragments
            wait_lgkm0();
            stage_barrier();
        }
    };
    auto flush_dh = [&]() {
        if constexpr (DH) {
            const unsigned char *At = slot(dh_sd);
            const int c = tid % CPC;
#pragma unroll
            for (int j = 0; j < NCHK; ++j) {
                const int k = (tid + j * NT) / CPC;
                const uint4 hv = *reinterpret_cast<const uint4 *>(At + k * (BM * 2) +
                                                                  ((c ^ swz_mn(k)) << 4));
                const i32x4_t v = {static_cast<int>(hv.x), static_cast<int>(hv.y),
                                   static_cast<int>(hv.z), static_cast<int>(hv.w)};
                __builtin_amdgcn_raw_buffer_store_b128(v, dh_rs, dh_off[j], 0, 0);
                dh_off[j] = OOB_OFFSET;  // a later flush before another stage is produced drops
            }
        }
    };

    auto half = [&](auto h_c, int64_t D, FR &cur, FR &nxt, auto mode_c) {
        constexpr int H = decltype(h_c)::value;
        constexpr bool MODE_LOADS = decltype(mode_c)::value != LOAD_NONE;
        constexpr int NLH = H == 1 && MODE_LOADS ? NG * G : 0;  // loads in this half
        constexpr int NOPS = NRD + NLH;
        // the reads of `cur` were issued during the previous half: retire
        // them here, so that no wait lands inside the interleaved sequence
        wait_lgkm0();
        if constexpr (H == 1) {
            // stage D + 1 has landed (it is the only one in flight); after
            // the barrier it is visible and every wave holds all of stage
            // D's fragments, so its slot takes stage D + 2
            // (DH: the newest NCHK operations are the previous stage's dh
            // stores, which may stay in flight)
            wait_vmcnt<DH ? NCHK : 0>();
            stage_barrier();
            if constexpr (DH) {
                if (D + 1 < s_end)
                    produce_dh(D + 1);
            }
        }
        // half 0 reads half 1 of the same stage; half 1 reads half 0 of D + 1
        const unsigned char *An = slot(H == 0 ? D : D + 1);
        const unsigned char *Bn = An + C::A_BYTES;
        // the reads and loads are spread over the first SPAN MFMAs: the last
        // read then has TAIL MFMAs of time to land before the next half
        // waits for it (measured: worth it for the 1 x 4 wave layout)
        constexpr int TAIL = (WM == 1 || WN == 1) ? 8 : 0;
        constexpr int SPAN = NMF - TAIL;
        static_assert(SPAN >= 2, "MFMA slots");
        Group grp;
        static_for<NMF>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            mfma_one<TM, TN, q>(acc, cur);
            if constexpr (ROWSQ && q < 2)
                rowsq_part(cur, std::integral_constant<int, q>{});
            constexpr int cnt = q < SPAN ? (q + 1) * NOPS / SPAN - q * NOPS / SPAN : 0;
            static_for<cnt>([&](auto oc) {
                constexpr int o = q * NOPS / SPAN + decltype(oc)::value;
                // loads spread evenly, from the first slot on (they have a
                // deadline; the reads only feed the next half); load li is
                // number li % G of group li / G
                constexpr int li = NLH > 0 && (o * NLH) % NOPS < NLH ? (o * NLH) / NOPS : -1;
                constexpr int rd = o - (o * NLH + NOPS - 1) / NOPS;
                if constexpr (li >= 0) {
                    if constexpr (li % G == 0)
                        grp = dma_prep(D + 2, li / G, mode_c);
                    issue(grp, std::integral_constant<int, li % G>{});
                } else {
                    read_one<AK, BKM, BM, BN, TM, TN, WTM, WTN, rd>(nxt, An, Bn, 1 - H, wm, wn,
                                                                    lane);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (H == 1)
            flush_dh();  // after this half's loads
    };

    FR fa, fb;  // half 0 and half 1 of a stage
    // EPI_MERGE on tiles of at most 128 x 128 (8 chunks, 32 VGPRs a thread):
    // the thread's chunks of W's tile are loaded before the K loop, in the
    // order the epilogue takes them, so their memory latency runs under the
    // product instead of after it.  They are older than every stage load, so
    // the stage waits below cover them too.
    constexpr int MCPR = C::EB / 8;
    constexpr int MITER = C::ER * MCPR / NT;
    constexpr int NPASS_ = WTM / C::ER;
    constexpr bool MPRE = C::DIRECT_ROWDOT && !DH && !ROWSQ && BM * BN <= 128 * 128;
    EChunk<uint16_t> wpre[MPRE ? WM * NPASS_ * (BN / C::EB) * MITER : 1];
    const bool mpre = MPRE && g.mode == EPI_MERGE;
    if constexpr (MPRE) {
        if (mpre) {
            static_for<WM>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
                static_for<NPASS_>([&](auto pc) {
                    constexpr int pass = decltype(pc)::value;
                    static_for<BN / C::EB>([&](auto sc) {
                        constexpr int sl = decltype(sc)::value;
                        constexpr int at = ((h * NPASS_ + pass) * (BN / C::EB) + sl) * MITER;
                        merge_chunk_load<C::ER, C::EB, NT, uint16_t>(
                            wpre + at, g, m0 + h * WTM + pass * C::ER, n0 + sl * C::EB, tid);
                    });
                });
            });
        }
    }
    if (s_begin < s_end) {
        // prologue: stages s_begin and s_begin + 1 in flight, then s_begin
        // visible and the fragments of its half 0 read
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            use_seg(s_begin + p >= st1 ? 1 : 0);
#pragma unroll
            for (int d = 0; d < NG; ++d) {
                const Group grp = dma_prep(s_begin + p, d, std::integral_constant<int, LOAD_ANY>{});
                static_for<G>([&](auto jc) { issue(grp, jc); });
            }
        }
        wait_vmcnt<C::LPS>();  // stage s_begin has landed
        stage_barrier();
        produce_dh(s_begin);
        flush_dh();
        static_for<NRD>([&](auto oc) {
            read_one<AK, BKM, BM, BN, TM, TN, WTM, WTN, decltype(oc)::value>(
                fa, slot(s_begin), slot(s_begin) + C::A_BYTES, 0, wm, wn, lane);
        });
        // the last stage still reads a (stale) next slot; nothing uses it
        // Stage D's half 1 loads stage L = D + 2.  The stages run as five
        // loops, each with one load mode: L inside segment 0's whole stages,
        // segment 0's tail stage, L inside segment 1's whole stages, segment
        // 1's tail stage, and L past this split's end (the last two stages).
        auto stages = [&](int64_t D0, int64_t D1, auto mode_c) {
            for (int64_t D = D0; D < D1; ++D) {
                half(std::integral_constant<int, 0>{}, D, fa, fb,
                     std::integral_constant<int, LOAD_ANY>{});
                half(std::integral_constant<int, 1>{}, D, fb, fa, mode_c);
            }
        };
        auto clamp = [](int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); };
        auto lesser = [](int64_t a, int64_t b) { return a < b ? a : b; };
        const int64_t full0 = g.seg[0].K / BK;
        const int64_t full1 = g.nseg > 1 ? g.seg[1].K / BK : 0;
        const int64_t e0 = clamp(lesser(full0, s_end) - 2, s_begin, s_end);
        const int64_t b1 = clamp(lesser(st1, s_end) - 2, e0, s_end);
        const int64_t e1 = clamp(lesser(st1 + full1, s_end) - 2, b1, s_end);
        const int64_t dd = clamp(s_end - 2, e1, s_end);
        // the first two loops load stages of segment 0, the next two of
        // segment 1 (stages past the split's end load nothing, whatever the
        // plan)
        if (s_begin < b1)
            use_seg(0);
        stages(s_begin, e0, std::integral_constant<int, LOAD_SEG0>{});
        stages(e0, b1, std::integral_constant<int, LOAD_ANY>{});
        use_seg(1);
        stages(b1, e1, std::integral_constant<int, LOAD_SEG1>{});
        stages(e1, dd, std::integral_constant<int, LOAD_ANY>{});
        stages(dd, s_end, std::integral_constant<int, LOAD_NONE>{});
        wait_vmcnt<0>();  // the empty loads past the end have deposited their zeros
    }
    stage_barrier();  // every wave is done reading the slots before LDS is reused

    if constexpr (DH) {
        // dm: the tile's threads of one column chunk summed in a fixed order
        constexpr int RS = NT / CPC;  // threads per column chunk
        float *red = reinterpret_cast<float *>(smem);  // [RS][BM]
#pragma unroll
        for (int q = 0; q < 8; ++q)
            red[(tid / CPC) * BM + (tid % CPC) * 8 + q] = dmacc[q];
        __syncthreads();
        for (int col = tid; col < BM; col += NT) {
            float sum = 0.f;
            for (int w = 0; w < RS; ++w)
                sum += red[w * BM + col];
            if (tn == 0 && m0 + col < g.M)
                g.dm_part[static_cast<int64_t>(z) * g.M + m0 + col] = sum;
        }
        __syncthreads();
    }

    if constexpr (ROWSQ) {
        if (g.rowsq != nullptr && tn == 0) {
#pragma unroll
            for (int u = 0; u < (TM + WN - 1) / WN; ++u) {
                const int i = wn + u * WN;
                float su = 0.f;
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    if (b == i)
                        su = sq[b][0] + sq[b][1];
                const float t = su + __shfl_xor(su, 32);
                const int64_t row = m0 + wm * WTM + i * 32 + lane;
                if (i < TM && lane < 32 && row < g.M)
                    g.rowsq[static_cast<int64_t>(z) * g.M + row] = t;
            }
        }
    }

    float *Cs = reinterpret_cast<float *>(smem);
    if constexpr (C::DIRECT_ROWDOT) {
        if (g.mode == EPI_ROWDOT) {
            // row dots straight from the accumulators (tiles whose staged epilogue
            // takes partial rows or column slabs)
            // rowdot[m] = sum over this tile's columns of C[m, n] E[m, n], reduced
            // from the accumulators: the E tile is staged in LDS, each lane forms
            // its rows' partial sums over its columns, lanes and then wave
            // columns are summed in a fixed order
            constexpr int CPRow = BN / 8;
            constexpr int NCH = BM * CPRow / NT;  // 16-byte E chunks per thread
            static_assert((BM * CPRow) % NT == 0, "E tile chunks must split over threads");
            const uint16_t *E = static_cast<const uint16_t *>(g.E);
            // all loads first, so their latencies overlap
            EChunk<uint16_t> ev[NCH];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int idx = tid + k * NT;
                const int64_t row = m0 + idx / CPRow, col = n0 + (idx % CPRow) * 8;
                if (row < g.M && col < g.N)
                    ev[k].load(E + row * g.lde + col, g.N - col < 8 ? static_cast<int>(g.N - col) : 8);
                else
                    ev[k].zero();
            }
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int idx = tid + k * NT;
                *reinterpret_cast<uint4 *>(smem + (idx / CPRow) * C::EP + (idx % CPRow) * 16) =
                    ev[k].raw;
            }
            __syncthreads();
            if (g.out != nullptr) {
                // the product itself as well (fp32, split z at out + z M ldc;
                // with out_accum, alpha times it added to what out holds): per
                // store, 32 lanes write 32 consecutive columns of one row
                float *o = static_cast<float *>(g.out) + static_cast<int64_t>(z) * g.M * g.ldc;
                const bool accum = g.out_accum != 0;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int64_t row =
                                m0 + wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                            const int64_t col = n0 + wn * WTN + j * 32 + (lane & 31);
                            if (row < g.M && col < g.N)
                                o[row * g.ldc + col] =
                                    accum ? o[row * g.ldc + col] + g.alpha * acc[i][j][v]
                                          : acc[i][j][v];
                        }
            }
            float *red = reinterpret_cast<float *>(smem + C::E_BYTES);  // [WN][BM]
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                float x[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rl = wm * WTM + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                    float p = 0.f;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int cl = wn * WTN + j * 32 + (lane & 31);
                        const float e = bf16_to_f32(
                            *reinterpret_cast<const uint16_t *>(smem + rl * C::EP + cl * 2));
                        const float prod = acc[i][j][v] * e;
                        p += n0 + cl < g.N ? prod : 0.f;
                    }
                    x[v] = p;
                }
                // Sum each of the 16 rows over the 32 lanes (columns) of a
                // half-wave: four halving exchanges over lane bits 4..1 leave one
                // row per lane (row index vid from those bits), summed over 16
                // lanes; a last exchange over bit 0 completes the 32.
#pragma unroll
                for (int b = 4, h = 8; b >= 1; --b, h >>= 1) {
                    const bool up = (lane >> b) & 1;
#pragma unroll
                    for (int k = 0; k < h; ++k) {
                        const float send = up ? x[k] : x[k + h];
                        const float keep = up ? x[k + h] : x[k];
                        x[k] = keep + __shfl_xor(send, 1 << b);
                    }
                }
                const float tot = x[0] + __shfl_xor(x[0], 1);
                const int vid = (((lane >> 4) & 1) << 3) | (((lane >> 3) & 1) << 2) |
                                (((lane >> 2) & 1) << 1) | ((lane >> 1) & 1);
                const int rl = wm * WTM + i * 32 + (vid >> 2) * 8 + (lane >> 5) * 4 + (vid & 3);
                if ((lane & 1) == 0)
                    red[wn * BM + rl] = tot;
            }
            __syncthreads();
            const int ntn = static_cast<int>((g.N + BN - 1) / BN);
            for (int r = tid; r < BM; r += NT) {
                float sum = 0.f;
                for (int w = 0; w < WN; ++w)
                    sum += red[w * BM + r];
                const int64_t m = m0 + r;
                if (m < g.M) {
                    g.rowdot[(static_cast<int64_t>(z) * ntn + tn) * g.M + m] = sum;
                    if (g.fin_n != nullptr) {
                        // the norm's finish: the partials summed in order z
                        double b = 0.0, c = 0.0;
                        for (int q = 0; q < g.fin_z; ++q) {
                            b += g.fin_base[static_cast<int64_t>(q) * g.M + m];
                            c += g.fin_cross[static_cast<int64_t>(q) * g.M + m];
                        }
                        g.fin_n[m] = norm_from_terms(b, c, static_cast<double>(sum), g.fin_s);
                    }
                }
            }
        } else {
            // ER rows of a wave row at a time: that wave stages them in LDS,
            // then every thread stores (or merges) them, EB columns per call
            constexpr int NPASS = WTM / C::ER, TMP = C::ER / 32;
            static_for<WM>([&](auto hc) __attribute__((always_inline)) {
                constexpr int h = decltype(hc)::value;
                static_for<NPASS>([&](auto pc) __attribute__((always_inline)) {
                    constexpr int pass = decltype(pc)::value;
                    if (wm == h) {
#pragma unroll
                        for (int i = 0; i < TMP; ++i)
#pragma unroll
                            for (int j = 0; j < TN; ++j)
#pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    const int row =
                                        i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                                    const int col = wn * WTN + j * 32 + (lane & 31);
                                    Cs[row * C::CST + col] = acc[pass * TMP + i][j][v];
                                }
                    }
                    __syncthreads();
                    static_for<BN / C::EB>([&](auto sc) __attribute__((always_inline)) {
                        constexpr int sl = decltype(sc)::value;
                        constexpr int at = MPRE ? ((h * NPASS + pass) * (BN / C::EB) + sl) * MITER
                                                : 0;
                        epilogue_rows<C::ER, C::EB, C::CST, NT, uint16_t>(
                            Cs + sl * C::EB, g, m0 + h * WTM + pass * C::ER, n0 + sl * C::EB, z,
                            tn, tid, mpre ? wpre + at : nullptr);
                    });
                    __syncthreads();
                });
            });
        }
    } else {
        // a wave row at a time: that wave stages its rows in LDS, then every
        // thread stores, merges or row-dots them
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
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool ROWSQ, bool DH = false>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_dma_kernel(GemmArgs g)
{
    int tm, tn;
    tile_coords(g.M, g.N, BM, BN, tm, tn);
    gemm_dma_tile<BM, BN, WM, WN, AK, BKM, ROWSQ, DH>(g, tm, tn, static_cast<int>(blockIdx.y));
}

// Several independent products in one launch (one tile configuration and
// operand layout): the workgroups of problem p are the linear ids
// [tile_start[p], tile_start[p + 1]), each problem's tiles x splits.
template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool ROWSQ>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_dma_grouped_kernel(GemmGroup grp)
{
    int p, tm, tn, z;
    group_coords(grp, BM, BN, p, tm, tn, z);
    gemm_dma_tile<BM, BN, WM, WN, AK, BKM, ROWSQ>(grp.p[p], tm, tn, z);
}

}  // namespace dma
}  // namespace dora
