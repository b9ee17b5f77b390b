// gemm_persistent.hpp - persistent variant of the pipelined bf16 GEMM for the
// large stored products (x W^T, the fused forward product, dx).
//
// One workgroup per CU walks its share of the output tiles (the XCD-aware
// order of tile_in_order: XCD x owns a contiguous run of logical tiles, its
// workgroups take them in turn) as one unbroken stream of K stages: the last
// two stages of a tile load the first two stages of the next, so the
// pipeline never drains between tiles and the per-tile fill of a
// one-tile-per-workgroup launch disappears.
//
// Its MFMAs are the 16 x 16 x 32 form (see read_frag16).  The epilogue runs
// per wave, without workgroup barriers, while the next tile's second stage
// is in flight (its first has landed):
//   * the MFMAs take the B fragment as their first operand and A as their
//     second, so each 16 x 16 accumulator block holds the transposed
//     product: lane l owns output row l & 15 and the four consecutive
//     columns 4 (l >> 4) + 0..3 -- after the fp32 -> bf16 rounding, eight
//     bytes of one row;
//   * a wave rounds 32 rows x 64 columns at a time into its own 4 KiB LDS
//     staging area (8-byte writes), reads them back as 16-byte row chunks
//     and stores 8 rows x 128 bytes per instruction (whole cache lines);
//   * with a magnitude scale (column factors m / n), two waves bring the m
//     and n of the next tile's 256 columns into LDS (one direct-to-LDS load
//     each, issued before that tile's first stage), each wave forms
//     g - 1 = (m - n) / n of its 128 columns once per tile, and the store
//     applies h + (g - 1) h in fp32 before the single rounding.
// The stores are the newest memory operations when the next tile starts;
// its first full wait (for its stage 1) also covers them.
#pragma once

#include "gemm_bf16_dma.hpp"

namespace dora {
namespace dma {

// The products run on v_mfma_f32_16x16x32_bf16: at the same matrix-core
// occupancy it draws less power per flop than the 32 x 32 x 16 form, so the
// part holds a higher clock under its power limit (measured from registers
// alone: 2.04 against 1.82 GHz, both 99% busy; x W^T at 8192 x 28672 x 8192
// 2.69 -> 2.54 ms).  A half stage (32 K values) is one K slice: lane l of a
// fragment holds index mn + (l & 15) and the 8 K values 32 h + 8 (l >> 4) +
// 0..7; the MFMAs take the B fragment as their first operand, so lane l of
// an accumulator block holds output row l & 15 and the four consecutive
// columns 4 (l >> 4) + 0..3.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int TM, int TN>
struct Frags16 {
    bf16x8_t a[TM], b[TN];
};

__device__ __forceinline__ bf16x8_t read_frag16(const unsigned char *tile, int mn, int h, int lane)
{
    const int row = mn + (lane & 15);
    const int fc = 4 * h + (lane >> 4);
    return *reinterpret_cast<const bf16x8_t *>(tile + row * ROW_BYTES + ((fc ^ swz(row)) << 4));
}

// The same fragment from an MN-major tile ([64 K rows][R], 16-byte chunk c
// of row k at c ^ swz_mn16(k)): two ds_read_b64_tr_b16, each giving the
// lanes of 16-lane group g the 16 columns from mn of 4 of their 8 rows.
// Groups 0 and 1 (and 2 and 3) read rows 8 apart at the same columns;
// swz_mn16 moves rows with bit 3 set by two chunks, so that the two groups'
// 4 rows x 32 bytes fall on distinct banks.
template <int R>
__device__ __forceinline__ bf16x8_t read_frag16_mn(const unsigned char *tile, int mn, int h,
                                                   int lane)
{
    constexpr int PITCH = R * 2;
    const int grp = lane >> 4, j = lane & 15;
    const int col = mn + 4 * (j & 3);
    const int k = 32 * h + 8 * grp + (j >> 2);
    const int k2 = k + 4;
    const unsigned char *p0 =
        tile + k * PITCH + (((col >> 3) ^ swz_mn16(k)) << 4) + ((col & 7) << 1);
    const unsigned char *p1 =
        tile + k2 * PITCH + (((col >> 3) ^ swz_mn16(k2)) << 4) + ((col & 7) << 1);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p1));
    const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Fragment read number O of half `h` (A fragments, then B; B K-major or
// MN-major).
template <bool BKM, int BN, int TM, int TN, int WTM, int WTN, int O>
__device__ __forceinline__ void read_one16(Frags16<TM, TN> &f, const unsigned char *As,
                                           const unsigned char *Bs, int h, int wm, int wn,
                                           int lane)
{
    if constexpr (O < TM)
        f.a[O] = read_frag16(As, wm * WTM + O * 16, h, lane);
    else if constexpr (BKM)
        f.b[O - TM] = read_frag16(Bs, wn * WTN + (O - TM) * 16, h, lane);
    else
        f.b[O - TM] = read_frag16_mn<BN>(Bs, wn * WTN + (O - TM) * 16, h, lane);
}

// MFMA number Q of a half (B fragment first: acc holds the transposed block).
template <int TM, int TN, int Q>
__device__ __forceinline__ void mfma_one16(f32x4_t (&acc)[TM][TN], const Frags16<TM, TN> &f)
{
    constexpr int i = Q / TN, j = Q % TN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// One direct-to-LDS load with a zero scalar offset, for loads issued outside
// the pipelined stage sequence.  The leading s_nop covers the wait states a
// VMEM instruction needs after a VALU write of an SGPR it reads (the
// descriptor may come from a register the compiler restores with
// v_readlane right before; it cannot see into the asm to insert them).
__device__ __forceinline__ void lds_dma16_once(__amdgpu_buffer_rsrc_t rsrc, uint32_t v)
{
    __asm__ volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:0 lds" ::"v"(v),
                     "s"(rsrc)
                     : "memory", "m0");
}

// LDS beyond the two stage slots: per wave, the bf16 staging rows and g - 1
// of its columns; per workgroup, m and n of a tile's columns (two buffers,
// alternating by tile).
constexpr int PST_STAGE_BYTES = 32 * 128;  // 32 rows x 64 bf16 columns
constexpr int PST_GM1_BYTES = 128 * 4;     // the wave's 128 columns
constexpr int PST_MN_BYTES = 2 * 256 * 4;  // m, then n, of 256 columns

template <int BM, int BN, int WM, int WN, bool BKM>
__global__ void __launch_bounds__(WM *WN * 64) gemm_bf16_dma_persistent_kernel(GemmArgs g)
{
    using C = DmaCfg<BM, BN, WM, WN>;
    constexpr bool AK = true;
    constexpr int G = group_size<(BM * ROW_BYTES / 1024) / (WM * WN),
                                 (BN * ROW_BYTES / 1024) / (WM * WN)>();
    using DA = OperandDma<AK, BM, WM * WN, G>;
    using DB = OperandDma<BKM, BN, WM * WN, G, !BKM>;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;  // 16 x 16 accumulator blocks
    static_assert(BN == 256 && WTN == 128 && NW >= 2, "m / n and staging layout");
    static_assert(DA::PER + DB::PER == C::LPS, "load count");
    constexpr int WAVE_OFF = C::OPS + 2 * PST_MN_BYTES;
    constexpr int SMEM = WAVE_OFF + NW * (PST_STAGE_BYTES + PST_GM1_BYTES);
    static_assert(SMEM <= 160 * 1024, "LDS");

    __shared__ __align__(1024) unsigned char smem[SMEM];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // this workgroup's tiles: first + k * per, k < count
    const int num_m = static_cast<int>((g.M + BM - 1) / BM);
    const int num_n = static_cast<int>((g.N + BN - 1) / BN);
    const int ntiles = num_m * num_n;
    int first, count, per;
    {
        const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
        const int xcd = b & 7, local = b >> 3;
        per = nb >> 3;
        const int q = ntiles >> 3, rem = ntiles & 7;
        const int start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
        const int len = q + (xcd < rem ? 1 : 0);
        first = start + local;
        count = local < len ? (len - local + per - 1) / per : 0;
    }
    if (count == 0)
        return;

    const int64_t st1 = (g.seg[0].K + BK - 1) / BK;
    const int64_t nst = st1 + (g.nseg > 1 ? (g.seg[1].K + BK - 1) / BK : 0);

    const int na0 = range_bytes(g.M * g.seg[0].lda * 2);
    const int nb0 = range_bytes((BKM ? g.N : g.seg[0].K) * g.seg[0].ldb * 2);
    int na1 = na0, nb1 = nb0;
    if (g.nseg > 1) {
        na1 = range_bytes(g.M * g.seg[1].lda * 2);
        nb1 = range_bytes((BKM ? g.N : g.seg[1].K) * g.seg[1].ldb * 2);
    }
    DA da;
    DB db;
    int plan_seg = -1, plan_tile = -1;
    // the load plan (per-lane offsets) of segment q of tile L
    auto use_plan = [&](int q, int L) {
        q = q > 0 && g.nseg > 1 ? 1 : 0;
        if (q != plan_seg || L != plan_tile) {
            int tm, tn;
            tile_in_order(L, g.M, g.N, BM, BN, tm, tn);
            // the lane index through an opaque move: the plan is then formed
            // here each time, not from lane-dependent terms the compiler
            // would otherwise hoist out of the tile loop and keep live
            int ln;
            __asm__ volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            da.init(g.M, g.seg[q].lda, static_cast<int64_t>(tm) * BM, wave, ln);
            db.init(g.N, g.seg[q].ldb, static_cast<int64_t>(tn) * BN, wave, ln);
            plan_seg = q;
            plan_tile = L;
        }
    };

    // running stage index S (over all of this workgroup's tiles) -> slot
    auto slot = [&](int64_t S) { return smem + static_cast<int>(S & 1) * C::STAGE_BYTES; };
    unsigned char *const stg = smem + WAVE_OFF + wave * (PST_STAGE_BYTES + PST_GM1_BYTES);
    float *const gm1 = reinterpret_cast<float *>(stg + PST_STAGE_BYTES);
    auto mn_area = [&](int k) {
        return reinterpret_cast<float *>(smem + C::OPS + (k & 1) * PST_MN_BYTES);
    };

    // m (wave 0) and n (wave 1) of the 256 columns of tile L into the m / n
    // buffer of tile number k (columns past N load as zeros): one
    // direct-to-LDS load each, 16 bytes a lane
    const bool scale = g.colm != nullptr;
    auto load_mn = [&](int L, int k) {
        if (wave < 2) {
            int tm, tn;
            tile_in_order(L, g.M, g.N, BM, BN, tm, tn);
            const int64_t col = static_cast<int64_t>(tn) * BN + 4 * lane;
            const __amdgpu_buffer_rsrc_t rs =
                scalar_rsrc(wave == 0 ? g.colm : g.coln, range_bytes(g.N * 4));
            const uint32_t off =
                col < g.N ? static_cast<uint32_t>(col * 4) + GROUP_BIAS : OOB_OFFSET;
            set_m0(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                (lds_void *)(mn_area(k) + wave * 256)))));
            lds_dma16_once(rs, off);
        }
    };

    constexpr int GA = DA::PER / G, NG = C::LPS / G;
    struct Group {
        __amdgpu_buffer_rsrc_t rs;
        uint32_t soff;
        uint32_t v[G];
    };
    // load group d of tile-relative stage sd into the slot of running stage
    // S (`some` false: the stage's loads fetch nothing)
    auto dma_prep = [&](int64_t S, int64_t sd, bool some, int d, auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        const bool live = MODE == LOAD_ANY ? some && sd < nst : true;
        const bool sg1 = MODE == LOAD_ANY ? sd >= st1 : MODE == LOAD_SEG1;
        const int64_t kd = (sg1 ? sd - st1 : sd) * BK;
        const int64_t kseg = sg1 ? g.seg[1].K : g.seg[0].K;
        constexpr int GB = DB::PER / G;
        const bool isa = BKM ? d < GA : d >= GB;
        const int i0 = (isa ? (BKM ? d : d - GB) : (BKM ? d - GA : d)) * G;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((lds_void *)(slot(S) + (isa ? 0 : C::A_BYTES) +
                                                     (wave * (isa ? DA::PER : DB::PER) + i0) *
                                                         1024))));
        Group grp;
        if (isa) {
            grp.rs = scalar_rsrc(sg1 ? g.seg[1].a : g.seg[0].a, live ? (sg1 ? na1 : na0) : 0);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t off = da.off[i0 + j];
                if constexpr (MODE == LOAD_ANY)
                    grp.v[j] = kd + DA::kchunk(wave, i0 + j, lane) < kseg ? off : OOB_OFFSET;
                else
                    grp.v[j] = off;
            }
            grp.soff = static_cast<uint32_t>(kd * 2);
        } else {
            grp.rs = scalar_rsrc(sg1 ? g.seg[1].b : g.seg[0].b, live ? (sg1 ? nb1 : nb0) : 0);
            const int64_t ld = sg1 ? g.seg[1].ldb : g.seg[0].ldb;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t off = db.off[i0 + j];
                if constexpr (BKM) {
                    if constexpr (MODE == LOAD_ANY)
                        grp.v[j] = kd + DB::kchunk(wave, i0 + j, lane) < kseg ? off : OOB_OFFSET;
                    else
                        grp.v[j] = off;
                } else {
                    grp.v[j] = off + static_cast<uint32_t>(kd * ld * 2);
                }
            }
            grp.soff = BKM ? static_cast<uint32_t>(kd * 2) : 0u;
        }
        set_m0(lds);
        return grp;
    };
    auto issue = [&](const Group &grp, auto j_c) {
        constexpr int J = decltype(j_c)::value;
        lds_dma16<J>(grp.rs, grp.v[J], grp.soff);
    };

    constexpr int NMF = TM * TN;  // MFMAs per half stage
    constexpr int NRD = TM + TN;  // fragment reads per half stage
    using FR = Frags16<TM, TN>;
    using ACC = f32x4_t[TM][TN];
    // fragment read O of half h, MFMA Q of a half
    auto read_op = [&](FR &f, const unsigned char *As, const unsigned char *Bs, int h, auto o_c) {
        read_one16<BKM, BN, TM, TN, WTM, WTN, decltype(o_c)::value>(f, As, Bs, h, wm, wn, lane);
    };
    auto mfma_op = [&](ACC &acc, const FR &f, auto q_c) {
        mfma_one16<TM, TN, decltype(q_c)::value>(acc, f);
    };

    // One half stage (as in gemm_dma_tile): the MFMAs of `cur`, the fragment
    // reads of the next half into `nxt` (READS), and in half 1 the loads of
    // tile-relative stage lsd into the slot of running stage S + 2, after
    // the m / n loads of tile mn_L where mn_L >= 0 (buffer of tile number
    // mn_k).
    auto half = [&](ACC &acc, auto h_c, int64_t S, int64_t lsd, bool some, FR &cur, FR &nxt,
                    auto mode_c, auto reads_c, int mn_L, int mn_k) {
        constexpr int H = decltype(h_c)::value;
        constexpr bool READS = decltype(reads_c)::value;
        constexpr bool MODE_LOADS = decltype(mode_c)::value != LOAD_NONE;
        constexpr int NLH = H == 1 && MODE_LOADS ? NG * G : 0;
        constexpr int NOPS = (READS ? NRD : 0) + NLH;
        wait_lgkm0();
        if constexpr (H == 1) {
            // stage D + 1 has landed (and the previous epilogue's stores,
            // the only other memory operations in flight, have completed)
            wait_vmcnt<0>();
            stage_barrier();
            if (mn_L >= 0)
                load_mn(mn_L, mn_k);
        }
        const unsigned char *An = slot(H == 0 ? S : S + 1);
        const unsigned char *Bn = An + C::A_BYTES;
        Group grp;
        static_for<NMF>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            mfma_op(acc, cur, std::integral_constant<int, q>{});
            constexpr int cnt = (q + 1) * NOPS / NMF - q * NOPS / NMF;
            static_for<cnt>([&](auto oc) {
                constexpr int o = q * NOPS / NMF + decltype(oc)::value;
                constexpr int li = NLH > 0 && (o * NLH) % NOPS < NLH ? (o * NLH) / NOPS : -1;
                constexpr int rd = o - (o * NLH + NOPS - 1) / NOPS;
                if constexpr (li >= 0) {
                    if constexpr (li % G == 0)
                        grp = dma_prep(S + 2, lsd, some, li / G, mode_c);
                    issue(grp, std::integral_constant<int, li % G>{});
                } else if constexpr (READS) {
                    read_op(nxt, An, Bn, 1 - H, std::integral_constant<int, rd>{});
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // output descriptor: the whole [M, ldc] bf16 matrix (the host keeps it
    // under 2 GiB)
    const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
        g.out, static_cast<short>(0),
        __builtin_amdgcn_readfirstlane(static_cast<int>(g.M * g.ldc * 2)), 0x00020000);
    typedef int i32x4_t __attribute__((ext_vector_type(4)));

    // Tile (m0, n0), tile number k, from the accumulators.  Staging rows are
    // 128 bytes (64 columns); 16-byte chunk c of row r sits at c ^ swz(r).
    auto epilogue = [&](ACC &acc, int64_t m0, int64_t n0, int k) {
        if (scale) {
            // g - 1 = (m - n) / n of the wave's columns 2 lane, 2 lane + 1
            const float *mn = mn_area(k) + wn * WTN + 2 * lane;
            const float2 mv = *reinterpret_cast<const float2 *>(mn);
            const float2 nv = *reinterpret_cast<const float2 *>(mn + 256);
            *reinterpret_cast<float2 *>(gm1 + 2 * lane) =
                make_float2((mv.x - nv.x) / nv.x, (mv.y - nv.y) / nv.y);
        }
        const int q4 = lane >> 4;
        // slab (i, hf): rows 32 i .. 32 i + 31 and columns 64 hf .. 64 hf + 63
        // of the wave tile, accumulator blocks (2 i + ii, 4 hf + jj)
#pragma unroll
        for (int i = 0; i < WTM / 32; ++i) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int rr = 16 * ii + (lane & 15);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = g.alpha * acc[2 * i + ii][4 * hf + jj][e];
                        if (scale) {
                            const float4 f = *reinterpret_cast<const float4 *>(
                                gm1 + hf * 64 + 16 * jj + 4 * q4);
                            v[0] = __fmaf_rn(f.x, v[0], v[0]);
                            v[1] = __fmaf_rn(f.y, v[1], v[1]);
                            v[2] = __fmaf_rn(f.z, v[2], v[2]);
                            v[3] = __fmaf_rn(f.w, v[3], v[3]);
                        }
                        // columns 16 jj + 4 q4 .. + 3: bytes 32 jj + 8 q4 of the row
                        const int c = 2 * jj + (q4 >> 1);
                        *reinterpret_cast<uint2 *>(stg + rr * 128 + ((c ^ swz(rr)) << 4) +
                                                   8 * (q4 & 1)) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                }
#pragma unroll
                for (int ps = 0; ps < 4; ++ps) {
                    const int rr = ps * 8 + (lane >> 3), c = lane & 7;
                    const uint4 u =
                        *reinterpret_cast<const uint4 *>(stg + rr * 128 + ((c ^ swz(rr)) << 4));
                    const i32x4_t v = {static_cast<int>(u.x), static_cast<int>(u.y),
                                       static_cast<int>(u.z), static_cast<int>(u.w)};
                    const int64_t m = m0 + wm * WTM + i * 32 + rr;
                    const int64_t col = n0 + wn * WTN + hf * 64 + c * 8;
                    const uint32_t off = m < g.M && col < g.N
                                             ? static_cast<uint32_t>((m * g.ldc + col) * 2)
                                             : OOB_OFFSET;
                    __builtin_amdgcn_raw_buffer_store_b128(v, out_rs, off, 0, 0);
                }
                // one slab at a time (left free, the scheduler converts every
                // block up front and runs out of registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto clamp = [](int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); };
    auto lesser = [](int64_t a, int64_t b) { return a < b ? a : b; };
    const int64_t full0 = g.seg[0].K / BK;
    const int64_t full1 = g.nseg > 1 ? g.seg[1].K / BK : 0;
    const int64_t e0 = clamp(lesser(full0, nst) - 2, 0, nst);
    const int64_t b1 = clamp(lesser(st1, nst) - 2, e0, nst);
    const int64_t e1 = clamp(lesser(st1 + full1, nst) - 2, b1, nst);
    const int64_t dd = nst - 2;  // nst >= 2 (host)

    FR fa, fb;
    // prologue: the first tile's m / n, then its stages 0 and 1
    if (scale)
        load_mn(first, 0);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        use_plan(p >= st1 ? 1 : 0, first);
#pragma unroll
        for (int d = 0; d < NG; ++d) {
            const Group grp = dma_prep(p, p, true, d, std::integral_constant<int, LOAD_ANY>{});
            static_for<G>([&](auto jc) { issue(grp, jc); });
        }
    }
    wait_vmcnt<C::LPS>();
    stage_barrier();
    static_for<NRD>([&](auto oc) { read_op(fa, slot(0), slot(0) + C::A_BYTES, 0, oc); });

    int64_t S0 = 0;  // running index of the current tile's stage 0
#pragma unroll 1
    for (int k = 0; k < count; ++k) {
        const int L = first + k * per;
        const bool has_next = k + 1 < count;
        ACC acc;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[i][j][v] = 0.f;
        auto stages = [&](int64_t D0, int64_t D1, auto mode_c) {
#pragma unroll 1
            for (int64_t D = D0; D < D1; ++D) {
                half(acc, std::integral_constant<int, 0>{}, S0 + D, D + 2, true, fa, fb,
                     std::integral_constant<int, LOAD_ANY>{}, std::true_type{}, -1, 0);
                half(acc, std::integral_constant<int, 1>{}, S0 + D, D + 2, true, fb, fa, mode_c,
                     std::true_type{}, -1, 0);
            }
        };
        if (0 < b1)
            use_plan(0, L);
        // the tile's first stage outside the stage loops: entered from the
        // zeroed accumulators, the loops' 64 four-register accumulators were
        // otherwise given other registers than the ones they leave in, and
        // copied back every stage
        int64_t D0 = 0;
        if (dd >= 1) {
            if (b1 == 0)
                use_plan(1, L);  // its loads (stage 2) lie in segment 1
            half(acc, std::integral_constant<int, 0>{}, S0, 2, true, fa, fb,
                 std::integral_constant<int, LOAD_ANY>{}, std::true_type{}, -1, 0);
            half(acc, std::integral_constant<int, 1>{}, S0, 2, true, fb, fa,
                 std::integral_constant<int, LOAD_ANY>{}, std::true_type{}, -1, 0);
            D0 = 1;
        }
        stages(std::min(D0, e0), e0, std::integral_constant<int, LOAD_SEG0>{});
        stages(std::max(D0, e0), b1, std::integral_constant<int, LOAD_ANY>{});
        use_plan(1, L);
        stages(std::max(D0, b1), e1, std::integral_constant<int, LOAD_SEG1>{});
        stages(std::max(D0, e1), dd, std::integral_constant<int, LOAD_ANY>{});
        // the last two stages load the next tile's stages 0 and 1 (the last
        // tile's load nothing: branch-free, with empty descriptor ranges)
        const int nxt = has_next ? L + per : L;
        {
            // stage nst - 2: its half 1 loads the next tile's m / n, then its
            // stage 0
            const int64_t D = dd;
            half(acc, std::integral_constant<int, 0>{}, S0 + D, 0, has_next, fa, fb,
                 std::integral_constant<int, LOAD_ANY>{}, std::true_type{}, -1, 0);
            use_plan(0 >= st1 ? 1 : 0, nxt);
            half(acc, std::integral_constant<int, 1>{}, S0 + D, 0, has_next, fb, fa,
                 std::integral_constant<int, LOAD_ANY>{}, std::true_type{},
                 scale && has_next ? nxt : -1, k + 1);
        }
        {
            // stage nst - 1: its half 1 loads the next tile's stage 1 and
            // reads no fragments (the next tile's first ones are read after
            // the epilogue, which then needs fewer registers)
            const int64_t D = nst - 1;
            half(acc, std::integral_constant<int, 0>{}, S0 + D, 1, has_next, fa, fb,
                 std::integral_constant<int, LOAD_ANY>{}, std::true_type{}, -1, 0);
            use_plan(1 >= st1 ? 1 : 0, nxt);
            half(acc, std::integral_constant<int, 1>{}, S0 + D, 1, has_next, fb, fa,
                 std::integral_constant<int, LOAD_ANY>{}, std::false_type{}, -1, 0);
        }
        int tm, tn;
        tile_in_order(L, g.M, g.N, BM, BN, tm, tn);
        epilogue(acc, static_cast<int64_t>(tm) * BM, static_cast<int64_t>(tn) * BN, k);
        S0 += nst;
        // the first fragments of the next tile (its stage 0 has landed: the
        // last half waited for it)
        static_for<NRD>([&](auto oc) { read_op(fa, slot(S0), slot(S0) + C::A_BYTES, 0, oc); });
    }
    wait_vmcnt<0>();  // the last tile's empty loads have deposited their zeros
}

}  // namespace dma
}  // namespace dora
