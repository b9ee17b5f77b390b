// dora_api.cpp - the C ABI of libdora.so (declared in include/dora.h).
//
// Host-side only: argument validation (before anything is enqueued), the
// launch plan (tile shape and split-K per product), the workspace carve-up
// and the launch sequences of the factored norm, the compose, the forward
// and the norm-detached backward.  Every step of the computation runs in
// the HIP kernels of gemm_bf16.hip, gemm_f32.hip and elementwise.hip.
#include <stdio.h>
#include <stdarg.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <vector>

#include "../../include/dora.h"
#include "dora_internal.hpp"

namespace dora {
namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(DORA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

int set_error(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

namespace {

#define DORA_LAUNCH(expr, what)                      \
    do {                                             \
        hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess)                        \
            return hip_fail(e_, what);               \
    } while (0)

constexpr int64_t kMaxDim = (1LL << 31) - 1;
constexpr size_t kAlign = 256;
constexpr int kCUs = 256;

size_t esize(int dtype) { return dtype == DORA_BF16 ? 2 : 4; }
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ planning
struct GPlan {
    int cfg = 0;         // bf16 tile configuration (fp32: unused)
    int BM = 0, BN = 0;
    int splits = 1;
    int64_t sps = 0;     // K steps per split
    int ntn = 0;         // tiles along N
};

// One product C[M, N] = sum_seg op(A) op(B) as the planner sees it.
struct GemmShape {
    int64_t M, N;
    int64_t K[2];
    int nseg;
    int layout;   // 0: A, B K-major; 1: B MN-major; 2: both MN-major
    bool dma_ok;  // direct-to-LDS kernel allowed (K-major K % 8, operands < 2 GiB)
    bool rowdot = false;  // EPI_ROWDOT epilogue (else EPI_STORE)
    bool rowsq = false;   // row sums of squares of A wanted
};

// Byte offsets of the direct-to-LDS kernel are 32-bit and carry a bias of
// up to 3 KiB (grouped loads); keep every operand's range below 2 GiB - 4 KiB.
constexpr int64_t kDmaBytes = (1LL << 31) - 4096;
constexpr double kWaveOverhead = 8e-6;  // seconds per wave of workgroups
// Extra seconds per wave when a row-dot epilogue stages the tile through LDS
// instead of dotting the accumulators directly (measured on the r-wide B G
// product of the norm at d_out 28672, r 384: 58.8 us on 256 x 256 tiles
// against 39.3 us on 128 x 384 ones, at equal tile counts and K steps).
constexpr double kStagedRowdotOverhead = 20e-6;

// Operands the direct-to-LDS kernel can take (bf16, byte offsets < 2 GiB):
// a K-major one of `rows` x `K` loads whole 16-byte chunks (K % 8) and zeros
// past K; an MN-major one ([K][ld]) loads its K tail as zeros but addresses
// up to one stage (64 rows) past K.
bool dma_operand(int64_t rows, int64_t K)
{
    return K % 8 == 0 && rows * K * 2 < kDmaBytes;
}
bool dma_mn_operand(int64_t K, int64_t ld)
{
    return ld % 8 == 0 && (K + GEMM_DMA_BK) * ld * 2 < kDmaBytes;
}

// Whether a bf16 product has an operand of ragged width: a K-major operand
// ([rows][K], ld = K) whose K is not a multiple of 8, or an MN-major one
// ([K][M or N], ld = M or N) whose M or N is not.  Only the element-masked
// configuration takes those.
bool shape_ragged(const GemmShape &sh)
{
    const bool ak = sh.layout < 2, bk = sh.layout == 0;
    for (int q = 0; q < sh.nseg; ++q)
        if ((ak || bk) && sh.K[q] % 8)
            return true;
    return (!ak && sh.M % 8) || (!bk && sh.N % 8);
}

GemmShape nt_shape(int64_t M, int64_t N, int64_t K)
{
    return GemmShape{M, N, {K, 0}, 1, 0, dma_operand(M, K) && dma_operand(N, K)};
}

// DORA_TILE_CFG=<index> (environment) restricts the bf16 planners to that
// tile configuration wherever it can serve the product, so that every tile
// shape can be run through every call; unset, the time model chooses.
int forced_tile_cfg()
{
    const char *e = getenv("DORA_TILE_CFG");
    if (e == nullptr || *e == '\0')
        return -1;
    char *end = nullptr;
    const long v = strtol(e, &end, 10);
    return (*end == '\0' && v >= 0 && v < gemm_bf16_num_cfgs()) ? static_cast<int>(v) : -1;
}

// Choose the tile configuration and the split-K count by a small time
// model: (256-CU waves) x (one workgroup's MFMA or VALU time), plus, for a
// split, writing and re-reading `part_per_split` fp32 values per split and
// one extra launch.  A split keeps at least 512 K values (128 for row-dot
// products, whose partials are one value per row and tile column) and its
// partials under 1 GiB.
GPlan plan_gemm(bool bf16, const GemmShape &sh, int64_t part_per_split, int only = -1)
{
    const double cu_flops = bf16 ? 4.0e12 : 157.3e12 / kCUs * 0.5;
    const double hbm = 5.0e12;
    GPlan best;
    double best_cost = -1.0;
    const int ncfg = bf16 ? gemm_bf16_num_cfgs() : 1;
    // `only`: plan that configuration alone (a product only it implements)
    const int forced = bf16 ? (only >= 0 ? only : forced_tile_cfg()) : -1;
    const bool ragged = bf16 && shape_ragged(sh);
    // pass 0: the forced configuration only (if any); pass 1: all of them,
    // when pass 0 found none that serves this product
    for (int pass = forced >= 0 ? 0 : 1; pass < (only >= 0 ? 1 : 2) && best_cost < 0; ++pass)
    for (int c = 0; c < ncfg; ++c) {
        int BM, BN, bk;
        float rel;
        if (pass == 0 && c != forced)
            continue;
        if (bf16) {
            const TileCfg t = gemm_bf16_cfg(c);
            if ((t.dma && !sh.dma_ok) || (!t.store_ok && !sh.rowdot) || (sh.rowsq && !t.rowsq_ok) ||
                (ragged && !t.ragged_ok))
                continue;
            BM = t.BM;
            BN = t.BN;
            bk = t.bk;
            rel = t.rel_speed;
        } else {
            BM = GEMM_F32_BM;
            BN = GEMM_F32_BN;
            bk = GEMM_F32_BK;
            rel = 1.0f;
        }
        int64_t steps = 0;
        for (int q = 0; q < sh.nseg; ++q)
            steps += (sh.K[q] + bk - 1) / bk;
        const int64_t tiles = ((sh.M + BM - 1) / BM) * ((sh.N + BN - 1) / BN);
        // a split keeps at least 512 K values (128 for a row-dot product)
        const int64_t kmin = sh.rowdot ? 128 : 512;
        const int64_t zmax = std::min<int64_t>(32, std::max<int64_t>(steps * bk / kmin, 1));
        for (int64_t z = 1; z <= zmax; ++z) {
            if (z > 1 && static_cast<double>(z) * part_per_split * 4.0 > (1LL << 30))
                break;
            const int64_t sps = (steps + z - 1) / z;
            const int64_t waves = std::max<int64_t>((tiles * z + kCUs - 1) / kCUs, 1);
            // a wave of workgroups also pays its pipeline fill and epilogue
            // (measured: about 8 us on the row-dot products of the norm)
            const bool staged_rowdot = sh.rowdot && !(bf16 && gemm_bf16_cfg(c).direct_rowdot);
            double cost = static_cast<double>(waves) *
                          (2.0 * BM * BN * bk * static_cast<double>(std::max<int64_t>(sps, 1)) /
                               (cu_flops * rel) +
                           kWaveOverhead + (staged_rowdot ? kStagedRowdotOverhead : 0.0));
            if (z > 1)
                cost += 2.0 * z * part_per_split * 4.0 / hbm + 3e-6;
            if (best_cost < 0 || cost < best_cost * 0.97) {
                best_cost = cost;
                best.cfg = c;
                best.BM = BM;
                best.BN = BN;
                best.splits = static_cast<int>(z);
                best.sps = sps;
                best.ntn = static_cast<int>((sh.N + BN - 1) / BN);
            }
        }
    }
    return best;
}

// Workspace carve-up: offsets are computed identically by the size queries
// and by the calls.
struct Carve {
    size_t off = 0;
    size_t take(size_t bytes)
    {
        const size_t at = off;
        off += align_up(bytes);
        return at;
    }
};

struct NormPlan {
    GPlan g, u, bg;
    // G = A A^T as extra tiles of the U = W A^T launch (one wave of
    // workgroups with room beside U's tiles, U unsplit): G's tiles take as
    // long as U's (the same K) and write G_hi / G_lo themselves
    bool g_with_u = false;
    // G = A A^T as split-K tiles of a split U launch (split like U, fp32
    // partials, then the fixed-order finalize), where both fit beside each
    // other on the CUs
    bool g_split_with_u = false;
    size_t o_gpart, o_gfin, o_base, o_cross, o_gram;
    size_t bytes;
};

NormPlan plan_norm(int64_t d_out, int64_t d_in, int64_t r, int dtype, Carve &cv)
{
    const bool bf = dtype == DORA_BF16;
    NormPlan p;
    p.g = plan_gemm(bf, nt_shape(r, r, d_in), r * r);
    GemmShape us = nt_shape(d_out, r, d_in);
    us.rowdot = us.rowsq = true;
    p.u = plan_gemm(bf, us, 2 * d_out);
    GemmShape bgs{d_out, r, {r, r}, bf ? 2 : 1, 1, dma_operand(d_out, r) && dma_mn_operand(r, r)};
    bgs.rowdot = true;
    p.bg = plan_gemm(bf, bgs, d_out);
    if (bf && p.u.splits == 1 && gemm_bf16_cfg(p.u.cfg).dma && gemm_bf16_cfg(p.u.cfg).store_ok) {
        const TileCfg t = gemm_bf16_cfg(p.u.cfg);
        const int64_t tu = ((d_out + t.BM - 1) / t.BM) * ((r + t.BN - 1) / t.BN);
        const int64_t tg = ((r + t.BM - 1) / t.BM) * ((r + t.BN - 1) / t.BN);
        if (tu + tg <= kCUs && dma_operand(r, d_in)) {
            p.g_with_u = true;
            p.g = p.u;
            p.g.ntn = static_cast<int>((r + t.BN - 1) / t.BN);
        }
    } else if (bf && p.u.splits > 1 && gemm_bf16_cfg(p.u.cfg).dma &&
               gemm_bf16_cfg(p.u.cfg).store_ok && dma_operand(r, d_in)) {
        // workgroups resident per CU: two stage slots of both operand tiles
        const TileCfg t = gemm_bf16_cfg(p.u.cfg);
        const int64_t per_cu = (160 * 1024) / (2 * (t.BM + t.BN) * GEMM_DMA_BK * 2);
        const int64_t tu = ((d_out + t.BM - 1) / t.BM) * ((r + t.BN - 1) / t.BN);
        const int64_t tg = ((r + t.BM - 1) / t.BM) * ((r + t.BN - 1) / t.BN);
        if ((tu + tg) * p.u.splits <= kCUs * per_cu) {
            p.g_split_with_u = true;
            p.g = p.u;
            p.g.ntn = static_cast<int>((r + t.BN - 1) / t.BN);
        }
    }
    const size_t start = cv.off;
    p.o_gpart = cv.take(static_cast<size_t>(p.g.splits) * r * r * 4);
    p.o_gfin = cv.take(bf ? 2 * r * r * 2 : r * r * 4);
    p.o_base = cv.take(static_cast<size_t>(p.u.splits) * d_out * 4);
    p.o_cross = cv.take(static_cast<size_t>(p.u.splits) * p.u.ntn * d_out * 4);
    p.o_gram = cv.take(static_cast<size_t>(p.bg.splits) * p.bg.ntn * d_out * 4);
    p.bytes = cv.off - start;
    return p;
}

struct LinPlan {
    GPlan g;
    size_t bytes;
};

// The base product's plan, shared by dora_forward and dora_linear.
GPlan plan_base(bool bf, int64_t T, int64_t d_in, int64_t d_out)
{
    return plan_gemm(bf, nt_shape(T, d_out, d_in), T * d_out);
}

LinPlan plan_linear(int64_t T, int64_t d_in, int64_t d_out, int dtype)
{
    LinPlan l;
    l.g = plan_base(dtype == DORA_BF16, T, d_in, d_out);
    l.bytes = l.g.splits > 1 ? align_up(static_cast<size_t>(l.g.splits) * T * d_out * 4) : 0;
    return l;
}

// Merge: the norm (unless the caller has it) and one product C = B A (M =
// d_out, N = d_in, K = r) whose epilogue forms W' = W + ((g - 1) W + g s C)
// by rows.  The epilogue needs whole sums, so the product is never split.
constexpr int64_t kNoSplit = int64_t(1) << 40;  // part_per_split that rules out split-K

struct MergePlan {
    NormPlan norm;
    GPlan g;
    size_t o_n;
    size_t bytes;
};

MergePlan plan_merge(int64_t d_out, int64_t d_in, int64_t r, int dtype)
{
    const bool bf = dtype == DORA_BF16;
    MergePlan p;
    Carve cv;
    p.norm = plan_norm(d_out, d_in, r, dtype, cv);
    p.o_n = cv.take(static_cast<size_t>(d_out) * 4);
    const GemmShape sh{d_out, d_in, {r, 0}, 1, 1,
                       dma_operand(d_out, r) && dma_mn_operand(r, d_in)};
    p.g = plan_gemm(bf, sh, kNoSplit);
    if (bf && sh.dma_ok && forced_tile_cfg() < 0) {
        // The product is short (K = r) and its epilogue streams W in and W'
        // out: 128 x 128 tiles keep two workgroups per CU, so one's epilogue
        // traffic overlaps the other's MFMAs (measured faster than the
        // compute-only time model's pick at 28672 x 8192, r 384).
        for (int c = 0; c < gemm_bf16_num_cfgs(); ++c) {
            const TileCfg t = gemm_bf16_cfg(c);
            if (t.dma && t.store_ok && t.BM == 128 && t.BN == 128) {
                p.g.cfg = c;
                p.g.BM = t.BM;
                p.g.BN = t.BN;
                p.g.splits = 1;
                p.g.sps = (r + t.bk - 1) / t.bk;
                p.g.ntn = static_cast<int>((d_in + t.BN - 1) / t.BN);
            }
        }
    }
    p.bytes = cv.off;
    return p;
}

// Forward: the norm, P = x A^T, then one K-concatenated product
// [x | s P] [W | B]^T whose fp32 accumulator h = x W^T + s P B^T is stored as
// (m/n) h by the epilogue (no [T, d_out] intermediate).
struct FwdPlan {
    NormPlan norm;
    GPlan p, fused;
    size_t o_P, o_Ppart, o_sP, o_part_fused;
    size_t bytes;
};

GemmShape fused_shape(int64_t T, int64_t d_in, int64_t d_out, int64_t r)
{
    return GemmShape{T, d_out, {d_in, r}, 2, 0,
                     dma_operand(T, d_in) && dma_operand(d_out, d_in) && dma_operand(T, r) &&
                         dma_operand(d_out, r)};
}

FwdPlan plan_forward(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype)
{
    const bool bf = dtype == DORA_BF16;
    FwdPlan f;
    Carve cv;
    f.norm = plan_norm(d_out, d_in, r, dtype, cv);
    f.p = plan_gemm(bf, nt_shape(T, r, d_in), T * r);
    f.fused = plan_gemm(bf, fused_shape(T, d_in, d_out, r), T * d_out);
    const size_t e = esize(dtype);
    f.o_P = cv.take(static_cast<size_t>(T) * r * e);
    f.o_Ppart = cv.take(f.p.splits > 1 ? static_cast<size_t>(f.p.splits) * T * r * 4 : 0);
    f.o_sP = cv.take(static_cast<size_t>(T) * r * e);
    f.o_part_fused =
        cv.take(f.fused.splits > 1 ? static_cast<size_t>(f.fused.splits) * T * d_out * 4 : 0);
    f.bytes = cv.off;
    return f;
}

struct BwdPlan {
    GPlan q, dx, dB, dA;
    // dh and the dm sums formed inside the dB product (one pass over dy and
    // y that also computes dB), else by the separate dh/dm pass
    bool fused_dhdm;
    int64_t sweep;  // rows per sweep of the dh/dm pass
    int nchunks;    // dm partial sums per column
    size_t o_dh, o_dmpart, o_Q, o_Qpart, o_dxpart, o_dBpart, o_dApart;
    size_t bytes;
};

BwdPlan plan_backward(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype)
{
    const bool bf = dtype == DORA_BF16;
    BwdPlan b;
    Carve cv;
    b.q = plan_gemm(bf, GemmShape{T, r, {d_out, 0}, 1, 1,
                                  dma_operand(T, d_out) && dma_mn_operand(d_out, r)},
                    T * r);
    b.dx = plan_gemm(bf, GemmShape{T, d_in, {d_out, r}, 2, 1,
                                   dma_operand(T, d_out) && dma_mn_operand(d_out, d_in) &&
                                       dma_operand(T, r) && dma_mn_operand(r, d_in)},
                     T * d_in);
    const GemmShape dbs{d_out, r, {T, 0}, 1, 2, dma_mn_operand(T, d_out) && dma_mn_operand(T, r)};
    b.dA = plan_gemm(bf, GemmShape{r, d_in, {T, 0}, 1, 2,
                                   dma_mn_operand(T, r) && dma_mn_operand(T, d_in)},
                     r * d_in);
    // dh/dm inside the dB product: bf16, the pipelined layout, tokens to
    // stream, and no tile configuration other than the one that implements
    // it requested (a test restricting the planners to another one runs the
    // separate pass)
    const int forced = forced_tile_cfg();
    b.fused_dhdm = false;
    if (bf && dbs.dma_ok && T > 0)
        for (int c = 0; c < gemm_bf16_num_cfgs() && !b.fused_dhdm; ++c)
            if (gemm_bf16_cfg(c).dhdm_ok && (forced < 0 || forced == c)) {
                b.dB = plan_gemm(bf, dbs, d_out * r, c);
                b.fused_dhdm = b.dB.cfg == c;
            }
    if (!b.fused_dhdm)
        b.dB = plan_gemm(bf, dbs, d_out * r);
    b.sweep = T > 0 ? dm_sweep_rows(T, d_out) : 0;
    b.nchunks = b.fused_dhdm ? b.dB.splits : static_cast<int>(b.sweep);
    const size_t e = esize(dtype);
    b.o_dh = cv.take(static_cast<size_t>(T) * d_out * e);
    b.o_dmpart = cv.take(static_cast<size_t>(std::max(b.nchunks, 1)) * d_out * 4);
    b.o_Q = cv.take(static_cast<size_t>(T) * r * e);
    b.o_Qpart = cv.take(b.q.splits > 1 ? static_cast<size_t>(b.q.splits) * T * r * 4 : 0);
    b.o_dxpart = cv.take(b.dx.splits > 1 ? static_cast<size_t>(b.dx.splits) * T * d_in * 4 : 0);
    b.o_dBpart = cv.take(b.dB.splits > 1 ? static_cast<size_t>(b.dB.splits) * d_out * r * 4 : 0);
    b.o_dApart = cv.take(b.dA.splits > 1 ? static_cast<size_t>(b.dA.splits) * r * d_in * 4 : 0);
    b.bytes = cv.off;
    return b;
}

// Backward through the norm: the detached plan's dh/dm, Q and dx, then the
// norm's gradient, with cs = -s m dm / n^2 and cB = cs (.) B:
//   dA = [Q^T | cB^T] [x ; W] + s (cB^T B) A
//   dB = s dh^T P + cs (.) (W A^T + s B G),   G = A A^T
// Every part lands as fp32 slots (split-K partials included) that one
// fixed-order pass sums and rounds.
struct ThruPlan {
    BwdPlan b;
    GPlan g, da, gs, z, y1, y2;
    int na, nb, ny;  // fp32 slots of dA, of dB's s dh^T P, of W A^T + s B G
    size_t o_cs, o_cB, o_gpart, o_gfin, o_gspart, o_gsfin, o_aslots, o_bslots, o_yslots;
    size_t bytes;
};

ThruPlan plan_through_norm(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype)
{
    const bool bf = dtype == DORA_BF16;
    ThruPlan p;
    p.b = plan_backward(T, d_in, d_out, r, dtype);
    p.g = plan_gemm(bf, nt_shape(r, r, d_in), r * r);
    p.da = plan_gemm(bf, GemmShape{r, d_in, {T, d_out}, 2, 2,
                                   dma_mn_operand(T, r) && dma_mn_operand(T, d_in) &&
                                       dma_mn_operand(d_out, r) && dma_mn_operand(d_out, d_in)},
                     r * d_in);
    p.gs = plan_gemm(bf, GemmShape{r, r, {d_out, 0}, 1, 2, dma_mn_operand(d_out, r)}, r * r);
    p.z = plan_gemm(bf, GemmShape{r, d_in, {r, r}, bf ? 2 : 1, 1,
                                  dma_operand(r, r) && dma_mn_operand(r, d_in)},
                    r * d_in);
    p.y1 = plan_gemm(bf, nt_shape(d_out, r, d_in), d_out * r);
    p.y2 = plan_gemm(bf, GemmShape{d_out, r, {r, r}, bf ? 2 : 1, 1,
                                   dma_operand(d_out, r) && dma_mn_operand(r, r)},
                     d_out * r);
    p.na = p.da.splits + p.z.splits;
    p.nb = p.b.dB.splits;
    p.ny = p.y1.splits + p.y2.splits;
    Carve cv;
    cv.off = p.b.bytes;
    const size_t e = esize(dtype);
    p.o_cs = cv.take(static_cast<size_t>(d_out) * 4);
    p.o_cB = cv.take(static_cast<size_t>(d_out) * r * e);
    p.o_gpart = cv.take(static_cast<size_t>(p.g.splits) * r * r * 4);
    p.o_gfin = cv.take(bf ? 2 * r * r * 2 : r * r * 4);
    p.o_gspart = cv.take(static_cast<size_t>(p.gs.splits) * r * r * 4);
    p.o_gsfin = cv.take(bf ? 2 * r * r * 2 : r * r * 4);
    p.o_aslots = cv.take(static_cast<size_t>(p.na) * r * d_in * 4);
    p.o_bslots = cv.take(static_cast<size_t>(p.nb) * d_out * r * 4);
    p.o_yslots = cv.take(static_cast<size_t>(p.ny) * d_out * r * 4);
    p.bytes = cv.off;
    return p;
}

// ---------------------------------------------------------------- validation
struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0)
        return false;
    const char *a0 = static_cast<const char *>(a.p), *b0 = static_cast<const char *>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_dtype(int dtype)
{
    if (dtype != DORA_F32 && dtype != DORA_BF16)
        return fail(DORA_E_DTYPE, "unknown dtype %d", dtype);
    return DORA_OK;
}

int check_dims(int dtype, int64_t T, int64_t d_in, int64_t d_out, int64_t r)
{
    if (T < 0 || T > kMaxDim)
        return fail(DORA_E_SHAPE, "T=%lld out of range [0, 2^31)", (long long)T);
    if (d_in < 1 || d_in > kMaxDim || d_out < 1 || d_out > kMaxDim || r < 1 || r > kMaxDim)
        return fail(DORA_E_SHAPE, "need 1 <= d_in, d_out, r < 2^31 (got %lld, %lld, %lld)",
                    (long long)d_in, (long long)d_out, (long long)r);
    return DORA_OK;
}

struct Ptr {
    const void *p;
    const char *name;
    bool required;
};

int check_ptrs(std::initializer_list<Ptr> ps)
{
    for (const Ptr &q : ps) {
        if (!q.p) {
            if (q.required)
                return fail(DORA_E_NULL, "%s is NULL", q.name);
            continue;
        }
        if (!aligned(q.p))
            return fail(DORA_E_ALIGN, "%s is not 16-byte aligned", q.name);
    }
    return DORA_OK;
}

int check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (need == 0)
        return DORA_OK;
    if (!ws)
        return fail(DORA_E_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (ws_bytes < need)
        return fail(DORA_E_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    if (!aligned(ws))
        return fail(DORA_E_ALIGN, "workspace is not 16-byte aligned");
    return DORA_OK;
}

struct Named {
    Range r;
    const char *name;
};

// Every output must be disjoint from every other listed buffer.
int check_disjoint(std::initializer_list<Named> outs, std::initializer_list<Named> others)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(o->r, o2->r))
                return fail(DORA_E_ALIAS, "%s overlaps %s", o->name, o2->name);
        for (const Named &b : others)
            if (overlap(o->r, b.r))
                return fail(DORA_E_ALIAS, "%s overlaps %s", o->name, b.name);
    }
    return DORA_OK;
}

#define DORA_CHECK(expr)             \
    do {                             \
        int rc_ = (expr);            \
        if (rc_ != DORA_OK)          \
            return rc_;              \
    } while (0)

// ----------------------------------------------------------------- launching
hipError_t run_gemm(bool bf16, const GPlan &p, GemmArgs a, int layout, bool rowsq, hipStream_t st)
{
    a.splits = p.splits;
    a.steps_per_split = p.sps;
    return bf16 ? launch_gemm_bf16(a, layout, p.cfg, rowsq, st)
                : launch_gemm_f32(a, layout, rowsq, st);
}

// Product into fp32 slots: split z writes alpha * its partial sum at
// slots + z * M * N (one slot when unsplit).
int run_slots(bool bf16, const GPlan &p, GemmArgs a, int layout, float *slots, float alpha,
              hipStream_t st, const char *what)
{
    a.mode = EPI_STORE;
    a.out = slots;
    a.ldc = a.N;
    a.out_f32 = 1;
    a.alpha = alpha;
    DORA_LAUNCH(run_gemm(bf16, p, a, layout, false, st), what);
    return DORA_OK;
}

GemmArgs seg1(int64_t M, int64_t N, const void *a, int64_t lda, const void *b, int64_t ldb,
              int64_t K)
{
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.M = M;
    g.N = N;
    g.seg[0] = GemmSeg{a, lda, b, ldb, K};
    g.nseg = 1;
    g.alpha = 1.0f;
    return g;
}

// A store-mode product: directly into `out` (dtype) when unsplit, otherwise
// through fp32 split partials and a fixed-order reduction.
int run_store(bool bf16, const GPlan &p, GemmArgs a, int layout, void *out, int64_t ldc,
              float alpha, float *part, hipStream_t st, const char *what)
{
    a.mode = EPI_STORE;
    if (p.splits <= 1) {
        a.out = out;
        a.ldc = ldc;
        a.out_f32 = bf16 ? 0 : 1;
        a.alpha = alpha;
        DORA_LAUNCH(run_gemm(bf16, p, a, layout, false, st), what);
    } else {
        a.out = part;
        a.ldc = a.N;
        a.out_f32 = 1;
        a.alpha = 1.0f;
        DORA_LAUNCH(run_gemm(bf16, p, a, layout, false, st), what);
        DORA_LAUNCH(launch_splitk_reduce(bf16, part, p.splits, a.M, a.N, alpha, out, st), what);
    }
    return DORA_OK;
}

// dh = g dy, the dm partial sums and the dB product in one pass over dy and
// y (BwdPlan::fused_dhdm): alpha dh^T P stored to `out` in the element type
// when `f32` is 0 (unsplit plans only), else as fp32 split slots (slot z at
// out + z d_out r).
int run_dhdm_dB(const BwdPlan &b, const void *dy, const void *y, const float *m, const float *n,
                const void *P, int64_t T, int64_t d_out, int64_t r, void *dh, float *dmpart,
                void *out, int f32, float alpha, hipStream_t st)
{
    if (!f32 && b.dB.splits > 1)
        return fail(DORA_E_HIP, "dh, dm and dB: a split product needs fp32 slots");
    GemmArgs a = seg1(d_out, r, dy, d_out, P, r, T);
    a.Y = y;
    a.dh_out = dh;
    a.dm_part = dmpart;
    a.dh_m = m;
    a.dh_n = n;
    a.mode = EPI_STORE;
    a.splits = b.dB.splits;
    a.steps_per_split = b.dB.sps;
    a.out = out;
    a.ldc = r;
    a.out_f32 = f32;
    a.alpha = alpha;
    DORA_LAUNCH(launch_gemm_bf16_dhdm(a, b.dB.cfg, st), "dh, dm and dB");
    return DORA_OK;
}

int norm_impl(const void *W, const void *A, const void *B, float s, int64_t d_out, int64_t d_in,
              int64_t r, int dtype, float *n, float *base, float *cross, float *gram,
              const NormPlan &p, char *ws, hipStream_t st, float *U_out = nullptr)
{
    const bool bf = dtype == DORA_BF16;
    float *gpart = reinterpret_cast<float *>(ws + p.o_gpart);
    void *gfin = ws + p.o_gfin;
    float *bpart = reinterpret_cast<float *>(ws + p.o_base);
    float *cpart = reinterpret_cast<float *>(ws + p.o_cross);
    float *gmpart = reinterpret_cast<float *>(ws + p.o_gram);
    // the finish rides in B G's epilogue where that product is unsplit with
    // one N tile on a kernel whose row dots come from the accumulators (and
    // the separate terms are not asked for)
    const bool fuse_finish = bf && base == nullptr && cross == nullptr && gram == nullptr &&
                             p.bg.splits == 1 && p.bg.ntn == 1 && p.u.ntn == 1 &&
                             gemm_bf16_cfg(p.bg.cfg).dma && gemm_bf16_cfg(p.bg.cfg).direct_rowdot;

    // G = A A^T, split-K partials, then a fixed-order sum (+ hi/lo split for
    // bf16); or, beside U's tiles, unsplit tiles writing G_hi and G_lo.
    GemmArgs gg = seg1(r, r, A, d_in, A, d_in, d_in);
    gg.mode = EPI_STORE;
    gg.ldc = r;
    if (p.g_with_u) {
        gg.out = gfin;
        gg.out_f32 = 0;
        gg.out2 = static_cast<uint16_t *>(gfin) + r * r;
        gg.out2_lo = 1;
        gg.splits = 1;
        gg.steps_per_split = p.g.sps;
    } else {
        gg.out = gpart;
        gg.out_f32 = 1;
        if (p.g_split_with_u) {
            gg.splits = p.g.splits;
            gg.steps_per_split = p.g.sps;
        } else {
            DORA_LAUNCH(run_gemm(bf, p.g, gg, 0, false, st), "gram A A^T");
            DORA_LAUNCH(launch_gram_finalize(bf, gpart, p.g.splits, r, gfin, st),
                        "gram finalize");
        }
    }
    // U = W A^T never leaves the tile: cross partials = rowdot(U_tile, B_tile),
    // base partials = row sums of W^2 from the same staged W.
    {
        GemmArgs g = seg1(d_out, r, W, d_in, A, d_in, d_in);
        g.mode = EPI_ROWDOT;
        g.E = B;
        g.lde = r;
        g.rowdot = cpart;
        g.rowsq = bpart;
        if (U_out && p.u.splits == 1) {
            // keep U itself (fp32), written by the same product
            g.out = U_out;
            g.ldc = r;
        }
        if (p.g_with_u || p.g_split_with_u) {
            // one launch: U's tiles, then G's
            GemmGroup grp;
            memset(&grp, 0, sizeof grp);
            grp.count = 2;
            grp.p[0] = g;
            grp.p[0].splits = p.u.splits;
            grp.p[0].steps_per_split = p.u.sps;
            grp.p[1] = gg;
            DORA_LAUNCH(launch_gemm_bf16_grouped(grp, 0, p.u.cfg, true, st), "cross W A^T, gram A A^T");
            if (p.g_split_with_u)
                DORA_LAUNCH(launch_gram_finalize(bf, gpart, p.g.splits, r, gfin, st),
                            "gram finalize");
        } else {
            DORA_LAUNCH(run_gemm(bf, p.u, g, 0, true, st), "cross W A^T");
        }
        if (U_out && p.u.splits > 1) {
            // a split product has only partial U tiles: form U once more,
            // unsplit (no workspace), as a plain fp32 product
            GemmArgs a = seg1(d_out, r, W, d_in, A, d_in, d_in);
            a.mode = EPI_STORE;
            a.out = U_out;
            a.ldc = r;
            a.out_f32 = 1;
            DORA_LAUNCH(run_gemm(bf, plan_gemm(bf, nt_shape(d_out, r, d_in), kNoSplit), a, 0,
                                 false, st),
                        "U = W A^T");
        }
    }
    // gram partials = rowdot(B G, B); bf16 forms B G as B G_hi + B G_lo.
    // With U_out, the same product adds s B G to the kept U: U_out then holds
    // V A^T = (W + s B A) A^T = U + s B G (an unsplit product: one writer per
    // element; a split one leaves it to an unsplit fp32 product).
    {
        GemmArgs g = seg1(d_out, r, B, r, gfin, r, r);
        if (bf) {
            g.seg[1] = GemmSeg{B, r, static_cast<const uint16_t *>(gfin) + r * r, r, r};
            g.nseg = 2;
        }
        GemmArgs a = g;
        g.mode = EPI_ROWDOT;
        g.E = B;
        g.lde = r;
        g.rowdot = gmpart;
        if (U_out && p.bg.splits == 1) {
            g.out = U_out;
            g.ldc = r;
            g.out_accum = 1;
            g.alpha = s;
        }
        if (fuse_finish) {
            // the whole Gram term is this product's row dot: its epilogue
            // also forms n (the finish kernel's arithmetic, same order)
            g.fin_n = n;
            g.fin_base = bpart;
            g.fin_cross = cpart;
            g.fin_z = p.u.splits;
            g.fin_s = s;
        }
        DORA_LAUNCH(run_gemm(bf, p.bg, g, 1, false, st), "gram B G");
        if (U_out && p.bg.splits > 1) {
            a.mode = EPI_STORE;
            a.out = U_out;
            a.ldc = r;
            a.out_f32 = 1;
            a.out_accum = 1;
            a.alpha = s;
            const GemmShape bgs{d_out, r, {r, r}, bf ? 2 : 1, 1,
                                dma_operand(d_out, r) && dma_mn_operand(r, r)};
            DORA_LAUNCH(run_gemm(bf, plan_gemm(bf, bgs, kNoSplit), a, 1, false, st),
                        "V A^T += s B G");
        }
    }
    if (!fuse_finish)
        DORA_LAUNCH(launch_norm_finish(bpart, p.u.splits, cpart, p.u.splits * p.u.ntn, gmpart,
                                       p.bg.splits * p.bg.ntn, d_out, s, n, base, cross, gram,
                                       st),
                    "norm finish");
    return DORA_OK;
}

// The forward's launch sequence (arguments already validated).
int forward_impl(const void *x, const void *W, const void *A, const void *B, const float *m,
                 float s, int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype, void *y,
                 float *n_out, void *P_out, const float *n_in, const FwdPlan &p, char *w,
                 hipStream_t st, float *U_out = nullptr)
{
    const bool bf = dtype == DORA_BF16;
    // 1. the row norm (factored), unless the caller has it.
    if (n_in) {
        if (n_in != n_out)
            DORA_LAUNCH(launch_copy_f32(n_in, n_out, d_out, st), "copy n_in");
    } else {
        DORA_CHECK(norm_impl(W, A, B, s, d_out, d_in, r, dtype, n_out, nullptr, nullptr, nullptr,
                             p.norm, w, st, U_out));
    }
    if (T == 0)
        return DORA_OK;
    void *P = P_out ? P_out : static_cast<void *>(w + p.o_P);
    // 2. P = x A^T (kept for the backward) and, unless s = 1, s P as the
    //    second K segment's operand: both from the same fp32 sums, each
    //    rounded once.
    void *sP = s != 1.0f ? static_cast<void *>(w + p.o_sP) : P;
    {
        GemmArgs g = seg1(T, r, x, d_in, A, d_in, d_in);
        g.mode = EPI_STORE;
        if (p.p.splits <= 1) {
            g.out = P;
            g.ldc = r;
            g.out_f32 = bf ? 0 : 1;
            if (sP != P) {
                g.out2 = sP;
                g.alpha2 = s;
            }
            DORA_LAUNCH(run_gemm(bf, p.p, g, 0, false, st), "adapter x A^T");
        } else {
            float *part = reinterpret_cast<float *>(w + p.o_Ppart);
            g.out = part;
            g.ldc = r;
            g.out_f32 = 1;
            DORA_LAUNCH(run_gemm(bf, p.p, g, 0, false, st), "adapter x A^T");
            DORA_LAUNCH(launch_splitk_reduce(bf, part, p.p.splits, T, r, 1.0f, P, st, nullptr,
                                             nullptr, sP != P ? sP : nullptr, s),
                        "adapter x A^T reduce");
        }
    }
    // 4. y = (m/n) (x W^T + s P B^T): one K-concatenated product; the epilogue
    //    applies the magnitude scale in the cancellation-safe form and rounds once.
    {
        GemmArgs g = seg1(T, d_out, x, d_in, W, d_in, d_in);
        g.seg[1] = GemmSeg{sP, r, B, r, r};
        g.nseg = 2;
        g.mode = EPI_STORE;
        g.colm = m;
        g.coln = n_out;
        if (p.fused.splits <= 1) {
            g.out = y;
            g.ldc = d_out;
            g.out_f32 = bf ? 0 : 1;
            DORA_LAUNCH(run_gemm(bf, p.fused, g, 0, false, st), "fused forward product");
        } else {
            // split-K: fp32 partials of h; the fixed-order sum applies the
            // same scale and rounds once
            float *part = reinterpret_cast<float *>(w + p.o_part_fused);
            g.colm = g.coln = nullptr;
            g.out = part;
            g.ldc = d_out;
            g.out_f32 = 1;
            DORA_LAUNCH(run_gemm(bf, p.fused, g, 0, false, st), "fused forward product");
            DORA_LAUNCH(launch_splitk_reduce(bf, part, p.fused.splits, T, d_out, 1.0f, y, st, m,
                                             n_out),
                        "fused forward reduce");
        }
    }
    return DORA_OK;
}

// ----------------------------------------------------------- grouped modules
// Many modules in few launches: up to kMaxGroup products per GEMM launch
// (one tile configuration for all of them) and per small-kernel launch.

int in_module(int rc, int i)
{
    if (rc != DORA_OK) {
        char tmp[sizeof g_last_error];
        snprintf(tmp, sizeof tmp, "module %d: %s", i, g_last_error);
        memcpy(g_last_error, tmp, sizeof tmp);
    }
    return rc;
}

int check_module(const dora_module &md, int i, int dtype, bool need_m)
{
    DORA_CHECK(in_module(check_dims(dtype, 0, md.d_in, md.d_out, md.r), i));
    return in_module(check_ptrs({{md.W, "W", true}, {md.A, "A", true}, {md.B, "B", true},
                                 {md.m, "m", need_m}}),
                     i);
}

// One grouped launch: tile configuration and a common split count.
struct GroupGemm {
    int cfg = -1;
    int splits = 1;
};

// Direct-to-LDS configuration for a set of products (every shape must allow
// it), and the split count when `split` is allowed (fp32 partial or row-dot
// outputs): the same time model as plan_gemm, summed over the products.
GroupGemm plan_group(const std::vector<GemmShape> &sh, bool split)
{
    GroupGemm best;
    double best_cost = -1.0;
    const double cu_flops = 4.0e12;
    for (const GemmShape &q : sh)
        if (!q.dma_ok)
            return best;
    const int forced = forced_tile_cfg();
    for (int pass = forced >= 0 ? 0 : 1; pass < 2 && best_cost < 0; ++pass)
    for (int c = 0; c < gemm_bf16_num_cfgs(); ++c) {
        const TileCfg t = gemm_bf16_cfg(c);
        if (!t.dma || (pass == 0 && c != forced))
            continue;
        bool ok = true, rowdot = false;
        int64_t zmax = split ? 32 : 1;
        for (const GemmShape &q : sh) {
            ok = ok && (t.store_ok || q.rowdot) && (!q.rowsq || t.rowsq_ok);
            rowdot = rowdot || q.rowdot;
            int64_t steps = 0;
            for (int k = 0; k < q.nseg; ++k)
                steps += (q.K[k] + t.bk - 1) / t.bk;
            // as in plan_gemm: 512 K values per split, 128 for a row-dot product
            zmax = std::min<int64_t>(zmax,
                                     std::max<int64_t>(steps * t.bk / (q.rowdot ? 128 : 512), 1));
        }
        if (!ok)
            continue;
        const double t_step = 2.0 * t.BM * t.BN * t.bk / (cu_flops * t.rel_speed);
        for (int64_t z = 1; z <= zmax; ++z) {
            double work = 0.0, longest = 0.0;
            int64_t tiles = 0;
            for (const GemmShape &q : sh) {
                int64_t steps = 0;
                for (int k = 0; k < q.nseg; ++k)
                    steps += (q.K[k] + t.bk - 1) / t.bk;
                const int64_t tl = ((q.M + t.BM - 1) / t.BM) * ((q.N + t.BN - 1) / t.BN) * z;
                const double tile_time = static_cast<double>((steps + z - 1) / z) * t_step;
                tiles += tl;
                work += tl * tile_time;
                longest = std::max(longest, tile_time);
            }
            const int64_t waves = std::max<int64_t>((tiles + kCUs - 1) / kCUs, 1);
            const double cost =
                std::max(work / kCUs, longest) +
                waves * (kWaveOverhead +
                         (rowdot && !t.direct_rowdot ? kStagedRowdotOverhead : 0.0));
            if (best_cost < 0 || cost < best_cost * 0.97) {
                best_cost = cost;
                best.cfg = c;
                best.splits = static_cast<int>(z);
            }
        }
    }
    return best;
}

GPlan as_gplan(const GroupGemm &g, const GemmShape &q)
{
    const TileCfg t = gemm_bf16_cfg(g.cfg);
    GPlan p;
    p.cfg = g.cfg;
    p.BM = t.BM;
    p.BN = t.BN;
    p.splits = g.splits;
    int64_t steps = 0;
    for (int k = 0; k < q.nseg; ++k)
        steps += (q.K[k] + t.bk - 1) / t.bk;
    p.sps = (steps + g.splits - 1) / g.splits;
    p.ntn = static_cast<int>((q.N + t.BN - 1) / t.BN);
    return p;
}

// The factored norm of modules [i0, i1) (at most kMaxGroup): G = A A^T of
// all of them in one launch, the hi/lo rounding in one, the W A^T row dots
// (with the row sums of squares of W) in one, the B G row dots in one and
// the finish in one.  fp32 modules, and bf16 ones the direct-to-LDS kernel
// cannot take, run module by module (norm_impl).
struct NormChunk {
    int i0 = 0, i1 = 0;
    bool grouped = false;
    GroupGemm g, u, bg;
    std::vector<GPlan> pg, pu, pbg;
    std::vector<NormPlan> single;
    std::vector<size_t> o_gpart, o_gfin, o_base, o_cross, o_gram;
    size_t bytes = 0;
};

NormChunk plan_norm_chunk(const dora_module *mods, int i0, int i1, int dtype)
{
    NormChunk c;
    c.i0 = i0;
    c.i1 = i1;
    const bool bf = dtype == DORA_BF16;
    std::vector<GemmShape> sg, su, sbg;
    for (int i = i0; i < i1; ++i) {
        const dora_module &md = mods[i];
        sg.push_back(nt_shape(md.r, md.r, md.d_in));
        GemmShape us = nt_shape(md.d_out, md.r, md.d_in);
        us.rowdot = us.rowsq = true;
        su.push_back(us);
        GemmShape b{md.d_out, md.r, {md.r, md.r}, 2, 1,
                    dma_operand(md.d_out, md.r) && dma_mn_operand(md.r, md.r)};
        b.rowdot = true;
        sbg.push_back(b);
    }
    if (bf) {
        c.g = plan_group(sg, true);
        c.u = plan_group(su, true);
        c.bg = plan_group(sbg, true);
        c.grouped = c.g.cfg >= 0 && c.u.cfg >= 0 && c.bg.cfg >= 0;
    }
    Carve cv;
    if (!c.grouped) {
        for (int i = i0; i < i1; ++i) {
            Carve one;
            c.single.push_back(plan_norm(mods[i].d_out, mods[i].d_in, mods[i].r, dtype, one));
            c.bytes = std::max(c.bytes, one.off);
        }
        return c;
    }
    for (int k = 0; k < i1 - i0; ++k) {
        const dora_module &md = mods[i0 + k];
        c.pg.push_back(as_gplan(c.g, sg[k]));
        c.pu.push_back(as_gplan(c.u, su[k]));
        c.pbg.push_back(as_gplan(c.bg, sbg[k]));
        c.o_gpart.push_back(cv.take(static_cast<size_t>(c.g.splits) * md.r * md.r * 4));
        c.o_gfin.push_back(cv.take(static_cast<size_t>(2) * md.r * md.r * 2));
        c.o_base.push_back(cv.take(static_cast<size_t>(c.u.splits) * md.d_out * 4));
        c.o_cross.push_back(
            cv.take(static_cast<size_t>(c.u.splits) * c.pu.back().ntn * md.d_out * 4));
        c.o_gram.push_back(
            cv.take(static_cast<size_t>(c.bg.splits) * c.pbg.back().ntn * md.d_out * 4));
    }
    c.bytes = cv.off;
    return c;
}

// Longest first: modules in order of decreasing d_in (the K of their
// largest product), so that each chunk holds products of similar length
// and a launch's long tiles start first.
std::vector<int> by_length(const dora_module *mods, std::vector<int> which)
{
    std::stable_sort(which.begin(), which.end(),
                     [&](int a, int b) { return mods[a].d_in > mods[b].d_in; });
    return which;
}

std::vector<NormChunk> plan_norm_group(const dora_module *mods, const std::vector<int> &which,
                                       int dtype, size_t &bytes)
{
    // `which` lists the modules to normalise (in chunk order); chunks are
    // runs of it
    std::vector<dora_module> sel;
    for (int i : which)
        sel.push_back(mods[i]);
    std::vector<NormChunk> out;
    bytes = 0;
    for (int i0 = 0; i0 < static_cast<int>(sel.size()); i0 += kMaxGroup) {
        const int i1 = std::min<int>(i0 + kMaxGroup, static_cast<int>(sel.size()));
        out.push_back(plan_norm_chunk(sel.data(), i0, i1, dtype));
        bytes = std::max(bytes, out.back().bytes);
    }
    return out;
}

int norm_group_impl(const dora_module *mods, const std::vector<int> &which, int dtype,
                    float *const *n, const std::vector<NormChunk> &chunks, char *ws,
                    hipStream_t st)
{
    const bool bf = dtype == DORA_BF16;
    for (const NormChunk &c : chunks) {
        const int cnt = c.i1 - c.i0;
        if (!c.grouped) {
            for (int k = 0; k < cnt; ++k) {
                const int i = which[c.i0 + k];
                const dora_module &md = mods[i];
                DORA_CHECK(norm_impl(md.W, md.A, md.B, md.s, md.d_out, md.d_in, md.r, dtype, n[i],
                                     nullptr, nullptr, nullptr, c.single[k], ws, st));
            }
            continue;
        }
        GemmGroup gg, gu, gbg;
        memset(&gg, 0, sizeof gg);
        memset(&gu, 0, sizeof gu);
        memset(&gbg, 0, sizeof gbg);
        ItemGroup<GramItem> fin;
        ItemGroup<NormFinishItem> nf;
        memset(&fin, 0, sizeof fin);
        memset(&nf, 0, sizeof nf);
        gg.count = gu.count = gbg.count = fin.count = nf.count = cnt;
        // the tiles of different modules share no operand rows: deal them
        // to the XCDs in turn so each XCD gets a share of every module (in
        // XCD runs the longest-first order gives the first XCDs all the
        // longest products: 3.39 -> 2.88 ms on 56 decoder projections)
        gg.spread = gu.spread = gbg.spread = 1;
        // B G's epilogue forms n when every B G of the chunk is unsplit with
        // one N tile (as for one module: the finish launch then goes)
        bool fuse = gemm_bf16_cfg(c.bg.cfg).direct_rowdot && c.bg.splits == 1;
        for (int k = 0; k < cnt; ++k)
            fuse = fuse && c.pbg[k].ntn == 1 && c.pu[k].ntn == 1;
        for (int k = 0; k < cnt; ++k) {
            const dora_module &md = mods[which[c.i0 + k]];
            const int64_t r = md.r, d_in = md.d_in, d_out = md.d_out;
            float *gpart = reinterpret_cast<float *>(ws + c.o_gpart[k]);
            void *gfin = ws + c.o_gfin[k];
            float *bpart = reinterpret_cast<float *>(ws + c.o_base[k]);
            float *cpart = reinterpret_cast<float *>(ws + c.o_cross[k]);
            float *gmpart = reinterpret_cast<float *>(ws + c.o_gram[k]);
            // G = A A^T (fp32 split partials)
            GemmArgs &g = gg.p[k];
            g = seg1(r, r, md.A, d_in, md.A, d_in, d_in);
            g.mode = EPI_STORE;
            g.out = gpart;
            g.ldc = r;
            g.out_f32 = 1;
            g.splits = c.pg[k].splits;
            g.steps_per_split = c.pg[k].sps;
            fin.it[k] = GramItem{gpart, gfin, c.pg[k].splits, r};
            // W A^T row dots against B, row sums of squares of W
            GemmArgs &u = gu.p[k];
            u = seg1(d_out, r, md.W, d_in, md.A, d_in, d_in);
            u.mode = EPI_ROWDOT;
            u.E = md.B;
            u.lde = r;
            u.rowdot = cpart;
            u.rowsq = bpart;
            u.splits = c.pu[k].splits;
            u.steps_per_split = c.pu[k].sps;
            // B [G_hi ; G_lo] row dots against B
            GemmArgs &b = gbg.p[k];
            b = seg1(d_out, r, md.B, r, gfin, r, r);
            b.seg[1] = GemmSeg{md.B, r, static_cast<const uint16_t *>(gfin) + r * r, r, r};
            b.nseg = 2;
            b.mode = EPI_ROWDOT;
            b.E = md.B;
            b.lde = r;
            b.rowdot = gmpart;
            b.splits = c.pbg[k].splits;
            b.steps_per_split = c.pbg[k].sps;
            if (fuse) {
                b.fin_n = n[which[c.i0 + k]];
                b.fin_base = bpart;
                b.fin_cross = cpart;
                b.fin_z = c.pu[k].splits;
                b.fin_s = md.s;
            }
            nf.it[k] = NormFinishItem{bpart,
                                      cpart,
                                      gmpart,
                                      c.pu[k].splits,
                                      c.pu[k].splits * c.pu[k].ntn,
                                      c.pbg[k].splits * c.pbg[k].ntn,
                                      d_out,
                                      md.s,
                                      n[which[c.i0 + k]]};
        }
        DORA_LAUNCH(launch_gemm_bf16_grouped(gg, 0, c.g.cfg, false, st), "grouped gram A A^T");
        DORA_LAUNCH(launch_gram_finalize_grouped(bf, fin, st), "grouped gram finalize");
        DORA_LAUNCH(launch_gemm_bf16_grouped(gu, 0, c.u.cfg, true, st), "grouped cross W A^T");
        DORA_LAUNCH(launch_gemm_bf16_grouped(gbg, 1, c.bg.cfg, false, st), "grouped gram B G");
        if (!fuse)
            DORA_LAUNCH(launch_norm_finish_grouped(nf, st), "grouped norm finish");
    }
    return DORA_OK;
}

// Sibling modules on one input x (for instance the query, key and value
// projections): the norms as above, then per chunk one launch of all
// P = x A^T, one of the s P scalings, and one of the fused products
// [x | sP][W | B]^T with the magnitude epilogue.
struct FwdGroupChunk {
    int i0, i1;
    GroupGemm p, fused;
    std::vector<GPlan> pp, pf;
    std::vector<size_t> o_P, o_sP;
};

struct FwdGroupPlan {
    std::vector<int> need_norm;
    std::vector<NormChunk> norm;
    size_t norm_bytes = 0;
    std::vector<FwdGroupChunk> chunks;
    bool grouped = true;
    std::vector<FwdPlan> single;  // module by module when not grouped
    size_t bytes = 0;
};

FwdGroupPlan plan_forward_group(const dora_module *mods, int count, int64_t T, int dtype,
                                const float *const *n_in, void *const *P_out)
{
    FwdGroupPlan f;
    for (int i = 0; i < count; ++i)
        if (!n_in || !n_in[i])
            f.need_norm.push_back(i);
    f.need_norm = by_length(mods, f.need_norm);
    f.norm = plan_norm_group(mods, f.need_norm, dtype, f.norm_bytes);
    const size_t e = esize(dtype);
    size_t most = 0;
    for (int i0 = 0; i0 < count; i0 += kMaxGroup) {
        FwdGroupChunk c;
        c.i0 = i0;
        c.i1 = std::min(i0 + kMaxGroup, count);
        std::vector<GemmShape> sp, sf;
        for (int i = c.i0; i < c.i1; ++i) {
            const dora_module &md = mods[i];
            sp.push_back(nt_shape(T, md.r, md.d_in));
            sf.push_back(fused_shape(T, md.d_in, md.d_out, md.r));
        }
        if (dtype == DORA_BF16) {
            c.p = plan_group(sp, false);
            c.fused = plan_group(sf, false);
        }
        if (c.p.cfg < 0 || c.fused.cfg < 0)
            f.grouped = false;
        Carve cv;
        for (int k = 0; k < c.i1 - c.i0; ++k) {
            const dora_module &md = mods[c.i0 + k];
            if (c.p.cfg >= 0 && c.fused.cfg >= 0) {
                c.pp.push_back(as_gplan(c.p, sp[k]));
                c.pf.push_back(as_gplan(c.fused, sf[k]));
            }
            const bool own_P = !P_out || !P_out[c.i0 + k];
            c.o_P.push_back(own_P ? cv.take(static_cast<size_t>(T) * md.r * e) : 0);
            c.o_sP.push_back(md.s != 1.0f ? cv.take(static_cast<size_t>(T) * md.r * e) : 0);
        }
        most = std::max(most, cv.off);
        f.chunks.push_back(c);
    }
    f.bytes = align_up(f.norm_bytes) + most;
    if (!f.grouped) {
        f.bytes = 0;
        for (int i = 0; i < count; ++i) {
            f.single.push_back(plan_forward(T, mods[i].d_in, mods[i].d_out, mods[i].r, dtype));
            f.bytes = std::max(f.bytes, f.single.back().bytes);
        }
    }
    return f;
}

int forward_group_impl(const void *x, int64_t T, const dora_module *mods, int count, int dtype,
                       void *const *y, float *const *n_out, void *const *P_out,
                       const float *const *n_in, const FwdGroupPlan &f, char *ws, hipStream_t st)
{
    const bool bf = dtype == DORA_BF16;
    if (!f.grouped) {
        for (int i = 0; i < count; ++i) {
            const dora_module &md = mods[i];
            DORA_CHECK(in_module(forward_impl(x, md.W, md.A, md.B, md.m, md.s, T, md.d_in,
                                              md.d_out, md.r, dtype, y[i], n_out[i],
                                              P_out ? P_out[i] : nullptr,
                                              n_in ? n_in[i] : nullptr, f.single[i], ws, st),
                                 i));
        }
        return DORA_OK;
    }
    // 1. the norms of every module without a cached one, then the cached ones
    DORA_CHECK(norm_group_impl(mods, f.need_norm, dtype, n_out, f.norm, ws, st));
    for (int i = 0; i < count; ++i)
        if (n_in && n_in[i] && n_in[i] != n_out[i])
            DORA_LAUNCH(launch_copy_f32(n_in[i], n_out[i], mods[i].d_out, st), "copy n_in");
    if (T == 0)
        return DORA_OK;
    char *w = ws + align_up(f.norm_bytes);
    for (const FwdGroupChunk &c : f.chunks) {
        const int cnt = c.i1 - c.i0;
        GemmGroup gp, gf;
        memset(&gp, 0, sizeof gp);
        memset(&gf, 0, sizeof gf);
        gp.count = gf.count = cnt;
        std::vector<const void *> sP(cnt);
        for (int k = 0; k < cnt; ++k) {
            const int i = c.i0 + k;
            const dora_module &md = mods[i];
            const int64_t d_in = md.d_in, r = md.r;
            void *P = (P_out && P_out[i]) ? P_out[i] : static_cast<void *>(w + c.o_P[k]);
            // 2. P = x A^T
            GemmArgs &g = gp.p[k];
            g = seg1(T, r, x, d_in, md.A, d_in, d_in);
            g.mode = EPI_STORE;
            g.out = P;
            g.ldc = r;
            g.out_f32 = bf ? 0 : 1;
            g.splits = 1;
            g.steps_per_split = c.pp[k].sps;
            // 3. s P from the same sums (rounded once), unless s = 1
            sP[k] = P;
            if (md.s != 1.0f) {
                g.out2 = w + c.o_sP[k];
                g.alpha2 = md.s;
                sP[k] = w + c.o_sP[k];
            }
            // 4. y = (m/n) (x W^T + s P B^T)
            GemmArgs &h = gf.p[k];
            h = seg1(T, md.d_out, x, d_in, md.W, d_in, d_in);
            h.seg[1] = GemmSeg{sP[k], r, md.B, r, r};
            h.nseg = 2;
            h.mode = EPI_STORE;
            h.colm = md.m;
            h.coln = n_out[i];
            h.out = y[i];
            h.ldc = md.d_out;
            h.out_f32 = bf ? 0 : 1;
            h.splits = 1;
            h.steps_per_split = c.pf[k].sps;
        }
        DORA_LAUNCH(launch_gemm_bf16_grouped(gp, 0, c.p.cfg, false, st), "grouped x A^T");
        DORA_LAUNCH(launch_gemm_bf16_grouped(gf, 0, c.fused.cfg, false, st),
                    "grouped fused forward product");
    }
    return DORA_OK;
}

// Shared validation of the grouped calls' module lists.
int check_group(const dora_module *mods, int count, int dtype, bool need_m)
{
    if (count < 0)
        return fail(DORA_E_SHAPE, "count=%d is negative", count);
    if (count > 0 && !mods)
        return fail(DORA_E_NULL, "modules is NULL");
    for (int i = 0; i < count; ++i)
        DORA_CHECK(check_module(mods[i], i, dtype, need_m));
    return DORA_OK;
}

}  // namespace
}  // namespace dora

using namespace dora;

extern "C" {

const char *dora_strerror(int status)
{
    switch (status) {
    case DORA_OK: return "ok";
    case DORA_E_NULL: return "required pointer is NULL";
    case DORA_E_SHAPE: return "invalid shape";
    case DORA_E_DTYPE: return "invalid dtype";
    case DORA_E_ALIGN: return "pointer not 16-byte aligned";
    case DORA_E_WORKSPACE: return "workspace missing or too small";
    case DORA_E_ALIAS: return "buffers overlap";
    case DORA_E_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *dora_last_error(void) { return g_last_error; }

size_t dora_norm_workspace(int64_t d_out, int64_t d_in, int64_t r, int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, 0, d_in, d_out, r))
        return 0;
    Carve cv;
    return plan_norm(d_out, d_in, r, dtype, cv).bytes;
}

size_t dora_forward_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, T, d_in, d_out, r))
        return 0;
    return plan_forward(T, d_in, d_out, r, dtype).bytes;
}

size_t dora_backward_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, T, d_in, d_out, r))
        return 0;
    return plan_backward(T, d_in, d_out, r, dtype).bytes;
}

int dora_factored_norm(const void *W, const void *A, const void *B, float s, int64_t d_out,
                       int64_t d_in, int64_t r, int dtype, float *n, float *base, float *cross,
                       float *gram, float *U_out, void *ws, size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, 0, d_in, d_out, r));
    DORA_CHECK(check_ptrs({{W, "W", true}, {A, "A", true}, {B, "B", true}, {n, "n", true},
                           {base, "base", false}, {cross, "cross", false}, {gram, "gram", false},
                           {U_out, "U_out", false}}));
    Carve cv;
    const NormPlan p = plan_norm(d_out, d_in, r, dtype, cv);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const size_t e = esize(dtype);
    const Range rW{W, d_out * d_in * e}, rA{A, r * d_in * e}, rB{B, d_out * r * e};
    const Range rws{ws, p.bytes};
    const size_t v = d_out * 4;
    DORA_CHECK(check_disjoint({{{n, v}, "n"}, {{base, v}, "base"}, {{cross, v}, "cross"},
                               {{gram, v}, "gram"}, {{U_out, static_cast<size_t>(d_out * r * 4)}, "U_out"},
                               {rws, "workspace"}},
                              {{rW, "W"}, {rA, "A"}, {rB, "B"}}));
    return norm_impl(W, A, B, s, d_out, d_in, r, dtype, n, base, cross, gram, p,
                     static_cast<char *>(ws), static_cast<hipStream_t>(stream), U_out);
}

int dora_compose(const void *base, const void *lora, const float *m, const float *n, float s,
                 int64_t T, int64_t d_out, int dtype, void *y, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    if (T < 0 || T > kMaxDim || d_out < 0 || d_out > kMaxDim)
        return fail(DORA_E_SHAPE, "T=%lld, d_out=%lld out of range", (long long)T,
                    (long long)d_out);
    const bool any = T > 0 && d_out > 0;  // empty tensors may come with NULL data
    DORA_CHECK(check_ptrs({{base, "base", any}, {lora, "lora", any}, {m, "m", d_out > 0},
                           {n, "n", d_out > 0}, {y, "y", any}}));
    const size_t bytes = static_cast<size_t>(T) * d_out * esize(dtype);
    if (y != base && overlap({y, bytes}, {base, bytes}))
        return fail(DORA_E_ALIAS, "y partially overlaps base");
    DORA_CHECK(check_disjoint({{{y, bytes}, "y"}},
                              {{{lora, bytes}, "lora"}, {{m, d_out * sizeof(float)}, "m"},
                               {{n, d_out * sizeof(float)}, "n"}}));
    DORA_LAUNCH(launch_compose(dtype == DORA_BF16, base, lora, m, n, s, T, d_out, y,
                               static_cast<hipStream_t>(stream)),
                "compose");
    return DORA_OK;
}

int dora_forward(const void *x, const void *W, const void *A, const void *B, const float *m,
                 float s, int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype, void *y,
                 float *n_out, void *P_out, const float *n_in, float *U_out, void *ws,
                 size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, T, d_in, d_out, r));
    const bool has_t = T > 0;  // empty tensors may come with NULL data
    DORA_CHECK(check_ptrs({{x, "x", has_t}, {W, "W", true}, {A, "A", true}, {B, "B", true},
                           {m, "m", true}, {y, "y", has_t}, {n_out, "n_out", true},
                           {P_out, "P_out", false}, {n_in, "n_in", false},
                           {U_out, "U_out", false}}));
    if (U_out && n_in)
        return fail(DORA_E_NULL, "U_out needs the norm computed here (n_in must be NULL)");
    const FwdPlan p = plan_forward(T, d_in, d_out, r, dtype);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const size_t e = esize(dtype);
    const Range rx{x, T * d_in * e}, rW{W, d_out * d_in * e}, rA{A, r * d_in * e},
        rB{B, d_out * r * e}, rm{m, d_out * sizeof(float)}, rnin{n_in, d_out * sizeof(float)};
    const Range ry{y, T * d_out * e}, rn{n_out, d_out * sizeof(float)}, rP{P_out, T * r * e}, rws{ws, p.bytes};
    const Range rU{U_out, static_cast<size_t>(d_out * r * 4)};
    if (n_in && n_in != n_out && overlap(rn, rnin))
        return fail(DORA_E_ALIAS, "n_out partially overlaps n_in");
    DORA_CHECK(check_disjoint({{ry, "y"}, {rn, "n_out"}, {rP, "P_out"}, {rU, "U_out"},
                               {rws, "workspace"}},
                              {{rx, "x"}, {rW, "W"}, {rA, "A"}, {rB, "B"}, {rm, "m"}}));
    DORA_CHECK(check_disjoint({{ry, "y"}, {rP, "P_out"}, {rws, "workspace"}}, {{rnin, "n_in"}}));

    return forward_impl(x, W, A, B, m, s, T, d_in, d_out, r, dtype, y, n_out, P_out, n_in, p,
                        static_cast<char *>(ws), static_cast<hipStream_t>(stream), U_out);
}

int dora_backward(const void *dy, const void *x, const void *W, const void *A, const void *B,
                  const float *m, const float *n, float s, const void *P, const void *y,
                  int64_t T, int64_t d_in, int64_t d_out, int64_t r, int dtype, void *dx, void *dA,
                  void *dB, float *dm, void *ws, size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, T, d_in, d_out, r));
    const bool has_t = T > 0;
    DORA_CHECK(check_ptrs({{dy, "dy", has_t}, {x, "x", has_t}, {W, "W", true}, {A, "A", true},
                           {B, "B", true}, {m, "m", true}, {n, "n", true}, {P, "P", has_t},
                           {y, "y", has_t}, {dx, "dx", has_t}, {dA, "dA", true}, {dB, "dB", true},
                           {dm, "dm", true}}));
    const BwdPlan p = plan_backward(T, d_in, d_out, r, dtype);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const bool bf = dtype == DORA_BF16;
    const size_t e = esize(dtype);
    DORA_CHECK(check_disjoint(
        {{{dx, T * d_in * e}, "dx"}, {{dA, r * d_in * e}, "dA"}, {{dB, d_out * r * e}, "dB"},
         {{dm, d_out * sizeof(float)}, "dm"}, {{ws, p.bytes}, "workspace"}},
        {{{dy, T * d_out * e}, "dy"}, {{x, T * d_in * e}, "x"}, {{W, d_out * d_in * e}, "W"},
         {{A, r * d_in * e}, "A"}, {{B, d_out * r * e}, "B"}, {{m, d_out * sizeof(float)}, "m"},
         {{n, d_out * sizeof(float)}, "n"}, {{P, T * r * e}, "P"}, {{y, T * d_out * e}, "y"}}));

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    void *dh = w + p.o_dh;
    float *dmpart = reinterpret_cast<float *>(w + p.o_dmpart);
    void *Q = w + p.o_Q;

    // 1. dh = g dy and dm partial sums (one pass over dy and y), then dm;
    //    with the fused plan the same pass also forms dB = s dh^T P.
    if (p.fused_dhdm) {
        float *part = reinterpret_cast<float *>(w + p.o_dBpart);
        const bool split = p.dB.splits > 1;
        DORA_CHECK(run_dhdm_dB(p, dy, y, m, n, P, T, d_out, r, dh, dmpart, split ? part : dB,
                               split ? 1 : 0, split ? 1.0f : s, st));
        if (split)
            DORA_LAUNCH(launch_splitk_reduce(bf, part, p.dB.splits, d_out, r, s, dB, st), "dB");
    } else {
        DORA_LAUNCH(launch_dh_dm_partial(bf, dy, y, m, n, T, d_out, p.sweep, dh, dmpart, st),
                    "dh/dm");
    }
    DORA_LAUNCH(launch_dm_finish(dmpart, p.nchunks, m, d_out, dm, st), "dm finish");
    // 2. Q = s dh B  (A K-major, B MN-major).
    DORA_CHECK(run_store(bf, p.q, seg1(T, r, dh, d_out, B, r, d_out), 1, Q, r, s,
                         reinterpret_cast<float *>(w + p.o_Qpart), st, "Q = s dh B"));
    // 3. dx = [dh | Q] [W ; A]  (K-concatenated segments, B MN-major).
    {
        GemmArgs g = seg1(T, d_in, dh, d_out, W, d_in, d_out);
        g.seg[1] = GemmSeg{Q, r, A, d_in, r};
        g.nseg = 2;
        DORA_CHECK(run_store(bf, p.dx, g, 1, dx, d_in, 1.0f,
                             reinterpret_cast<float *>(w + p.o_dxpart), st, "dx"));
    }
    // 4. dB = s dh^T P  (both MN-major, K = T), unless formed in step 1.
    if (!p.fused_dhdm)
        DORA_CHECK(run_store(bf, p.dB, seg1(d_out, r, dh, d_out, P, r, T), 2, dB, r, s,
                             reinterpret_cast<float *>(w + p.o_dBpart), st, "dB"));
    // 5. dA = Q^T x  (both MN-major, K = T).
    DORA_CHECK(run_store(bf, p.dA, seg1(r, d_in, Q, r, x, d_in, T), 2, dA, d_in, 1.0f,
                         reinterpret_cast<float *>(w + p.o_dApart), st, "dA"));
    return DORA_OK;
}

size_t dora_backward_through_norm_workspace(int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                            int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, T, d_in, d_out, r))
        return 0;
    return plan_through_norm(T, d_in, d_out, r, dtype).bytes;
}

int dora_backward_through_norm(const void *dy, const void *x, const void *W, const void *A,
                               const void *B, const float *m, const float *n, float s,
                               const void *P, const void *y, const float *U, int64_t T,
                               int64_t d_in, int64_t d_out, int64_t r, int dtype, void *dx,
                               void *dA, void *dB, float *dm, void *ws, size_t ws_bytes,
                               void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, T, d_in, d_out, r));
    const bool has_t = T > 0;
    DORA_CHECK(check_ptrs({{dy, "dy", has_t}, {x, "x", has_t}, {W, "W", true}, {A, "A", true},
                           {B, "B", true}, {m, "m", true}, {n, "n", true}, {P, "P", has_t},
                           {y, "y", has_t}, {dx, "dx", has_t}, {dA, "dA", true}, {dB, "dB", true},
                           {dm, "dm", true}, {U, "U", false}}));
    const ThruPlan p = plan_through_norm(T, d_in, d_out, r, dtype);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const bool bf = dtype == DORA_BF16;
    const size_t e = esize(dtype);
    DORA_CHECK(check_disjoint(
        {{{dx, T * d_in * e}, "dx"}, {{dA, r * d_in * e}, "dA"}, {{dB, d_out * r * e}, "dB"},
         {{dm, d_out * sizeof(float)}, "dm"}, {{ws, p.bytes}, "workspace"}},
        {{{dy, T * d_out * e}, "dy"}, {{x, T * d_in * e}, "x"}, {{W, d_out * d_in * e}, "W"},
         {{A, r * d_in * e}, "A"}, {{B, d_out * r * e}, "B"}, {{m, d_out * sizeof(float)}, "m"},
         {{n, d_out * sizeof(float)}, "n"}, {{P, T * r * e}, "P"}, {{y, T * d_out * e}, "y"},
         {{U, d_out * r * sizeof(float)}, "U"}}));

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    const BwdPlan &b = p.b;
    void *dh = w + b.o_dh;
    float *dmpart = reinterpret_cast<float *>(w + b.o_dmpart);
    void *Q = w + b.o_Q;
    float *cs = reinterpret_cast<float *>(w + p.o_cs);
    void *cB = w + p.o_cB;
    float *aslots = reinterpret_cast<float *>(w + p.o_aslots);
    float *bslots = reinterpret_cast<float *>(w + p.o_bslots);
    float *yslots = reinterpret_cast<float *>(w + p.o_yslots);
    const size_t gsz = bf ? static_cast<size_t>(r) * r * 2 : 0;  // lo half of a hi/lo pair

    // 1-3. As with n held constant: dh = g dy and dm (with the fused plan the
    //      same pass also puts s dh^T P into dB's fp32 slots), Q = s dh B,
    //      dx = [dh | Q] [W ; A].
    if (b.fused_dhdm)
        DORA_CHECK(run_dhdm_dB(b, dy, y, m, n, P, T, d_out, r, dh, dmpart, bslots, 1, s, st));
    else
        DORA_LAUNCH(launch_dh_dm_partial(bf, dy, y, m, n, T, d_out, b.sweep, dh, dmpart, st),
                    "dh/dm");
    DORA_LAUNCH(launch_dm_finish(dmpart, b.nchunks, m, d_out, dm, st), "dm finish");
    DORA_CHECK(run_store(bf, b.q, seg1(T, r, dh, d_out, B, r, d_out), 1, Q, r, s,
                         reinterpret_cast<float *>(w + b.o_Qpart), st, "Q = s dh B"));
    {
        GemmArgs g = seg1(T, d_in, dh, d_out, W, d_in, d_out);
        g.seg[1] = GemmSeg{Q, r, A, d_in, r};
        g.nseg = 2;
        DORA_CHECK(run_store(bf, b.dx, g, 1, dx, d_in, 1.0f,
                             reinterpret_cast<float *>(w + b.o_dxpart), st, "dx"));
    }
    // 4. The norm's row coefficient cs = -s m dm / n^2 and cB = cs (.) B.
    DORA_LAUNCH(launch_norm_grad_coef(bf, m, dm, n, s, B, d_out, r, cs, cB, st), "norm grad coef");
    // 5. dA = [Q^T | cB^T] [x ; W] + s (cB^T B) A.
    {
        GemmArgs g = seg1(r, d_in, cB, r, W, d_in, d_out);
        if (T > 0) {
            g.seg[1] = g.seg[0];
            g.seg[0] = GemmSeg{Q, r, x, d_in, T};
            g.nseg = 2;
        }
        DORA_CHECK(run_slots(bf, p.da, g, 2, aslots, 1.0f, st, "dA: Q^T x + cB^T W"));
        float *gspart = reinterpret_cast<float *>(w + p.o_gspart);
        char *gs = w + p.o_gsfin;
        DORA_CHECK(run_slots(bf, p.gs, seg1(r, r, cB, r, B, r, d_out), 2, gspart, 1.0f, st,
                             "dA: cB^T B"));
        DORA_LAUNCH(launch_gram_finalize(bf, gspart, p.gs.splits, r, gs, st), "dA: cB^T B sum");
        GemmArgs z = seg1(r, d_in, gs, r, A, d_in, r);
        if (bf) {
            z.seg[1] = GemmSeg{gs + gsz, r, A, d_in, r};
            z.nseg = 2;
        }
        DORA_CHECK(run_slots(bf, p.z, z, 1, aslots + static_cast<size_t>(p.da.splits) * r * d_in,
                             s, st, "dA: s (cB^T B) A"));
        DORA_LAUNCH(launch_combine_rows(bf, aslots, p.da.splits,
                                        aslots + static_cast<size_t>(p.da.splits) * r * d_in,
                                        p.z.splits, nullptr, r, d_in, dA, st),
                    "dA combine");
    }
    // 6. dB = s dh^T P + cs (.) V A^T,  V A^T = W A^T + s B G,  G = A A^T.
    {
        if (!b.fused_dhdm)
            DORA_CHECK(run_slots(bf, b.dB, seg1(d_out, r, dh, d_out, P, r, T), 2, bslots, s, st,
                                 "dB: s dh^T P"));
        // V A^T = W A^T + s B G: the norm's own product when the caller kept it
        // (U), else formed here
        if (!U) {
            float *gpart = reinterpret_cast<float *>(w + p.o_gpart);
            char *G = w + p.o_gfin;
            DORA_CHECK(run_slots(bf, p.g, seg1(r, r, A, d_in, A, d_in, d_in), 0, gpart, 1.0f,
                                 st, "dB: A A^T"));
            DORA_LAUNCH(launch_gram_finalize(bf, gpart, p.g.splits, r, G, st), "dB: A A^T sum");
            DORA_CHECK(run_slots(bf, p.y1, seg1(d_out, r, W, d_in, A, d_in, d_in), 0, yslots,
                                 1.0f, st, "dB: W A^T"));
            GemmArgs g = seg1(d_out, r, B, r, G, r, r);
            if (bf) {
                g.seg[1] = GemmSeg{B, r, G + gsz, r, r};
                g.nseg = 2;
            }
            DORA_CHECK(run_slots(bf, p.y2, g, 1,
                                 yslots + static_cast<size_t>(p.y1.splits) * d_out * r, s, st,
                                 "dB: s B G"));
        }
        DORA_LAUNCH(launch_combine_rows(bf, bslots, p.nb, yslots, U ? 0 : p.ny, cs, d_out, r, dB,
                                        st, U),
                    "dB combine");
    }
    return DORA_OK;
}

size_t dora_factored_norm_grouped_workspace(const dora_module *mods, int count, int dtype)
{
    if (check_dtype(dtype) || check_group(mods, count, dtype, false))
        return 0;
    std::vector<int> all(count);
    for (int i = 0; i < count; ++i)
        all[i] = i;
    all = by_length(mods, all);
    size_t bytes = 0;
    plan_norm_group(mods, all, dtype, bytes);
    return bytes;
}

int dora_factored_norm_grouped(const dora_module *mods, int count, int dtype, float *const *n,
                               void *ws, size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_group(mods, count, dtype, false));
    if (count == 0)
        return DORA_OK;
    if (!n)
        return fail(DORA_E_NULL, "n is NULL");
    std::vector<int> all(count);
    for (int i = 0; i < count; ++i)
        all[i] = i;
    all = by_length(mods, all);
    size_t bytes = 0;
    const std::vector<NormChunk> chunks = plan_norm_group(mods, all, dtype, bytes);
    DORA_CHECK(check_ws(ws, ws_bytes, bytes));
    const size_t e = esize(dtype);
    const Range rws{ws, bytes};
    for (int i = 0; i < count; ++i) {
        const dora_module &md = mods[i];
        DORA_CHECK(in_module(check_ptrs({{n[i], "n", true}}), i));
        const Range rn{n[i], md.d_out * sizeof(float)};
        DORA_CHECK(in_module(check_disjoint({{rws, "workspace"}},
                                            {{{md.W, md.d_out * md.d_in * e}, "W"},
                                             {{md.A, md.r * md.d_in * e}, "A"},
                                             {{md.B, md.d_out * md.r * e}, "B"}, {rn, "n"}}),
                             i));
        for (int j = 0; j < count; ++j) {
            const dora_module &mj = mods[j];
            DORA_CHECK(in_module(check_disjoint({{rn, "n"}},
                                                {{{mj.W, mj.d_out * mj.d_in * e}, "a W"},
                                                 {{mj.A, mj.r * mj.d_in * e}, "an A"},
                                                 {{mj.B, mj.d_out * mj.r * e}, "a B"}}),
                                 i));
            if (j > i && overlap(rn, {n[j], mj.d_out * sizeof(float)}))
                return fail(DORA_E_ALIAS, "n of modules %d and %d overlap", i, j);
        }
    }
    return norm_group_impl(mods, all, dtype, n, chunks, static_cast<char *>(ws),
                           static_cast<hipStream_t>(stream));
}

size_t dora_forward_grouped_workspace(const dora_module *mods, int count, int64_t T,
                                      int dtype, const float *const *n_in,
                                      void *const *P_out)
{
    if (check_dtype(dtype) || check_group(mods, count, dtype, true) ||
        check_dims(dtype, T, 8, 8, 8))
        return 0;
    return plan_forward_group(mods, count, T, dtype, n_in, P_out).bytes;
}

int dora_forward_grouped(const void *x, int64_t T, int64_t d_in, const dora_module *mods,
                         int count, int dtype, void *const *y, float *const *n_out,
                         void *const *P_out, const float *const *n_in, void *ws, size_t ws_bytes,
                         void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_group(mods, count, dtype, true));
    DORA_CHECK(check_dims(dtype, T, d_in, 8, 8));
    if (count == 0)
        return DORA_OK;
    const bool has_t = T > 0;
    DORA_CHECK(check_ptrs({{x, "x", has_t}}));
    if (!n_out || (has_t && !y))
        return fail(DORA_E_NULL, "%s is NULL", !n_out ? "n_out" : "y");
    const FwdGroupPlan f = plan_forward_group(mods, count, T, dtype, n_in, P_out);
    DORA_CHECK(check_ws(ws, ws_bytes, f.bytes));
    const size_t e = esize(dtype);
    const Range rx{x, T * d_in * e}, rws{ws, f.bytes};
    // every output of every module is disjoint from every input and from the
    // other outputs (a cached n may be its own n_out)
    std::vector<Named> outs, ins;
    outs.push_back({rws, "workspace"});
    ins.push_back({rx, "x"});
    for (int i = 0; i < count; ++i) {
        const dora_module &md = mods[i];
        if (md.d_in != d_in)
            return fail(DORA_E_SHAPE, "module %d: d_in=%lld, x has %lld", i, (long long)md.d_in,
                        (long long)d_in);
        void *Pi = P_out ? P_out[i] : nullptr;
        const float *ni = n_in ? n_in[i] : nullptr;
        DORA_CHECK(in_module(check_ptrs({{y ? y[i] : nullptr, "y", has_t},
                                         {n_out[i], "n_out", true}, {Pi, "P_out", false},
                                         {ni, "n_in", false}}),
                             i));
        outs.push_back({{y ? y[i] : nullptr, T * md.d_out * e}, "a y"});
        outs.push_back({{n_out[i], md.d_out * sizeof(float)}, "an n_out"});
        outs.push_back({{Pi, T * md.r * e}, "a P_out"});
        ins.push_back({{md.W, md.d_out * d_in * e}, "a W"});
        ins.push_back({{md.A, md.r * d_in * e}, "an A"});
        ins.push_back({{md.B, md.d_out * md.r * e}, "a B"});
        ins.push_back({{md.m, md.d_out * sizeof(float)}, "an m"});
        if (ni && ni != n_out[i])
            ins.push_back({{ni, md.d_out * sizeof(float)}, "an n_in"});
    }
    for (size_t a = 0; a < outs.size(); ++a) {
        for (size_t b = a + 1; b < outs.size(); ++b)
            if (overlap(outs[a].r, outs[b].r))
                return fail(DORA_E_ALIAS, "%s overlaps %s", outs[a].name, outs[b].name);
        for (const Named &q : ins)
            if (overlap(outs[a].r, q.r))
                return fail(DORA_E_ALIAS, "%s overlaps %s", outs[a].name, q.name);
    }
    return forward_group_impl(x, T, mods, count, dtype, y, n_out, P_out, n_in, f,
                              static_cast<char *>(ws), static_cast<hipStream_t>(stream));
}

size_t dora_merge_workspace(int64_t d_out, int64_t d_in, int64_t r, int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, 0, d_in, d_out, r))
        return 0;
    return plan_merge(d_out, d_in, r, dtype).bytes;
}

int dora_merge(const void *W, const void *A, const void *B, const float *m, float s,
               int64_t d_out, int64_t d_in, int64_t r, int dtype, const float *n_in, void *W_out,
               void *ws, size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, 0, d_in, d_out, r));
    DORA_CHECK(check_ptrs({{W, "W", true}, {A, "A", true}, {B, "B", true}, {m, "m", true},
                           {W_out, "W_out", true}, {n_in, "n_in", false}}));
    const MergePlan p = plan_merge(d_out, d_in, r, dtype);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const bool bf = dtype == DORA_BF16;
    const size_t e = esize(dtype);
    const Range rW{W, d_out * d_in * e}, rA{A, r * d_in * e}, rB{B, d_out * r * e},
        rm{m, d_out * sizeof(float)}, rnin{n_in, d_out * sizeof(float)};
    const Range rout{W_out, d_out * d_in * e}, rws{ws, p.bytes};
    if (W_out != W && overlap(rout, rW))
        return fail(DORA_E_ALIAS, "W_out partially overlaps W");
    DORA_CHECK(check_disjoint({{rout, "W_out"}, {rws, "workspace"}},
                              {{rA, "A"}, {rB, "B"}, {rm, "m"}, {rnin, "n_in"}}));
    DORA_CHECK(check_disjoint({{rws, "workspace"}}, {{rW, "W"}, {rout, "W_out"}}));

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    const float *n = n_in;
    if (n == nullptr) {
        float *nw = reinterpret_cast<float *>(w + p.o_n);
        DORA_CHECK(norm_impl(W, A, B, s, d_out, d_in, r, dtype, nw, nullptr, nullptr, nullptr,
                             p.norm, w, st));
        n = nw;
    }
    GemmArgs g = seg1(d_out, d_in, B, r, A, d_in, r);
    g.mode = EPI_MERGE;
    g.E = W;
    g.lde = d_in;
    g.colm = m;
    g.coln = n;
    g.alpha = s;
    g.out = W_out;
    g.ldc = d_in;
    DORA_LAUNCH(run_gemm(bf, p.g, g, 1, false, st), "merge W + s B A");
    return DORA_OK;
}

size_t dora_linear_workspace(int64_t T, int64_t d_in, int64_t d_out, int dtype)
{
    if (check_dtype(dtype) || check_dims(dtype, T, d_in, d_out, 8))
        return 0;
    return plan_linear(T, d_in, d_out, dtype).bytes;
}

int dora_linear(const void *x, const void *W, int64_t T, int64_t d_in, int64_t d_out, int dtype,
                void *y, void *ws, size_t ws_bytes, void *stream)
{
    g_last_error[0] = '\0';
    DORA_CHECK(check_dtype(dtype));
    DORA_CHECK(check_dims(dtype, T, d_in, d_out, 8));
    const bool has_t = T > 0;
    DORA_CHECK(check_ptrs({{x, "x", has_t}, {W, "W", true}, {y, "y", has_t}}));
    const LinPlan p = plan_linear(T, d_in, d_out, dtype);
    DORA_CHECK(check_ws(ws, ws_bytes, p.bytes));
    const size_t e = esize(dtype);
    DORA_CHECK(check_disjoint({{{y, T * d_out * e}, "y"}, {{ws, p.bytes}, "workspace"}},
                              {{{x, T * d_in * e}, "x"}, {{W, d_out * d_in * e}, "W"}}));
    if (T == 0)
        return DORA_OK;
    return run_store(dtype == DORA_BF16, p.g, seg1(T, d_out, x, d_in, W, d_in, d_in), 0, y, d_out,
                     1.0f, static_cast<float *>(ws), static_cast<hipStream_t>(stream),
                     "linear x W^T");
}

}  // extern "C"
