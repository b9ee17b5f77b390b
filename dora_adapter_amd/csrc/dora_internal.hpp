// dora_internal.hpp - types shared by the HIP kernels and the C-ABI layer of
// libdora.so (gfx950).  Not part of the public interface (include/dora.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

// ---------------------------------------------------------------- GEMM plan
// C[M, N] = sum over segments of op(A_seg) * op(B_seg), accumulated in fp32.
// A_seg is K-major ([M][lda], K contiguous) or MN-major ([K][lda], M
// contiguous); likewise B_seg ([N][ldb] or [K][ldb]).  Up to two segments
// are concatenated along K (e.g. dx = [dh | Q] [W ; A]).  Each segment's K
// range is walked in BK-wide steps with the tail zero-filled, and split-K
// slices the concatenated step list into `splits` contiguous ranges
// (blockIdx.y).
struct GemmSeg {
    const void *a;
    int64_t lda;
    const void *b;
    int64_t ldb;
    int64_t K;
};

enum EpiMode : int {
    EPI_STORE = 0,   // out[m, n] = alpha * C (dtype of the kernel or fp32), split z at out + z*M*ldc
    EPI_ROWDOT = 1,  // rowdot[(z*ntn + tn)*M + m] = sum_{n in tile} C[m, n] * E[m, n];
                     // with out set, C itself as well (fp32, split z at out + z*M*ldc)
    // out[m, n] = E[m, n] + ((g_m - 1) E[m, n] + g_m alpha C[m, n]), g_m =
    // colm[m] / coln[m] (row factors here), rounded once; one split only
    EPI_MERGE = 2,
};

struct GemmArgs {
    int64_t M, N;
    GemmSeg seg[2];
    int nseg;
    int splits;
    int64_t steps_per_split;  // BK-steps per split slice
    int mode;
    // EPI_STORE
    void *out;
    int64_t ldc;
    int out_f32;             // 1: fp32 output (split-K partials); 0: kernel dtype
    // fp32 output only: 1 adds to what `out` holds instead of overwriting
    // it (one writer per element: unsplit products only)
    int out_accum;
    float alpha;
    // EPI_STORE, unsplit only: an optional second output of the same type,
    // layout and ldc receiving alpha2 * C, rounded once (the forward's P and
    // s P from one accumulator); with out2_lo (bf16 only) it receives instead
    // the rounding residual C - bf16(C) of the first output, rounded to bf16
    // (the Gram matrix's hi / lo pair)
    //
    // EPI_ROWDOT on the direct-to-LDS kernels whose row dots come from the
    // accumulators, unsplit and one N tile (the norm's B G, whose row dot is
    // the whole Gram term): with fin_n set, the same fields instead carry the
    // norm's finish, n[m] = norm_from_terms(sum_z fin_base[z M + m],
    // sum_z fin_cross[z M + m], rowdot of row m, fin_s) over z < fin_z.
    union {
        void *out2;
        float *fin_n;
    };
    union {
        float alpha2;
        float fin_s;
    };
    union {
        int out2_lo;
        int fin_z;
    };
    // optional per-column magnitude scale of the store: with colm and coln
    // set, column n of alpha * C is stored as h + ((colm[n] - coln[n]) /
    // coln[n]) h, i.e. (m/n) h in the cancellation-safe form (EPI_MERGE:
    // per-row factors)
    union {
        const float *colm;
        const float *fin_base;
    };
    union {
        const float *coln;
        const float *fin_cross;
    };
    // EPI_ROWDOT, EPI_MERGE: E (ld lde); EPI_ROWDOT: rowdot; and an
    // optional sum of squares of A's rows over each split's K range (K-major
    // A only; written by the tiles of the first N block): rowsq[z*M + m].
    // dh/dm production (launch_gemm_bf16_dhdm, an EPI_STORE product) uses
    // the same places for y in A's layout, the raw dm sums dm_part[z*M + m]
    // and the dh output (A's layout and lda), with g_m = dh_m[m] / dh_n[m]
    // for A's index m.
    union {
        const void *E;
        const void *Y;
    };
    int64_t lde;
    union {
        float *rowdot;
        float *dm_part;
    };
    union {
        float *rowsq;
        void *dh_out;
    };
    const float *dh_m, *dh_n;
};

// n = sqrt(max(base + 2 s cross + s^2 gram, 0)) from the three terms of the
// factored norm, in fp64 (the finish kernel and the fused B G epilogue).
__device__ __forceinline__ float norm_from_terms(double b, double c, double g, float s)
{
    const double sd = static_cast<double>(s);
    double n2 = b + 2.0 * sd * c + sd * sd * g;
    if (n2 < 0.0)
        n2 = 0.0;
    return static_cast<float>(sqrt(n2));
}

// Up to kMaxGroup independent products in one launch (passed by value as the
// kernel argument, so no descriptor table lives in device memory).  Every
// problem uses the launch's tile configuration and operand layout; problem
// p owns the linear workgroup ids [tile_start[p], tile_start[p + 1]), i.e.
// its tiles times its splits.
constexpr int kMaxGroup = 16;
struct GemmGroup {
    GemmArgs p[kMaxGroup];
    int tile_start[kMaxGroup + 1];
    int count;
    // 0: each XCD takes a contiguous run of the linear workgroup ids (L2
    // locality between neighbouring tiles); 1: ids in dispatch order, dealt
    // to the XCDs in turn, so that every problem spreads over all of them
    // (for problems whose tiles share no operand rows)
    int spread;
};
static_assert(sizeof(GemmGroup) <= 4096, "a group must fit the kernel argument space");

// Launchers (gemm_bf16.hip / gemm_f32.hip).  `layout` selects the operand
// orders: 0 = A K-major, B K-major (C = A B^T); 1 = A K-major, B MN-major
// (C = A B); 2 = A MN-major, B MN-major (C = A^T B).  `cfg` picks the tile
// shape (see gemm_configs in the .hip file).
hipError_t launch_gemm_bf16(const GemmArgs &a, int layout, int cfg, bool rowsq, hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs &a, int layout, bool rowsq, hipStream_t st);
// The backward's dB = alpha dh^T P with dh = g (.) dy and the dm sums formed
// in the same pass (both operands MN-major, one segment: a.seg[0].a = dy,
// a.seg[0].b = P; a.Y, a.dh_out, a.dm_part, a.dh_m / a.dh_n set).  Only the
// configurations with dhdm_ok take it.
hipError_t launch_gemm_bf16_dhdm(const GemmArgs &a, int cfg, hipStream_t st);
// Grouped launch of the pipelined bf16 kernel (cfg must be a direct-to-LDS
// configuration); tile_start and count are filled in here from the problems'
// shapes and splits.
hipError_t launch_gemm_bf16_grouped(GemmGroup &g, int layout, int cfg, bool rowsq, hipStream_t st);

// Tile configurations of the bf16 MFMA GEMM, indexable by `cfg`.  Two
// kernels: the general one (any shape, operands staged through registers, K
// step 64) and the pipelined direct-to-LDS one (K stage 64; K-major operands
// need K % 8 == 0, and every operand must stay under 2 GiB).
struct TileCfg {
    int BM, BN;
    int bk;           // K values per step
    bool dma;         // pipelined direct-to-LDS kernel
    float rel_speed;  // relative throughput of a full tile, for planning
    bool store_ok;    // EPI_STORE supported (else EPI_ROWDOT only)
    bool rowsq_ok;    // row sums of squares of A supported
    bool direct_rowdot;  // EPI_ROWDOT formed from the accumulators (no LDS staging)
    bool ragged_ok;      // also takes operands of any width (element-masked loads)
    bool dhdm_ok;        // has the dh/dm-producing variant (launch_gemm_bf16_dhdm)
};
int gemm_bf16_num_cfgs();
TileCfg gemm_bf16_cfg(int cfg);
constexpr int GEMM_BK = 64;      // bf16 K step of the general kernel
constexpr int GEMM_DMA_BK = 64;  // bf16 K stage of the direct-to-LDS kernel
constexpr int GEMM_F32_BM = 64;  // fp32 VALU tile
constexpr int GEMM_F32_BN = 64;
constexpr int GEMM_F32_BK = 16;

// Elementwise / reduction kernels (elementwise.hip).  `bf16` selects the
// matrix element type (1: bf16, 0: fp32).
hipError_t launch_compose(int bf16, const void *base, const void *lora, const float *m,
                          const float *n, float s, int64_t T, int64_t d_out, void *y,
                          hipStream_t st);
// out = alpha * sum_z part[z] (fixed order); with colm/coln set, column n is
// then scaled as h + ((colm[n] - coln[n]) / coln[n]) h before the rounding.
// With out2 set, out2 = alpha2 * sum_z part[z] as well (one rounding each).
hipError_t launch_splitk_reduce(int bf16, const float *part, int splits, int64_t M, int64_t N,
                                float alpha, void *out, hipStream_t st,
                                const float *colm = nullptr, const float *coln = nullptr,
                                void *out2 = nullptr, float alpha2 = 1.0f);
hipError_t launch_gram_finalize(int bf16, const float *part, int splits, int64_t r, void *G_out,
                                hipStream_t st);
hipError_t launch_norm_finish(const float *base_part, int zb, const float *cross_part, int zc,
                              const float *gram_part, int zg, int64_t d_out, float s, float *n,
                              float *base, float *cross, float *gram, hipStream_t st);
hipError_t launch_dh_dm_partial(int bf16, const void *dy, const void *y, const float *m,
                                const float *n, int64_t T, int64_t d_out, int64_t sweep,
                                void *dh, float *dm_part, hipStream_t st);
hipError_t launch_dm_finish(const float *dm_part, int nchunks, const float *m, int64_t d_out,
                            float *dm, hipStream_t st);
// Backward through the norm: cs = -s m dm / n^2 per row and cB = cs (.) B.
hipError_t launch_norm_grad_coef(int bf16, const float *m, const float *dm, const float *n, float s,
                                 const void *B, int64_t d_out, int64_t r, float *cs, void *cB,
                                 hipStream_t st);
// out = sum_z part[z] + rowscale (.) (y0 + sum_u ypart[u]) ([M, N] fp32 slots;
// rowscale nullable = 1, y0 nullable = 0), fixed order, rounded once to the
// element type.
hipError_t launch_combine_rows(int bf16, const float *part, int np, const float *ypart, int ny,
                               const float *rowscale, int64_t M, int64_t N, void *out,
                               hipStream_t st, const float *y0 = nullptr);
// Grouped small kernels: one launch over up to kMaxGroup modules (items
// passed by value; blockIdx.y selects the item), the same arithmetic as the
// single-module launchers.
template <typename Item>
struct ItemGroup {
    Item it[kMaxGroup];
    int count;
};
struct GramItem {
    const float *part;
    void *G;
    int splits;
    int64_t r;
};
struct NormFinishItem {
    const float *bp, *cp, *gp;
    int zb, zc, zg;
    int64_t d_out;
    float s;
    float *n;
};
hipError_t launch_gram_finalize_grouped(int bf16, const ItemGroup<GramItem> &g, hipStream_t st);
hipError_t launch_norm_finish_grouped(const ItemGroup<NormFinishItem> &g, hipStream_t st);
hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t st);
hipError_t launch_fill_f32(float *dst, float v, int64_t n, hipStream_t st);

// The thread-local message dora_last_error() returns (dora_api.cpp): set it
// and return `status`, or clear it.
int set_error(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// dh/dm pass: rows per sweep of the grid, which is also the number of dm
// partial sums per column (thread t0 sums rows t0, t0 + sweep, ...).
int64_t dm_sweep_rows(int64_t T, int64_t d_out);

}  // namespace dora
