// elementwise.hip - the HBM-bound kernels of the DoRA module (gfx950).
//
//   compose      y = base + ((g - 1) base + g s lora), g = m / n: the single
//                pass with the cancellation-safe near-unity form ("Scaling
//                DoRA" abstract, fused compose).  6 bytes per bf16 element.
//   dh / dm      dh = g dy and dm_i = sum_t dy y / m_i for the norm-detached
//                backward (DoRA summary, "Statistical analysis"), one pass
//                over dy and y with fixed-order partial sums.
//   small ones   split-K reduction, Gram matrix finalisation (fp32 sum of
//                split partials, bf16 hi/lo split) and the row-norm finish.
//
// Streaming layout: a thread owns one group of 8 consecutive columns and
// every R-th row from its first, so per-column factors (g - 1, g s) are
// formed once per thread; every access is a 16-byte load / store and
// consecutive threads cover consecutive 16-byte groups of a row, the grid
// sweeping R whole rows at a time (fully coalesced, in address order).
#include "dora_internal.hpp"
#include "epilogue.hpp"

namespace dora {
namespace {

constexpr int EW_THREADS = 256;
// The two-in / one-out streams (compose, dh / dm) run between 2^17 and 2^18
// threads: enough that a thread streams at least 64 rows of its column group
// (the per-column factors it forms once, in fp64, are then paid for over
// that many rows), up to the launch size at which a plain stream of this
// pattern moves the most bytes (4096 x 4096 to 16384 x 27648 bf16: 5.0 - 5.9
// TB/s with the MALL flushed, against 4.4 - 5.6 at 2^20 threads).  Measured
// on the compose: 2^17 threads 6 - 10% faster than 2^18 at 4096^2 and 8192^2
// (16 and 64 rows a thread), 2^18 7% faster at 8192 x 28672 (112 rows).
constexpr int64_t STREAM_THREADS_MIN = int64_t(1) << 17;
constexpr int64_t STREAM_THREADS_MAX = int64_t(1) << 18;
constexpr int64_t STREAM_ROWS_PER_THREAD = 64;

// 16-byte streaming accesses with the nontemporal hint: data read or written
// once per launch should not displace what other waves still reuse (about
// 17% more bandwidth than plain accesses for the [T, d_out] streams here).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load16(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stream_store16(void *p, uint4 v)
{
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}

template <typename T>
struct Vec8;
template <>
struct Vec8<uint16_t> {
    __device__ static void load(const uint16_t *p, float (&v)[8])
    {
        const uint4 u = stream_load16(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(w[q] << 16);
            v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
    __device__ static void store(uint16_t *p, const float (&v)[8])
    {
        stream_store16(p, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                     pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
    }
    __device__ static float load1(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ static void store1(uint16_t *p, float v) { *p = f32_to_bf16(v); }
};
template <>
struct Vec8<float> {
    __device__ static void load(const float *p, float (&v)[8])
    {
        const uint4 a = stream_load16(p), b = stream_load16(p + 4);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
    __device__ static void store(float *p, const float (&v)[8])
    {
        stream_store16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                     __float_as_uint(v[2]), __float_as_uint(v[3])));
        stream_store16(p + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                         __float_as_uint(v[6]), __float_as_uint(v[7])));
    }
    __device__ static float load1(const float *p) { return *p; }
    __device__ static void store1(float *p, float v) { *p = v; }
};

// Rows a [T, d_out] stream with gpr 16-byte column groups advances per
// sweep: thread g takes column group g % gpr and rows g / gpr, g / gpr + R,
// g / gpr + 2 R, ..., so that per-column factors are formed once per thread
// and every sweep of the grid reads R whole consecutive rows (the memory is
// streamed in address order).
__host__ __device__ inline int64_t sweep_rows(int64_t T, int64_t gpr)
{
    int64_t th = gpr * T / STREAM_ROWS_PER_THREAD;
    th = th < STREAM_THREADS_MIN ? STREAM_THREADS_MIN
                                 : (th > STREAM_THREADS_MAX ? STREAM_THREADS_MAX : th);
    int64_t R = (th + gpr / 2) / (gpr > 0 ? gpr : 1);
    if (R < 1)
        R = 1;
    if (R > T)
        R = T;
    return R;
}

// One compose element in the stable form: y = b + ((g - 1) b + g s l).
__device__ __forceinline__ float compose1(float b, float l, float gm1, float gs)
{
    return b + __fmaf_rn(gm1, b, gs * l);
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(EW_THREADS)
    compose_kernel(const T *__restrict__ base, const T *__restrict__ lora,
                   const float *__restrict__ m, const float *__restrict__ n, float s, int64_t Tn,
                   int64_t d_out, int64_t R, T *y)
{
    const int64_t gpr = (d_out + 7) / 8;
    const int64_t gi = static_cast<int64_t>(blockIdx.x) * EW_THREADS + threadIdx.x;
    const int64_t c = gi % gpr, t0 = gi / gpr;
    if (t0 >= R)
        return;
    const int64_t i0 = c * 8;
    const int cnt = (d_out - i0) < 8 ? static_cast<int>(d_out - i0) : 8;
    // the first row's loads go out before the factors are formed, so their
    // latency covers that arithmetic
    float b0[8], l0[8];
    if (VEC) {
        Vec8<T>::load(base + t0 * d_out + i0, b0);
        Vec8<T>::load(lora + t0 * d_out + i0, l0);
    }
    // per-column factors, once per thread, each rounded once to fp32 from
    // fp64 (g - 1 = (m - n) / n and g s = m s / n): the lora term then
    // carries two roundings (g s, its product with lora) instead of three
    float gm1[8], gs[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const double mi = q < cnt ? m[i0 + q] : 1.0;
        const double ni = q < cnt ? n[i0 + q] : 1.0;
        gm1[q] = static_cast<float>((mi - ni) / ni);
        gs[q] = static_cast<float>(mi * static_cast<double>(s) / ni);
    }
    // y may be base itself: each element is read, then written, by the same
    // thread
    if (VEC) {
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            o[q] = compose1(b0[q], l0[q], gm1[q], gs[q]);
        Vec8<T>::store(y + t0 * d_out + i0, o);
    }
    for (int64_t t = VEC ? t0 + R : t0; t < Tn; t += R) {
        const int64_t off = t * d_out + i0;
        if (VEC) {
            float b[8], l[8], o[8];
            Vec8<T>::load(base + off, b);
            Vec8<T>::load(lora + off, l);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                o[q] = compose1(b[q], l[q], gm1[q], gs[q]);
            Vec8<T>::store(y + off, o);
        } else {
            for (int q = 0; q < cnt; ++q)
                Vec8<T>::store1(y + off + q, compose1(Vec8<T>::load1(base + off + q),
                                                      Vec8<T>::load1(lora + off + q), gm1[q],
                                                      gs[q]));
        }
    }
}

// dh = g dy and dm partial sums: thread (column group c, first row t0)
// sums dy y over rows t0, t0 + R, ... into dm_part[t0][c * 8 ..].
template <typename T, bool VEC>
__global__ void __launch_bounds__(EW_THREADS)
    dh_dm_kernel(const T *__restrict__ dy, const T *__restrict__ yv, const float *__restrict__ m,
                 const float *__restrict__ n, int64_t Tn, int64_t d_out, int64_t R,
                 T *__restrict__ dh, float *__restrict__ dm_part)
{
    const int64_t gpr = (d_out + 7) / 8;
    const int64_t gi = static_cast<int64_t>(blockIdx.x) * EW_THREADS + threadIdx.x;
    const int64_t c = gi % gpr, t0 = gi / gpr;
    if (t0 >= R)
        return;
    const int64_t i0 = c * 8;
    const int cnt = (d_out - i0) < 8 ? static_cast<int>(d_out - i0) : 8;
    float g[8], acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        g[q] = q < cnt ? m[i0 + q] / n[i0 + q] : 0.f;
        acc[q] = 0.f;
    }
    for (int64_t t = t0; t < Tn; t += R) {
        const int64_t off = t * d_out + i0;
        if (VEC) {
            float a[8], b[8], o[8];
            Vec8<T>::load(dy + off, a);
            Vec8<T>::load(yv + off, b);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                o[q] = g[q] * a[q];
                acc[q] = __fmaf_rn(a[q], b[q], acc[q]);
            }
            Vec8<T>::store(dh + off, o);
        } else {
            for (int q = 0; q < cnt; ++q) {
                const float a = Vec8<T>::load1(dy + off + q);
                Vec8<T>::store1(dh + off + q, g[q] * a);
                acc[q] = __fmaf_rn(a, Vec8<T>::load1(yv + off + q), acc[q]);
            }
        }
    }
    for (int q = 0; q < cnt; ++q)
        dm_part[t0 * d_out + i0 + q] = acc[q];
}

__global__ void dm_finish_kernel(const float *__restrict__ part, int nchunks,
                                 const float *__restrict__ m, int64_t d_out, float *__restrict__ dm)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= d_out)
        return;
    // fixed summation order; loads in batches of 8 so they are in flight
    // together
    float acc = 0.f;
    int k = 0;
    for (; k + 8 <= nchunks; k += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = part[static_cast<int64_t>(k + u) * d_out + i];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc += v[u];
    }
    for (; k < nchunks; ++k)
        acc += part[static_cast<int64_t>(k) * d_out + i];
    dm[i] = acc / m[i];
}

template <typename T>
__global__ void splitk_reduce_kernel(const float *__restrict__ part, int splits, int64_t MN,
                                     int64_t N, float alpha, T *__restrict__ out,
                                     const float *__restrict__ colm,
                                     const float *__restrict__ coln, T *__restrict__ out2,
                                     float alpha2)
{
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < MN;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float acc = 0.f;
        for (int z = 0; z < splits; ++z)
            acc += part[static_cast<int64_t>(z) * MN + e];
        float v = alpha * acc;
        if (colm != nullptr) {
            const int64_t n = e % N;
            v = __fmaf_rn((colm[n] - coln[n]) / coln[n], v, v);
        }
        Vec8<T>::store1(out + e, v);
        if (out2 != nullptr)
            Vec8<T>::store1(out2 + e, alpha2 * acc);
    }
}

// G = sum_z part[z] (fixed order).  bf16: writes G_hi = bf16(G) into rows
// [0, r) and G_lo = bf16(G - G_hi) into rows [r, 2r) of a [2r, r] matrix, so
// that B G = B G_hi + B G_lo keeps about 16 bits of G on bf16 MFMAs.
// fp32: writes G itself.
__device__ __forceinline__ void gram_finalize_all(const float *__restrict__ part, int splits,
                                                  int64_t r, int bf16, void *__restrict__ G_out)
{
    const int64_t rr = r * r;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < rr;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float acc = 0.f;
        for (int z = 0; z < splits; ++z)
            acc += part[static_cast<int64_t>(z) * rr + e];
        if (bf16) {
            uint16_t *G = static_cast<uint16_t *>(G_out);
            const uint16_t hi = f32_to_bf16(acc);
            G[e] = hi;
            G[rr + e] = f32_to_bf16(acc - bf16_to_f32(hi));
        } else {
            static_cast<float *>(G_out)[e] = acc;
        }
    }
}

__global__ void gram_finalize_kernel(const float *__restrict__ part, int splits, int64_t r, int bf16,
                                     void *__restrict__ G_out)
{
    gram_finalize_all(part, splits, r, bf16, G_out);
}

// One module of a group per blockIdx.y.
__global__ void gram_finalize_grouped_kernel(ItemGroup<GramItem> g, int bf16)
{
    const GramItem &it = g.it[blockIdx.y];
    gram_finalize_all(it.part, it.splits, it.r, bf16, it.G);
}

// Backward through the norm: cs_i = -s m_i dm_i / n_i^2 (the row
// coefficient of the norm's gradient, times -s) and cB = cs (.) B.  VEC: a
// thread takes 8 consecutive elements of a row (r a multiple of 8).
template <typename T, bool VEC>
__global__ void norm_grad_coef_kernel(const float *__restrict__ m, const float *__restrict__ dm,
                                      const float *__restrict__ n, float s,
                                      const T *__restrict__ B, int64_t d_out, int64_t r,
                                      float *__restrict__ cs, T *__restrict__ cB)
{
    const int64_t per = VEC ? r / 8 : r;  // work items per row
    const int64_t total = d_out * per;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < total;
         q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t i = q / per;
        const float c = -s * m[i] * dm[i] / (n[i] * n[i]);
        if (q % per == 0)
            cs[i] = c;
        if (VEC) {
            const int64_t e = q * 8;
            float v[8];
            Vec8<T>::load(B + e, v);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                v[k] = c * v[k];
            Vec8<T>::store(cB + e, v);
        } else {
            Vec8<T>::store1(cB + q, c * Vec8<T>::load1(B + q));
        }
    }
}

// out[i, j] = sum_z part[z][i, j] + f_i (y0[i, j] + sum_u ypart[u][i, j])
// (f_i = rowscale[i] or 1, y0 optional), in this fixed order, rounded once.  VEC: 8 consecutive elements of
// a row per thread (N a multiple of 8).
template <typename T, bool VEC>
__global__ void combine_rows_kernel(const float *__restrict__ part, int np,
                                    const float *__restrict__ ypart, int ny,
                                    const float *__restrict__ rowscale, int64_t M, int64_t N,
                                    T *__restrict__ out, const float *__restrict__ y0)
{
    const int64_t MN = M * N;
    constexpr int L = VEC ? 8 : 1;
    const int64_t items = MN / L;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < items;
         q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t e = q * L;
        float a[L], y[L], t[L];
#pragma unroll
        for (int k = 0; k < L; ++k)
            a[k] = y[k] = 0.f;
        if (y0 != nullptr) {
            if constexpr (VEC) {
                Vec8<float>::load(y0 + e, y);
            } else {
                y[0] = y0[e];
            }
        }
        for (int z = 0; z < np; ++z) {
            if constexpr (VEC) {
                Vec8<float>::load(part + static_cast<int64_t>(z) * MN + e, t);
            } else {
                t[0] = part[static_cast<int64_t>(z) * MN + e];
            }
#pragma unroll
            for (int k = 0; k < L; ++k)
                a[k] += t[k];
        }
        for (int u = 0; u < ny; ++u) {
            if constexpr (VEC) {
                Vec8<float>::load(ypart + static_cast<int64_t>(u) * MN + e, t);
            } else {
                t[0] = ypart[static_cast<int64_t>(u) * MN + e];
            }
#pragma unroll
            for (int k = 0; k < L; ++k)
                y[k] += t[k];
        }
        const float f = rowscale != nullptr ? rowscale[e / N] : 1.f;
#pragma unroll
        for (int k = 0; k < L; ++k)
            t[k] = __fmaf_rn(f, y[k], a[k]);
        if constexpr (VEC) {
            Vec8<T>::store(out + e, t);
        } else {
            Vec8<T>::store1(out + e, t[0]);
        }
    }
}

// n_i = sqrt(max(base + 2 s cross + s^2 gram, 0)) from fixed-order sums of
// the per-split / per-tile partials, combined in fp64.
__device__ __forceinline__ void norm_finish_row(int64_t i, const float *__restrict__ bp, int zb,
                                                const float *__restrict__ cp, int zc,
                                                const float *__restrict__ gp, int zg,
                                                int64_t d_out, float s, float *__restrict__ n,
                                                float *base, float *cross, float *gram)
{
    // each sum in order z = 0, 1, ...; the loads of eight partials go out
    // together (a missing one adds +0.0, which changes no sum)
    auto sum = [&](const float *__restrict__ p, int nz) {
        double acc = 0.0;
        for (int z0 = 0; z0 < nz; z0 += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = z0 + q < nz ? p[static_cast<int64_t>(z0 + q) * d_out + i] : 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc += v[q];
        }
        return acc;
    };
    const double b = sum(bp, zb), c = sum(cp, zc), g = sum(gp, zg);
    n[i] = norm_from_terms(b, c, g, s);
    if (base)
        base[i] = static_cast<float>(b);
    if (cross)
        cross[i] = static_cast<float>(c);
    if (gram)
        gram[i] = static_cast<float>(g);
}

__global__ void norm_finish_kernel(const float *__restrict__ bp, int zb, const float *__restrict__ cp,
                                   int zc, const float *__restrict__ gp, int zg, int64_t d_out,
                                   float s, float *__restrict__ n, float *base, float *cross,
                                   float *gram)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < d_out)
        norm_finish_row(i, bp, zb, cp, zc, gp, zg, d_out, s, n, base, cross, gram);
}

__global__ void norm_finish_grouped_kernel(ItemGroup<NormFinishItem> g)
{
    const NormFinishItem &it = g.it[blockIdx.y];
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < it.d_out;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        norm_finish_row(i, it.bp, it.zb, it.cp, it.zc, it.gp, it.zg, it.d_out, it.s, it.n, nullptr,
                        nullptr, nullptr);
}

__global__ void copy_f32_kernel(const float *__restrict__ src, float *__restrict__ dst, int64_t n)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n)
        dst[i] = src[i];
}

__global__ void fill_f32_kernel(float *__restrict__ dst, float v, int64_t n)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n)
        dst[i] = v;
}

unsigned blocks_for(int64_t threads)
{
    return static_cast<unsigned>((threads + EW_THREADS - 1) / EW_THREADS);
}

}  // namespace

int64_t dm_sweep_rows(int64_t T, int64_t d_out)
{
    return sweep_rows(T, (d_out + 7) / 8);
}

hipError_t launch_compose(int bf16, const void *base, const void *lora, const float *m,
                          const float *n, float s, int64_t T, int64_t d_out, void *y,
                          hipStream_t st)
{
    if (T == 0 || d_out == 0)
        return hipSuccess;
    const int64_t gpr = (d_out + 7) / 8;
    const int64_t R = sweep_rows(T, gpr);
    const dim3 grid(blocks_for(gpr * R));
    const bool vec = (d_out % 8) == 0;
    if (bf16) {
        auto *b = static_cast<const uint16_t *>(base);
        auto *l = static_cast<const uint16_t *>(lora);
        auto *o = static_cast<uint16_t *>(y);
        if (vec)
            hipLaunchKernelGGL((compose_kernel<uint16_t, true>), grid, dim3(EW_THREADS), 0, st, b, l,
                               m, n, s, T, d_out, R, o);
        else
            hipLaunchKernelGGL((compose_kernel<uint16_t, false>), grid, dim3(EW_THREADS), 0, st, b,
                               l, m, n, s, T, d_out, R, o);
    } else {
        auto *b = static_cast<const float *>(base);
        auto *l = static_cast<const float *>(lora);
        auto *o = static_cast<float *>(y);
        if (vec)
            hipLaunchKernelGGL((compose_kernel<float, true>), grid, dim3(EW_THREADS), 0, st, b, l, m,
                               n, s, T, d_out, R, o);
        else
            hipLaunchKernelGGL((compose_kernel<float, false>), grid, dim3(EW_THREADS), 0, st, b, l,
                               m, n, s, T, d_out, R, o);
    }
    return hipGetLastError();
}

hipError_t launch_dh_dm_partial(int bf16, const void *dy, const void *y, const float *m,
                                const float *n, int64_t T, int64_t d_out, int64_t R,
                                void *dh, float *dm_part, hipStream_t st)
{
    if (T == 0 || d_out == 0)
        return hipSuccess;
    const int64_t gpr = (d_out + 7) / 8;
    const dim3 grid(blocks_for(gpr * R));
    const bool vec = (d_out % 8) == 0;
    if (bf16) {
        auto *a = static_cast<const uint16_t *>(dy);
        auto *b = static_cast<const uint16_t *>(y);
        auto *o = static_cast<uint16_t *>(dh);
        if (vec)
            hipLaunchKernelGGL((dh_dm_kernel<uint16_t, true>), grid, dim3(EW_THREADS), 0, st, a, b,
                               m, n, T, d_out, R, o, dm_part);
        else
            hipLaunchKernelGGL((dh_dm_kernel<uint16_t, false>), grid, dim3(EW_THREADS), 0, st, a, b,
                               m, n, T, d_out, R, o, dm_part);
    } else {
        auto *a = static_cast<const float *>(dy);
        auto *b = static_cast<const float *>(y);
        auto *o = static_cast<float *>(dh);
        if (vec)
            hipLaunchKernelGGL((dh_dm_kernel<float, true>), grid, dim3(EW_THREADS), 0, st, a, b, m,
                               n, T, d_out, R, o, dm_part);
        else
            hipLaunchKernelGGL((dh_dm_kernel<float, false>), grid, dim3(EW_THREADS), 0, st, a, b, m,
                               n, T, d_out, R, o, dm_part);
    }
    return hipGetLastError();
}

hipError_t launch_dm_finish(const float *dm_part, int nchunks, const float *m, int64_t d_out,
                            float *dm, hipStream_t st)
{
    if (d_out == 0)
        return hipSuccess;
    hipLaunchKernelGGL(dm_finish_kernel, dim3(blocks_for(d_out)), dim3(EW_THREADS), 0, st, dm_part,
                       nchunks, m, d_out, dm);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(int bf16, const float *part, int splits, int64_t M, int64_t N,
                                float alpha, void *out, hipStream_t st, const float *colm,
                                const float *coln, void *out2, float alpha2)
{
    const int64_t MN = M * N;
    if (MN == 0)
        return hipSuccess;
    int64_t blocks = (MN + EW_THREADS - 1) / EW_THREADS;
    if (blocks > 8192)
        blocks = 8192;
    if (bf16)
        hipLaunchKernelGGL((splitk_reduce_kernel<uint16_t>), dim3(static_cast<unsigned>(blocks)),
                           dim3(EW_THREADS), 0, st, part, splits, MN, N, alpha,
                           static_cast<uint16_t *>(out), colm, coln,
                           static_cast<uint16_t *>(out2), alpha2);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<float>), dim3(static_cast<unsigned>(blocks)),
                           dim3(EW_THREADS), 0, st, part, splits, MN, N, alpha,
                           static_cast<float *>(out), colm, coln, static_cast<float *>(out2),
                           alpha2);
    return hipGetLastError();
}

hipError_t launch_gram_finalize(int bf16, const float *part, int splits, int64_t r, void *G_out,
                                hipStream_t st)
{
    int64_t blocks = (r * r + EW_THREADS - 1) / EW_THREADS;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(gram_finalize_kernel, dim3(static_cast<unsigned>(blocks)), dim3(EW_THREADS), 0,
                       st, part, splits, r, bf16, G_out);
    return hipGetLastError();
}

hipError_t launch_norm_finish(const float *base_part, int zb, const float *cross_part, int zc,
                              const float *gram_part, int zg, int64_t d_out, float s, float *n,
                              float *base, float *cross, float *gram, hipStream_t st)
{
    if (d_out == 0)
        return hipSuccess;
    hipLaunchKernelGGL(norm_finish_kernel, dim3(blocks_for(d_out)), dim3(EW_THREADS), 0, st,
                       base_part, zb, cross_part, zc, gram_part, zg, d_out, s, n, base, cross, gram);
    return hipGetLastError();
}

hipError_t launch_norm_grad_coef(int bf16, const float *m, const float *dm, const float *n, float s,
                                 const void *B, int64_t d_out, int64_t r, float *cs, void *cB,
                                 hipStream_t st)
{
    if (d_out == 0)
        return hipSuccess;
    const bool vec = r % 8 == 0;
    int64_t blocks = (d_out * (vec ? r / 8 : r) + EW_THREADS - 1) / EW_THREADS;
    if (blocks > 8192)
        blocks = 8192;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (bf16) {
        auto *b = static_cast<const uint16_t *>(B);
        auto *o = static_cast<uint16_t *>(cB);
        if (vec)
            hipLaunchKernelGGL((norm_grad_coef_kernel<uint16_t, true>), grid, dim3(EW_THREADS), 0,
                               st, m, dm, n, s, b, d_out, r, cs, o);
        else
            hipLaunchKernelGGL((norm_grad_coef_kernel<uint16_t, false>), grid, dim3(EW_THREADS), 0,
                               st, m, dm, n, s, b, d_out, r, cs, o);
    } else {
        auto *b = static_cast<const float *>(B);
        auto *o = static_cast<float *>(cB);
        if (vec)
            hipLaunchKernelGGL((norm_grad_coef_kernel<float, true>), grid, dim3(EW_THREADS), 0, st,
                               m, dm, n, s, b, d_out, r, cs, o);
        else
            hipLaunchKernelGGL((norm_grad_coef_kernel<float, false>), grid, dim3(EW_THREADS), 0, st,
                               m, dm, n, s, b, d_out, r, cs, o);
    }
    return hipGetLastError();
}

hipError_t launch_combine_rows(int bf16, const float *part, int np, const float *ypart, int ny,
                               const float *rowscale, int64_t M, int64_t N, void *out,
                               hipStream_t st, const float *y0)
{
    if (M == 0 || N == 0)
        return hipSuccess;
    const bool vec = N % 8 == 0;
    int64_t blocks = (M * N / (vec ? 8 : 1) + EW_THREADS - 1) / EW_THREADS;
    if (blocks > 8192)
        blocks = 8192;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (bf16) {
        auto *o = static_cast<uint16_t *>(out);
        if (vec)
            hipLaunchKernelGGL((combine_rows_kernel<uint16_t, true>), grid, dim3(EW_THREADS), 0, st,
                               part, np, ypart, ny, rowscale, M, N, o, y0);
        else
            hipLaunchKernelGGL((combine_rows_kernel<uint16_t, false>), grid, dim3(EW_THREADS), 0,
                               st, part, np, ypart, ny, rowscale, M, N, o, y0);
    } else {
        auto *o = static_cast<float *>(out);
        if (vec)
            hipLaunchKernelGGL((combine_rows_kernel<float, true>), grid, dim3(EW_THREADS), 0, st,
                               part, np, ypart, ny, rowscale, M, N, o, y0);
        else
            hipLaunchKernelGGL((combine_rows_kernel<float, false>), grid, dim3(EW_THREADS), 0, st,
                               part, np, ypart, ny, rowscale, M, N, o, y0);
    }
    return hipGetLastError();
}

hipError_t launch_gram_finalize_grouped(int bf16, const ItemGroup<GramItem> &g, hipStream_t st)
{
    int64_t most = 0;
    for (int k = 0; k < g.count; ++k)
        most = most > g.it[k].r * g.it[k].r ? most : g.it[k].r * g.it[k].r;
    if (g.count == 0 || most == 0)
        return hipSuccess;
    int64_t blocks = (most + EW_THREADS - 1) / EW_THREADS;
    if (blocks > 1024)
        blocks = 1024;
    hipLaunchKernelGGL(gram_finalize_grouped_kernel,
                       dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(g.count)),
                       dim3(EW_THREADS), 0, st, g, bf16);
    return hipGetLastError();
}

hipError_t launch_norm_finish_grouped(const ItemGroup<NormFinishItem> &g, hipStream_t st)
{
    int64_t most = 0;
    for (int k = 0; k < g.count; ++k)
        most = most > g.it[k].d_out ? most : g.it[k].d_out;
    if (g.count == 0 || most == 0)
        return hipSuccess;
    hipLaunchKernelGGL(norm_finish_grouped_kernel,
                       dim3(blocks_for(most), static_cast<unsigned>(g.count)), dim3(EW_THREADS), 0,
                       st, g);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t st)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(copy_f32_kernel, dim3(blocks_for(n)), dim3(EW_THREADS), 0, st, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float *dst, float v, int64_t n, hipStream_t st)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks_for(n)), dim3(EW_THREADS), 0, st, dst, v, n);
    return hipGetLastError();
}

}  // namespace dora
