// stream_ceiling.hip - measurement helper (libstreamceil.so, not part of the
// DoRA library): the HBM rate this part sustains for the access pattern of
// the compose and the backward's dh/dm pass, two streams read and one
// written, 16 bytes per lane and access, with the non-temporal hint.  The
// benchmark sweeps its launch shapes and takes the best as the ceiling the
// two streaming kernels are compared with.  Nothing of the DoRA method is
// computed here: c = a + b on 32-bit words.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld(const u32x4_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4_t *p, u32x4_t v) { __builtin_nontemporal_store(v, p); }

// Grid-stride over 16-byte vectors, U vectors of each input in flight per
// thread before any store.
template <int U>
__global__ void __launch_bounds__(256) stream_kernel(const u32x4_t *__restrict__ a,
                                                     const u32x4_t *__restrict__ b,
                                                     u32x4_t *__restrict__ c, int64_t nvec)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < nvec; i += U * stride) {
        u32x4_t x[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            x[u] = ld(a + i + u * stride);
            y[u] = ld(b + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            st(c + i + u * stride, x[u] + y[u]);
    }
    for (; i < nvec; i += stride)
        st(c + i, ld(a + i) + ld(b + i));
}

// The compose kernel's own order: a thread takes one 16-byte column group of
// a [rows, cols] matrix and a run of `run` consecutive rows, four rows in
// flight.
__global__ void __launch_bounds__(256) rows_kernel(const u32x4_t *__restrict__ a,
                                                   const u32x4_t *__restrict__ b,
                                                   u32x4_t *__restrict__ c, int64_t rows,
                                                   int64_t gpr, int64_t run)
{
    const int64_t gi = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t col = gi % gpr, t0 = (gi / gpr) * run;
    if (t0 >= rows)
        return;
    const int64_t t1 = t0 + run < rows ? t0 + run : rows;
    int64_t t = t0;
    for (; t + 4 <= t1; t += 4) {
        u32x4_t x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = ld(a + (t + u) * gpr + col);
            y[u] = ld(b + (t + u) * gpr + col);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            st(c + (t + u) * gpr + col, x[u] + y[u]);
    }
    for (; t < t1; ++t)
        st(c + t * gpr + col, ld(a + t * gpr + col) + ld(b + t * gpr + col));
}

}  // namespace

// variant 0..3: grid-stride with 1, 2, 4, 8 vectors in flight per input;
// variant 4: the [rows, cols] run order (row_bytes per row, a multiple of
// 16).  `threads` sets the launch size.  Returns a hipError_t code.
extern "C" int stream_ceiling_launch(const void *a, const void *b, void *c, int64_t bytes,
                                     int64_t row_bytes, int variant, int64_t threads,
                                     void *stream)
{
    if (bytes % 16 || row_bytes <= 0 || row_bytes % 16 || bytes % row_bytes || threads < 256)
        return hipErrorInvalidValue;
    auto *pa = static_cast<const u32x4_t *>(a);
    auto *pb = static_cast<const u32x4_t *>(b);
    auto *pc = static_cast<u32x4_t *>(c);
    const int64_t nvec = bytes / 16;
    const dim3 block(256), grid(static_cast<unsigned>((threads + 255) / 256));
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (variant) {
    case 0: hipLaunchKernelGGL(stream_kernel<1>, grid, block, 0, st, pa, pb, pc, nvec); break;
    case 1: hipLaunchKernelGGL(stream_kernel<2>, grid, block, 0, st, pa, pb, pc, nvec); break;
    case 2: hipLaunchKernelGGL(stream_kernel<4>, grid, block, 0, st, pa, pb, pc, nvec); break;
    case 3: hipLaunchKernelGGL(stream_kernel<8>, grid, block, 0, st, pa, pb, pc, nvec); break;
    case 4: {
        const int64_t gpr = row_bytes / 16, rows = bytes / row_bytes;
        int64_t runs = threads / gpr;
        runs = runs < 1 ? 1 : (runs > rows ? rows : runs);
        const int64_t run = (rows + runs - 1) / runs;
        const int64_t used = ((rows + run - 1) / run) * gpr;
        hipLaunchKernelGGL(rows_kernel, dim3(static_cast<unsigned>((used + 255) / 256)), block, 0,
                           st, pa, pb, pc, rows, gpr, run);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
