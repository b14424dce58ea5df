// Measurement probes (include/kda_peak.h): a plain HBM stream with the chunk kernel's
// five-to-one read/write mix, and a loop of independent bf16 MFMAs.  They give the
// practical ceilings against which the KDA kernels' HBM and matrix-core fractions are read.
#include <hip/hip_runtime.h>

#include "../../include/kda_peak.h"
#include "kda_device.hpp"

namespace kda {

// One 16-byte element of every array per thread, loads and stores non-temporal: of the stream
// shapes measured on MI355X (grid-stride loops with 2 or 4 elements per thread and 8-32
// workgroups per CU; contiguous tiles of 256-65536 elements per workgroup with 1, 2 or 4
// elements per thread; staggered array offsets; temporal or non-temporal loads and stores)
// this one was the fastest, 5.9-6.0 TB/s at the 5:1 mix.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void peak_stream_kernel(const u32x4 *a, const u32x4 *b, const u32x4 *c,
                                                          const u32x4 *d, const u32x4 *e, u32x4 *out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const u32x4 r = __builtin_nontemporal_load(a + i) ^ __builtin_nontemporal_load(b + i) ^
                    __builtin_nontemporal_load(c + i) ^ __builtin_nontemporal_load(d + i) ^
                    __builtin_nontemporal_load(e + i);
    __builtin_nontemporal_store(r, out + i);
}

// Eight independent accumulator chains per wave keep the matrix core's pipeline full; the
// operands depend on the lane so that nothing folds at compile time.
__global__ __launch_bounds__(256) void peak_mfma_kernel(float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    float fa[8], fb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        fa[e] = 1e-3f * (float)((lane * 8 + e) % 17);
        fb[e] = 1e-3f * (float)((lane * 5 + e) % 13);
    }
    Frag8<bf16> a, b;
    a.set(fa);
    b.set(fb);
    f32x16 acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 8; ++m) mma32(acc[m], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[m][r];
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace kda

extern "C" {

kda_status_t kda_peak_stream(const void *const in[5], void *out, int64_t n16, void *stream)
{
    if (!in || !out) return KDA_ERR_NULL;
    for (int i = 0; i < 5; ++i)
        if (!in[i]) return KDA_ERR_NULL;
    if (n16 <= 0) return KDA_ERR_SHAPE;
    const int64_t blocks = (n16 + 255) / 256;
    if (blocks > INT32_MAX) return KDA_ERR_SHAPE;
    typedef kda::u32x4 V;
    hipLaunchKernelGGL(kda::peak_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const V *)in[0], (const V *)in[1], (const V *)in[2], (const V *)in[3], (const V *)in[4],
                       (V *)out, n16);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_peak_mfma(float *out, int32_t workgroups, int32_t iters, void *stream)
{
    if (!out) return KDA_ERR_NULL;
    if (workgroups <= 0 || iters <= 0) return KDA_ERR_SHAPE;
    hipLaunchKernelGGL(kda::peak_mfma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
