// COMBINE kernel: the sequential scan of segment maps for chains too few to
// fill the GPU (the segment-scan COMBINE of the cudnn-frontend Hopper KDA
// prefill PR #1056, which scans "independent value-row slabs").
//
// A segment of a chain maps its start state affinely to its end state,
//     S_end = M_s S_start + C_s,
// where M_s is the segment's end state from (V = 0, S_start = I) and C_s from
// S_start = 0 (both built by the chunk kernel's segment roles).  Columns of S
// evolve independently, so one workgroup owns one 32-column value slab of one
// chain and walks the segments in order: start[0] = initial state,
// start[s+1] = M_s start[s] + C_s, in fp32 on the fp32 matrix cores
// (M_s and C_s stay fp32: they compose many chunk maps).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void combine_kernel(const CombineParams p)
{
    constexpr int NW = D / 32, NT = 64 * NW, ST_LD = D + 4;
    __shared__ __attribute__((aligned(16))) float sS[32 * ST_LD];   // slab, transposed: [v][key channel]
    const int chain = blockIdx.x, slab = blockIdx.y;
    const int n = chain / p.H, h = chain % p.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;
    const int v0 = 32 * slab;
    for (int e = tid; e < D * 32; e += NT) {
        const int ch = e >> 5, v = e & 31;
        sS[v * ST_LD + ch] = p.s0 ? p.s0[n * p.s0_sn + h * p.s0_sh + ch * p.s0_sr + v0 + v] : 0.f;
    }
    __syncthreads();
    for (int s = 0; s < p.nseg; ++s) {
        float *st = p.start + ((int64_t)chain * p.nseg + s) * D * D;
        for (int e = tid; e < D * 32; e += NT) {
            const int ch = e >> 5, v = e & 31;
            st[ch * D + v0 + v] = sS[v * ST_LD + ch];
        }
        if (s == p.nseg - 1) break;
        const float *M = p.maps + (((int64_t)chain * p.nseg + s) * 2) * D * D;
        const float *C = M + D * D;
        f32x16 acc;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[4 * q + r] = C[(32 * wave + 8 * q + 4 * g2 + r) * D + v0 + l32];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            Frag8<float> fa, fb;
            const float *mrow = M + (32 * wave + l32) * D + 16 * ks + 4 * g2;
            fa.load44(mrow, mrow + 8);
            const float *srow = sS + l32 * ST_LD + 16 * ks + 4 * g2;
            fb.load44(srow, srow + 8);
            mma32(acc, fa, fb);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *(float4 *)(sS + l32 * ST_LD + 32 * wave + 8 * q + 4 * g2) =
                make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
        __syncthreads();
    }
}

hipError_t launch_combine(const CombineParams &p, int D, int chains, hipStream_t st)
{
    if (chains <= 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(combine_kernel<128>, dim3(chains, 4), dim3(256), 0, st, p);
    else if (D == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(chains, 2), dim3(128), 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
