// COMBINE kernel: the sequential scan of segment maps for chains too few to
// fill the GPU (the segment-scan COMBINE of the cudnn-frontend Hopper KDA
// prefill PR #1056, which scans "independent value-row slabs").
//
// A segment of a chain maps its start state affinely to its end state,
//     S_end = M_s S_start + C_s,
// where M_s is the segment's end state from (V = 0, S_start = I) and C_s from
// S_start = 0 (both built by the chunk kernel's segment roles).  Columns of S
// evolve independently, so one workgroup owns one 16-column value slab of one
// chain and walks the segments in order: start[0] = initial state,
// start[s+1] = M_s start[s] + C_s, in fp32 on the fp32 matrix cores (M_s and
// C_s stay fp32: they compose many chunk maps).  Narrow slabs put D/16
// workgroups on every chain, so a handful of chains still spreads over many
// CUs; M_s and C_s do not depend on the scan, so each wave loads the operands
// of the segments two steps ahead while it multiplies the current one.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void combine_kernel(const CombineParams p)
{
    constexpr int NW = D / 16, NT = 64 * NW, SL = 16, ST_LD = D + 4, KB = D / 16;
    // the slab's current state, transposed ([value column][key channel]), double-buffered so
    // that one barrier per segment orders every write after the reads it replaces
    __shared__ __attribute__((aligned(16))) float sS[2][SL * ST_LD];
    const int lchain = blockIdx.x, chain = p.seg_chain0 + lchain, slab = blockIdx.y, v0 = SL * slab;
    const int n = chain / p.H, h = chain % p.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    float *start = p.start + (int64_t)lchain * p.nseg * D * D;
    const float *maps = p.maps + map_offset(lchain, p.nseg, 0, 0, D);

    for (int e = tid; e < D * SL; e += NT) {
        const int ch = e / SL, v = e % SL;
        const int64_t at = n * p.s0_sn + h * p.s0_sh + ch * p.s0_sr + v0 + v;
        const float x = p.s0 ? p.s0[at] : p.s0h ? (float)p.s0h[at] : 0.f;
        sS[0][v * ST_LD + ch] = x;
        start[ch * D + v0 + v] = x;
    }
    // Wave w produces rows 16w..16w+15 of the slab with 16x16x4 fp32 MFMAs.  The sum over key
    // channels k is taken in the order k = 16j + 4(lane/16) + e for MFMA 4j + e, so each lane
    // feeds four consecutive MFMAs from one 16-byte read of its M row and one of the slab.
    // M is stored in this read order (map_m_index): load j of a wave is one contiguous 1 KB run.
    // M_s and C_s of the next PF segments wait in registers, a ring indexed at compile time (the
    // segment loop is unrolled PF times).  Every step issues the same loads -- those of segment
    // s + PF, clamped to the last one -- and the loop has no exit inside its unrolled body, so
    // the compiler's wait before a step's products covers only the loads of that step, issued
    // PF steps earlier, not the younger ones in flight.
    constexpr int PF = 2;
    float4 m[PF][KB];
    float c[PF][4];
    auto load_maps = [&](int s, float4 (&mm)[KB], float (&cc)[4]) {
        const float *M = maps + (int64_t)s * 2 * D * D, *C = M + D * D;
#pragma unroll
        for (int j = 0; j < KB; ++j) mm[j] = *(const float4 *)(M + ((wave * KB + j) * 64 + lane) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) cc[r] = C[(16 * wave + 4 * g4 + r) * D + v0 + l16];
    };
    const int steps = p.nseg - 1;        // start[s + 1] = M_s start[s] + C_s for s < steps
    const int last = steps - 1;
#pragma unroll
    for (int u = 0; u < PF; ++u) load_maps(min(u, last), m[u], c[u]);
    __syncthreads();
    auto step = [&](int s, float4 (&mm)[KB], float (&cc)[4]) {
        const float *cur = sS[s & 1];
        f32x4 acc = {cc[0], cc[1], cc[2], cc[3]};
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const float4 b = *(const float4 *)(cur + l16 * ST_LD + 16 * j + 4 * g4);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].x, b.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].y, b.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].z, b.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].w, b.w, acc, 0, 0, 0);
        }
        load_maps(min(s + PF, last), mm, cc);
        // lane (column l16, group g4) holds rows 16w + 4 g4 + r of start[s+1]
        *(float4 *)(sS[(s + 1) & 1] + l16 * ST_LD + 16 * wave + 4 * g4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        float *st = start + (int64_t)(s + 1) * D * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(16 * wave + 4 * g4 + r) * D + v0 + l16] = acc[r];
        __syncthreads();
    };
    int s = 0;
    for (; s + PF <= steps; s += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) step(s + u, m[u], c[u]);
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (s + u < steps) step(s + u, m[u], c[u]);
}

hipError_t launch_combine(const CombineParams &p, int D, int chains, hipStream_t st)
{
    if (chains <= 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(combine_kernel<128>, dim3(chains, 128 / 16), dim3(64 * 128 / 16), 0, st, p);
    else if (D == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(chains, 64 / 16), dim3(64 * 64 / 16), 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
