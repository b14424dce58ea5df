// COMBINE kernel: the sequential scan of segment maps for chains too few to
// fill the GPU (the segment-scan COMBINE of the cudnn-frontend Hopper KDA
// prefill PR #1056, which scans the state's value columns in independent slabs).
//
// A segment of a chain maps its start state affinely to its end state,
//     S_end = M_s S_start + C_s,
// where M_s is the segment's end state from (V = 0, S_start = I) and C_s from
// S_start = 0 (both built by the chunk kernel's segment roles).  Columns of S
// evolve independently, so one workgroup owns one 16-column value slab of one
// chain and walks the segments in order: start[0] = initial state,
// start[s+1] = M_s start[s] + C_s.  Narrow slabs put D/16 workgroups on every
// chain, so a handful of chains still spreads over many CUs; M_s and C_s do not
// depend on the scan, so each wave loads the operands of the segments two steps
// ahead while it multiplies the current one.
//
// M_s and start[s] compose many chunk maps, so the product keeps about 16 bits:
// on bf16 I/O each is split into two bf16 parts (x = xh + xl, the split the map
// pass already stored M_s in) and M start runs as Mh Sh + Mh Sl + Ml Sh on the
// bf16 matrix cores (16x16x32), relative error near 2^-16; on fp32 I/O (the
// debug mode) it runs in fp32 on the fp32 matrix cores (16x16x4).  C_s and the
// start states in HBM stay fp32.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * (D / 16)) void combine_kernel(const CombineParams p)
{
    constexpr int NW = D / 16, NT = 64 * NW, SL = 16, KB = D / 16;
    // the slab's current state, transposed ([value column][key channel]), double-buffered so
    // that one barrier per segment orders every write after the reads it replaces: fp32, or its
    // bf16 parts (high, low) in two planes
    constexpr int ST_LD = D + 4, SP_LD = D + 8;
    constexpr int PLANE = SL * SP_LD;                      // bf16 elements per plane
    constexpr int BUF_BYTES = SPLIT ? 2 * PLANE * 2 : SL * ST_LD * 4;
    __shared__ __attribute__((aligned(16))) char sbuf[2][BUF_BYTES];
    const int lchain = blockIdx.x, chain = p.seg_chain0 + lchain, slab = blockIdx.y, v0 = SL * slab;
    const int n = chain / p.H, h = chain % p.H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    float *start = p.start + (int64_t)lchain * p.nseg * D * D;
    const float *maps = p.maps + map_offset(lchain, p.nseg, 0, 0, D);

    for (int e = tid; e < D * SL; e += NT) {
        const int ch = e / SL, v = e % SL;
        const int64_t at = n * p.s0_sn + h * p.s0_sh + ch * p.s0_sr + v0 + v;
        const float x = p.s0 ? p.s0[at] : p.s0h ? (float)p.s0h[at] : 0.f;
        if constexpr (SPLIT) {
            bf16 *pl = (bf16 *)sbuf[0];
            const bf16 xh = (bf16)x;
            pl[v * SP_LD + ch] = xh;
            pl[PLANE + v * SP_LD + ch] = (bf16)(x - (float)xh);
        } else {
            ((float *)sbuf[0])[v * ST_LD + ch] = x;
        }
        start[ch * D + v0 + v] = x;
    }
    // Wave w produces rows 16w..16w+15 of the slab; lane l holds row 16w + l % 16 of M_s and
    // feeds the matrix cores from one 16-byte load per run of M (map_m_index, map_m_split_index).
    // fp32: the sum over key channels k is taken in the order k = 16j + 4(l/16) + e for MFMA
    // 4j + e.  split: MFMAs of 32 channels, k = 32b + 8(l/16) + 0..7 in block b.
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
        f32x4 acc = {cc[0], cc[1], cc[2], cc[3]};
        if constexpr (SPLIT) {
            const bf16 *cur = (const bf16 *)sbuf[s & 1];
#pragma unroll
            for (int b = 0; b < KB / 2; ++b) {
                const bf16x8 mh = __builtin_bit_cast(bf16x8, mm[2 * b]), ml = __builtin_bit_cast(bf16x8, mm[2 * b + 1]);
                const bf16x8 sh = *(const bf16x8 *)(cur + l16 * SP_LD + 32 * b + 8 * g4);
                const bf16x8 sl = *(const bf16x8 *)(cur + PLANE + l16 * SP_LD + 32 * b + 8 * g4);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh, sh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh, sl, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ml, sh, acc, 0, 0, 0);
            }
        } else {
            const float *cur = (const float *)sbuf[s & 1];
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const float4 b = *(const float4 *)(cur + l16 * ST_LD + 16 * j + 4 * g4);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].x, b.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].y, b.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].z, b.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mm[j].w, b.w, acc, 0, 0, 0);
            }
        }
        load_maps(min(s + PF, last), mm, cc);
        // lane (column l16, group g4) holds rows 16w + 4 g4 + r of start[s+1]
        if constexpr (SPLIT) {
            bf16 *nx = (bf16 *)sbuf[(s + 1) & 1];
            uint32_t h01, l01, h23, l23;
            split2(acc[0], acc[1], h01, l01);
            split2(acc[2], acc[3], h23, l23);
            *(uint2 *)(nx + l16 * SP_LD + 16 * wave + 4 * g4) = make_uint2(h01, h23);
            *(uint2 *)(nx + PLANE + l16 * SP_LD + 16 * wave + 4 * g4) = make_uint2(l01, l23);
        } else {
            *(float4 *)((float *)sbuf[(s + 1) & 1] + l16 * ST_LD + 16 * wave + 4 * g4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
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

hipError_t launch_combine(const CombineParams &p, int D, bool split, int chains, hipStream_t st)
{
    if (chains <= 0) return hipSuccess;
    if (D == 128 && split) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(chains, 128 / 16), dim3(64 * 128 / 16), 0, st, p);
    else if (D == 64 && split) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(chains, 64 / 16), dim3(64 * 64 / 16), 0, st, p);
    else if (D == 64) hipLaunchKernelGGL((combine_kernel<64, false>), dim3(chains, 64 / 16), dim3(64 * 64 / 16), 0, st, p);
    else return hipErrorInvalidValue;    // fp32 I/O runs at D = 64 only
    return hipGetLastError();
}

}  // namespace kda
