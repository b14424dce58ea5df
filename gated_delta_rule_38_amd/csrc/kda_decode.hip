// DECODE kernel: the KDA recurrence token by token against a pool of states --
// the decode / multi-token (MTP) verify side of KDA serving that TensorRT-LLM
// PR #19960 describes (a verify kernel over a few draft tokens, fp32 and bf16
// state pools, a replay-only mode that commits accepted drafts to the state).
//
// For request r and head h the state S = pool[idx[r], h] (d_k x d_v, row = key
// channel) runs through the request's first n_r tokens,
//     S <- Diag(e^{g_t}) S;   S <- S + k_t (beta_t (v_t - k_t^T S))^T;   o_t = S^T q_t,
// the same recurrence the prefill kernels compute in chunked form.  Outputs go
// to out[r, t] when out is given; the slot is overwritten with the last state
// when update is set (the pool is only read otherwise: the verify pass).
//
// Columns of S evolve independently.  One 256-thread workgroup owns one
// (request, head): lane group c (D/4 lanes) covers four consecutive value
// columns 4c..4c+3 of the state, the row groups split the key rows, and every
// thread keeps its rows x 4 columns in registers, so each state row moves
// through HBM as whole 16-byte (fp32) or 8-byte (bf16) lanes.  The two sums
// over key channels per token (k^T S and q^T S) are reduced across row groups
// in a fixed order (lane butterflies inside a wave, then the 4 waves through
// LDS), so results do not depend on timing.  The few tokens are staged in LDS
// once.  An index outside [0, P) skips the request (no output rows, no state
// write), so a bad index can never address memory.  With an output gate the
// output row is normalised before it is written (gated RMS norm over the D
// value channels: o * rsqrt(mean(o^2) + eps) * weight * sigmoid(gate)).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16>(const bf16 *p) { return (float)*p; }
// four consecutive elements: one 16-byte (fp32) or 8-byte (bf16) access
__device__ __forceinline__ void ld4(const float *p, float (&x)[4])
{
    const float4 v = *(const float4 *)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void ld4(const bf16 *p, float (&x)[4]) { Vec4<bf16>::unpack(Vec4<bf16>::load(p), x); }
// State and output rows are written once per launch and not read back by it: non-temporal
// stores (on the fp32 pool 19% faster than plain stores in an A/B on MI355X; no change on the
// bf16 pool).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st4(float *p, const float (&x)[4])
{
    const f32x4 v = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(v, (f32x4 *)p);
}
__device__ __forceinline__ void st4(bf16 *p, const float (&x)[4])    // RNE
{
    const uint2 u = Vec4<bf16>::pack(x);
    const u32x2 w = {u.x, u.y};
    __builtin_nontemporal_store(w, (u32x2 *)p);
}

// STALL: the test build with one wave stalled after every barrier (the results must not change).
template <int D, typename IT, typename ST, bool STALL>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p)
{
    constexpr int NCQ = D / 4;            // column quads = lanes per row group
    constexpr int NRG = 256 / NCQ;        // row groups (8 for D = 128, 16 for D = 64)
    constexpr int RPG = D / NRG;          // rows per thread
    constexpr int TM = DECODE_MAX_TOKENS;
    __shared__ __attribute__((aligned(16))) float sK[TM][D], sQ[TM][D], sE[TM][D], sV[TM][D], sB[TM];
    __shared__ __attribute__((aligned(16))) float sRed[2][4][D];
    const int h = blockIdx.x % p.H, r = blockIdx.x / p.H;
    const int tid = threadIdx.x, lane = tid & 63, cq = tid % NCQ, rg = tid / NCQ, wave = tid >> 6;
    const int slot = p.idx[r];
    if (slot < 0 || slot >= p.P) return;
    const int n = p.ntok ? min(max(p.ntok[r], 0), p.T) : p.T;
    const IT *q = (const IT *)p.q + r * p.q_sr + h * p.q_sh;
    const IT *k = (const IT *)p.k + r * p.k_sr + h * p.k_sh;
    const IT *v = (const IT *)p.v + r * p.v_sr + h * p.v_sh;
    const float *g = p.g + r * p.g_sr + h * p.g_sh;
    // the state rows are requested before the tokens are staged, so that both loads are in
    // flight together (one memory round trip per workgroup, not two)
    ST *ps = (ST *)p.pool + slot * p.p_sn + h * p.p_sh + (int64_t)(rg * RPG) * p.p_sr + 4 * cq;
    float s[RPG][4];
#pragma unroll
    for (int j = 0; j < RPG; ++j) ld4(ps + j * p.p_sr, s[j]);
    for (int e = tid; e < n * D; e += 256) {
        const int t = e / D, ch = e % D;
        sK[t][ch] = ld(k + t * p.k_st + ch);
        sQ[t][ch] = ld(q + t * p.q_st + ch);
        sV[t][ch] = ld(v + t * p.v_st + ch);
        const float x = g[t * p.g_st + ch];
        sE[t][ch] = fast_exp(p.gate_act ? gate_act(x, p.gate_lb) : x);
    }
    if (tid < n) {
        const float b = p.beta[r * p.b_sr + tid * p.b_st + h * p.b_sh];
        sB[tid] = p.beta_act ? sigmoid_act(b) : b;
    }
    auto sync = [&]() {
        __syncthreads();
        if constexpr (STALL) {
            if (wave == p.stall_wave)
                for (int i = 0; i < p.stall_iters; ++i) __builtin_amdgcn_s_sleep(127);
        }
    };
    sync();

    // sum of x over the row groups, for this lane's 4 columns: butterflies over the row-group
    // lanes of the wave, then the 4 waves' partials in a fixed order
    auto reduce = [&](float (&x)[4], float (*red)[D], float (&sum)[4]) {
#pragma unroll
        for (int off = NCQ; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += __shfl_xor(x[e], off);
        if (lane < NCQ) *(float4 *)&red[wave][4 * cq] = make_float4(x[0], x[1], x[2], x[3]);
        sync();
        const float4 a = *(const float4 *)&red[0][4 * cq], b = *(const float4 *)&red[1][4 * cq];
        const float4 c = *(const float4 *)&red[2][4 * cq], d = *(const float4 *)&red[3][4 * cq];
        sum[0] = (a.x + b.x) + (c.x + d.x);
        sum[1] = (a.y + b.y) + (c.y + d.y);
        sum[2] = (a.z + b.z) + (c.z + d.z);
        sum[3] = (a.w + b.w) + (c.w + d.w);
    };
    IT *o = p.o ? (IT *)p.o + r * p.o_sr + h * p.o_sh + 4 * cq : nullptr;
    for (int t = 0; t < n; ++t) {
        // decay, then the read k^T D S of this thread's rows
        float pr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPG; ++j) {
            const int i = rg * RPG + j;
            const float e = sE[t][i], kk = sK[t][i];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s[j][c] *= e;
                pr[c] += kk * s[j][c];
            }
        }
        float kS[4];
        reduce(pr, sRed[0], kS);
        const float4 v4 = *(const float4 *)&sV[t][4 * cq];
        const float b = sB[t];
        const float u[4] = {b * (v4.x - kS[0]), b * (v4.y - kS[1]), b * (v4.z - kS[2]), b * (v4.w - kS[3])};
        float po[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPG; ++j) {
            const int i = rg * RPG + j;
            const float kk = sK[t][i], qq = sQ[t][i];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s[j][c] += kk * u[c];
                po[c] += qq * s[j][c];
            }
        }
        float os[4];
        reduce(po, sRed[1], os);
        if (p.z) {
            // gated RMS norm of the output row: every lane holds the sums of its 4 columns, and a
            // butterfly over the lanes of one row group adds the D/4 lane groups in a fixed order
            float ss = (os[0] * os[0] + os[1] * os[1]) + (os[2] * os[2] + os[3] * os[3]);
#pragma unroll
            for (int off = 1; off < NCQ; off <<= 1) ss += __shfl_xor(ss, off);
            const float rn = __builtin_amdgcn_rsqf(ss * (1.f / D) + p.eps);
            if (o && tid < NCQ) {
                float zz[4];
                ld4((const IT *)p.z + r * p.z_sr + h * p.z_sh + t * p.z_st + 4 * cq, zz);
                const float4 w4 = *(const float4 *)(p.nw + 4 * cq);
                os[0] = os[0] * rn * w4.x * sigmoid_act(zz[0]);
                os[1] = os[1] * rn * w4.y * sigmoid_act(zz[1]);
                os[2] = os[2] * rn * w4.z * sigmoid_act(zz[2]);
                os[3] = os[3] * rn * w4.w * sigmoid_act(zz[3]);
            }
        }
        if (o && tid < NCQ) st4(o + t * p.o_st, os);
    }
    if (p.update) {
#pragma unroll
        for (int j = 0; j < RPG; ++j) st4(ps + j * p.p_sr, s[j]);
    }
}

template <int D, typename IT, typename ST>
static void launch_decode_t(const DecodeParams &p, unsigned blocks, hipStream_t stream)
{
    if (p.stall_wave >= 0 && p.stall_iters > 0)
        hipLaunchKernelGGL((decode_kernel<D, IT, ST, true>), dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, IT, ST, false>), dim3(blocks), dim3(256), 0, stream, p);
}

hipError_t launch_decode(const DecodeParams &p, int D, bool io_f32, bool state_bf16, hipStream_t stream)
{
    const int64_t blocks = (int64_t)p.R * p.H;
    if (blocks <= 0) return hipSuccess;
#define KDA_DECODE(DD, IT, ST) launch_decode_t<DD, IT, ST>(p, (unsigned)blocks, stream)
    if (D == 128 && !io_f32 && !state_bf16) KDA_DECODE(128, bf16, float);
    else if (D == 128 && !io_f32 && state_bf16) KDA_DECODE(128, bf16, bf16);
    else if (D == 128 && io_f32 && !state_bf16) KDA_DECODE(128, float, float);
    else if (D == 128 && io_f32 && state_bf16) KDA_DECODE(128, float, bf16);
    else if (D == 64 && !io_f32 && !state_bf16) KDA_DECODE(64, bf16, float);
    else if (D == 64 && !io_f32 && state_bf16) KDA_DECODE(64, bf16, bf16);
    else if (D == 64 && io_f32 && !state_bf16) KDA_DECODE(64, float, float);
    else if (D == 64 && io_f32 && state_bf16) KDA_DECODE(64, float, bf16);
    else return hipErrorInvalidValue;
#undef KDA_DECODE
    return hipGetLastError();
}

}  // namespace kda
