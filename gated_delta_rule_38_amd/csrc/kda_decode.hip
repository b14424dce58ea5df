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
// Columns of S evolve independently, so one 256-thread workgroup owns one
// 32-column value slab of one (request, head): thread (column c, row group j)
// keeps rows [j D/8, (j+1) D/8) of column c in registers, and the two sums over
// key channels per token (k^T S and q^T S) are reduced across the 8 row groups
// in a fixed order (lane pairs, then the 4 waves through LDS), so results do not
// depend on timing.  The work is the state's round trip through HBM; the few
// tokens are staged in LDS once.  An index outside [0, P) skips the request (no
// output rows, no state write), so a bad index can never address memory.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16>(const bf16 *p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st(T *p, float x);
template <> __device__ __forceinline__ void st<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void st<bf16>(bf16 *p, float x) { *p = (bf16)x; }   // round to nearest even

template <int D, typename IT, typename ST>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p)
{
    constexpr int NSLAB = D / 32, RPG = D / 8, TM = DECODE_MAX_TOKENS;
    __shared__ float sK[TM][D], sQ[TM][D], sE[TM][D], sV[TM][32], sB[TM];
    __shared__ float sRed[2][4][32];
    const int slab = blockIdx.x % NSLAB, rh = blockIdx.x / NSLAB;
    const int h = rh % p.H, r = rh / p.H;
    const int tid = threadIdx.x, c = tid & 31, grp = tid >> 5, wave = tid >> 6;
    const int slot = p.idx[r];
    if (slot < 0 || slot >= p.P) return;
    const int n = p.ntok ? min(max(p.ntok[r], 0), p.T) : p.T;
    const int v0 = 32 * slab;
    const IT *q = (const IT *)p.q + r * p.q_sr + h * p.q_sh;
    const IT *k = (const IT *)p.k + r * p.k_sr + h * p.k_sh;
    const IT *v = (const IT *)p.v + r * p.v_sr + h * p.v_sh + v0;
    const float *g = p.g + r * p.g_sr + h * p.g_sh;
    for (int e = tid; e < n * D; e += 256) {
        const int t = e / D, ch = e % D;
        sK[t][ch] = ld(k + t * p.k_st + ch);
        sQ[t][ch] = ld(q + t * p.q_st + ch);
        const float x = g[t * p.g_st + ch];
        sE[t][ch] = fast_exp(p.gate_act ? gate_act(x, p.gate_lb) : x);
    }
    for (int e = tid; e < n * 32; e += 256) sV[e / 32][e % 32] = ld(v + (e / 32) * p.v_st + e % 32);
    if (tid < n) {
        const float b = p.beta[r * p.b_sr + tid * p.b_st + h * p.b_sh];
        sB[tid] = p.beta_act ? sigmoid_act(b) : b;
    }
    ST *ps = (ST *)p.pool + slot * p.p_sn + h * p.p_sh + (int64_t)(grp * RPG) * p.p_sr + v0 + c;
    float s[RPG];
#pragma unroll
    for (int j = 0; j < RPG; ++j) s[j] = ld(ps + j * p.p_sr);
    __syncthreads();

    IT *o = p.o ? (IT *)p.o + r * p.o_sr + h * p.o_sh + v0 + c : nullptr;
    for (int t = 0; t < n; ++t) {
        // decay, then the read k^T D S of this thread's rows
        float pr = 0.f;
#pragma unroll
        for (int j = 0; j < RPG; ++j) {
            const int i = grp * RPG + j;
            s[j] *= sE[t][i];
            pr += sK[t][i] * s[j];
        }
        pr += __shfl_xor(pr, 32);            // row groups 2w and 2w + 1 of wave w
        if ((tid & 63) < 32) sRed[0][wave][c] = pr;
        __syncthreads();
        const float kS = (sRed[0][0][c] + sRed[0][1][c]) + (sRed[0][2][c] + sRed[0][3][c]);
        const float u = sB[t] * (sV[t][c] - kS);
        float po = 0.f;
#pragma unroll
        for (int j = 0; j < RPG; ++j) {
            const int i = grp * RPG + j;
            s[j] += sK[t][i] * u;
            po += sQ[t][i] * s[j];
        }
        po += __shfl_xor(po, 32);
        if ((tid & 63) < 32) sRed[1][wave][c] = po;
        __syncthreads();
        if (o && tid < 32) st(o + t * p.o_st, (sRed[1][0][c] + sRed[1][1][c]) + (sRed[1][2][c] + sRed[1][3][c]));
    }
    if (p.update) {
#pragma unroll
        for (int j = 0; j < RPG; ++j) st(ps + j * p.p_sr, s[j]);
    }
}

hipError_t launch_decode(const DecodeParams &p, int D, bool io_f32, bool state_bf16, hipStream_t stream)
{
    const int64_t blocks = (int64_t)p.R * p.H * (D / 32);
    if (blocks <= 0) return hipSuccess;
#define KDA_DECODE(DD, IT, ST) hipLaunchKernelGGL((decode_kernel<DD, IT, ST>), dim3((unsigned)blocks), dim3(256), 0, stream, p)
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
