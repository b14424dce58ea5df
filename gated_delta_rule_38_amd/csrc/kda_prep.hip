// PREP kernel: the in-chunk inclusive cumulative sum of the log decays g.
//
// Chunks are `chunk` tokens (the chunk kernel's length) and restart at every sequence start, so a chunk never
// straddles two sequences -- the virtual chunk map, safe across sequence gaps, of the
// cudnn-frontend Hopper KDA prefill PR (#1056, walkthrough).  Virtual chunk v
// maps to (sequence n, chunk j of n) through the running count of
// ceil(len_n / chunk); the packed layout's grid is the host-known bound
// ceil(T_tot / chunk) + N and the surplus workgroups exit at once.  One thread per
// key channel adds the chunk's g values in token order in fp32, the same
// sequential order the chunk kernel's fused scan uses, so both produce the same
// bits.  With gate_act each g is first taken as a logit x and replaced by
// gate_lb * sigmoid(x) (the same device function the fused scans use).
#include <algorithm>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

__global__ __launch_bounds__(128) void prep_kernel(const PrepParams p)
{
    const int v = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, nt = blockDim.x;
    __shared__ int s_scan[128];
    __shared__ int s_found[2];
    int n = -1, j = 0;
    if (!p.cu) {
        n = v / p.chunks_per_seq;
        j = v % p.chunks_per_seq;
        if (n >= p.N) return;
    } else {
        if (tid == 0) { s_found[0] = -1; s_found[1] = 0; }
        __syncthreads();
        int carry = 0;
        for (int base = 0; base < p.N; base += nt) {
            const int s = base + tid;
            const int cnt = (s < p.N) ? (p.cu[s + 1] - p.cu[s] + p.chunk - 1) / p.chunk : 0;
            s_scan[tid] = cnt;
            __syncthreads();
            for (int off = 1; off < nt; off <<= 1) {         // inclusive Hillis-Steele scan
                const int add = (tid >= off) ? s_scan[tid - off] : 0;
                __syncthreads();
                s_scan[tid] += add;
                __syncthreads();
            }
            const int incl = carry + s_scan[tid], excl = incl - cnt;
            if (s < p.N && v >= excl && v < incl) { s_found[0] = s; s_found[1] = v - excl; }
            carry += s_scan[nt - 1];
            __syncthreads();
        }
        __syncthreads();
        n = s_found[0];
        j = s_found[1];
        if (n < 0) return;
    }
    if (tid >= p.D) return;
    int64_t t0, bsel;
    int len;
    seq_range(p.cu, n, p.T, t0, len, bsel);
    const int tok0 = j * p.chunk, L = min(p.chunk, len - tok0);
    const float *src = p.g + bsel * p.g_sb + h * p.g_sh + (t0 + tok0) * p.g_st + tid;
    float *dst = p.gamma + bsel * p.y_sb + h * p.y_sh + (t0 + tok0) * p.y_st + tid;
    float acc = 0.f;
    for (int i = 0; i < L; ++i) {
        const float x = src[(int64_t)i * p.g_st];
        acc = acc + (p.gate_act ? gate_act(x, p.gate_lb) : x);
        dst[(int64_t)i * p.y_st] = acc;
    }
}

// cu_seqlens check (the debug mode): flag = 1 unless cu[0] == 0, cu is non-decreasing and
// cu[N] == T_tot.  One workgroup; every thread folds a strided share, then one OR across it.
__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t *cu, int32_t N, int64_t Ttot, int32_t *flag)
{
    int bad = 0;
    for (int i = threadIdx.x; i < N; i += blockDim.x) bad |= cu[i] > cu[i + 1];
    if (threadIdx.x == 0) bad |= (cu[0] != 0) | ((int64_t)cu[N] != Ttot);
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *flag = bad;
}

hipError_t launch_check_cu(const int32_t *cu, int32_t N, int64_t Ttot, int32_t *flag, hipStream_t st)
{
    hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, st, cu, N, Ttot, flag);
    return hipGetLastError();
}

// g range check (the debug mode): flag = 1 when any element of the token-major view lies
// outside [lo, hi] or is NaN.  Element i of the view is (row r, head h, channel c) with row
// r = b * rows_per_b + t.  A grid-stride loop with one element per thread and step; every
// thread that finds a bad value stores the same 1 (the flag starts at 0).
__global__ __launch_bounds__(256) void check_g_kernel(const CheckG c, int32_t *flag)
{
    const int64_t total = c.rows * c.H * c.D;
    int bad = 0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = i % c.D, rh = i / c.D;
        const int64_t h = rh % c.H, r = rh / c.H;
        const int64_t b = r / c.rows_per_b, t = r % c.rows_per_b;
        const float x = c.g[b * c.sb + t * c.st + h * c.sh + ch];
        bad |= !(x >= c.lo && x <= c.hi);
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) *flag = 1;
}

hipError_t launch_check_g(const CheckG &c, int32_t *flag, hipStream_t st)
{
    const int64_t total = c.rows * c.H * c.D;
    if (total <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(check_g_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, flag);
    return hipGetLastError();
}

// Decode slot check (the debug mode): flag = 1 when two requests name the same slot in
// [0, P) (with the state update on, both would write it).  Thread i compares its slot with
// every later request's, the indices staged in LDS 256 at a time: O(R^2) comparisons.
__global__ __launch_bounds__(256) void check_slots_kernel(const int32_t *idx, int32_t R, int32_t P, int32_t *flag)
{
    __shared__ int32_t tile[256];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int vi = (i < R) ? idx[i] : -1;
    const bool valid = vi >= 0 && vi < P;
    int bad = 0;
    for (int base = 0; base < R; base += 256) {
        __syncthreads();
        tile[threadIdx.x] = (base + (int)threadIdx.x < R) ? idx[base + threadIdx.x] : -1;
        __syncthreads();
        if (valid) {
            const int jn = min(256, R - base);
            for (int j = 0; j < jn; ++j) bad |= (base + j > i) & (tile[j] == vi);
        }
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) *flag = 1;
}

hipError_t launch_check_slots(const int32_t *idx, int32_t R, int32_t P, int32_t *flag, hipStream_t st)
{
    if (R <= 1) return hipSuccess;
    hipLaunchKernelGGL(check_slots_kernel, dim3((R + 255) / 256), dim3(256), 0, st, idx, R, P, flag);
    return hipGetLastError();
}

hipError_t launch_prep(const PrepParams &p, int nvc, hipStream_t st)
{
    if (nvc <= 0 || p.H <= 0) return hipSuccess;
    hipLaunchKernelGGL(prep_kernel, dim3(nvc, p.H), dim3(128), 0, st, p);
    return hipGetLastError();
}

}  // namespace kda
