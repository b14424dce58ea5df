// Pipelined CHUNK kernel for d_k = d_v = 128, bf16: the production path.
//
// Same mathematics as kda_chunk.hip (the WY/UT chunk form of the gated delta
// rule; see the comment there), with 32-token chunks and the work of a chain
// split between two wave roles of one 512-thread workgroup:
//   * 4 consumer waves own the fp32 128x128 state -- wave w keeps value columns
//     [32w, 32w+32) in MFMA accumulators for the whole chain -- and run the
//     state path of chunk c:
//         R = V - Kt S,   U = (T diag(beta)) R,   O = Qt S + P U,
//         S <- Diag(e^{G_L}) S + Kh^T U
//     (U = T diag(beta) (V - Kt S) is the UT form's U = Ut - W S with
//     Ut = T diag(beta) V and W = T diag(beta) Kt folded together, so W is
//     never formed);
//   * 4 producer waves meanwhile build the state-independent operators of the
//     next chunk: the in-chunk gate scan, A and P on 16x16 MFMA tiles, and the
//     diagonal blocks of T diag(beta), T = (I + A)^-1.  The gate-factored operands
//     are built by all 8 waves (consumers: gate sub-block 0, producers: sub-block 1),
//     and the off-diagonal block of T diag(beta) is finished a step later by
//     consumer wave 0: the consumers' own share of interval 1 is short.
// The roles meet in a double buffer in LDS.  Step t: the producers build chunk
// t into buffer t%2 while the consumers run chunk t-1 from buffer (t-1)%2.
// Every wave executes the same two workgroup barriers per step; no buffer is
// written before the barrier that ends the last read of its previous contents
// (the reader/writer ordering TensorRT-LLM PR #19826 had to add to its fused
// prefill between a chunk's readers and the next chunk's writers).  A VALU-heavy
// producer wave and an MFMA-heavy consumer wave share each SIMD.
//
//   interval 1: all waves -- gate-factored operands of chunk t; q, k, v of t+1 requested
//               producers -- raw g of t+1 staged, g of t+2 requested
//               consumers -- R of chunk t-1; wave 0 also the off-diagonal block of
//               T diag(beta) of chunk t-1
//   interval 2: producer waves 0, 2 -- A (0,0), A (1,1) and the diagonal blocks of
//               T diag(beta) of chunk t; waves 1, 3 -- the other A and P tiles, then
//               the gate scan of chunk t+1
//               consumers -- U and O of chunk t-1 (O stored), then the state update
//
// 32-token chunks hold two 16-token gate sub-blocks: diagonal sub-blocks factor
// the decay through the block start (factors within [e^-80, e^80] for g >= -5),
// the off-diagonal one through the last token of block 0 (factors <= 1).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace pipe {

constexpr int C = 32;           // tokens per chunk
constexpr int D = 128;
constexpr int NT = 512;         // 4 consumer + 4 producer waves
// leading dimensions (elements); padding matches each tile's read width
constexpr int W_LD = D + 4;     // Qt, -Kt [32][128] bf16, 8-byte reads
constexpr int KR_LD = D + 32;   // Kh, V [32][128] bf16, row-major, read transposed (4 rows x 32 B per 16 lanes;
                                // this stride makes those reads free of LDS bank conflicts)
constexpr int P_LD = C + 4;     // P, T diag(beta) [32][32] bf16, 8-byte reads
constexpr int G_LD = D + 4;     // Gamma * log2(e) [32][128] fp32
constexpr int X_LD = D + 16;    // X, Y, Z, Kb [rows][128] bf16, 16-byte reads (bank-conflict free at this stride)
constexpr int A_LD = 16 + 4;    // 16x16 blocks: A10 (bf16), A diagonal (fp32), T_00 (fp32), T_11 (bf16)
// one operand buffer (bytes)
constexpr int B_QT = 0;
constexpr int B_KT = B_QT + C * W_LD * 2;
constexpr int B_KH = B_KT + C * W_LD * 2;
constexpr int B_V = B_KH + C * KR_LD * 2;
constexpr int B_P = B_V + C * KR_LD * 2;
constexpr int B_T = B_P + C * P_LD * 2;
constexpr int B_SIZE = B_T + C * P_LD * 2;
// producer scratch
constexpr int S_G = 2 * B_SIZE;
constexpr int GT_LD = C + 4;    // raw g staged transposed [128 channels][32 tokens] fp32
constexpr int S_GRAW = S_G + C * G_LD * 4;   // raw g of the next chunk, staged for the scan
constexpr int S_X = S_GRAW + D * GT_LD * 4;
constexpr int S_Y = S_X + C * X_LD * 2;
constexpr int S_Z = S_Y + C * X_LD * 2;
constexpr int S_KB = S_Z + C * X_LD * 2;
constexpr int S_A10 = S_KB + 16 * X_LD * 2;
constexpr int S_AD = S_A10 + 16 * A_LD * 2;
constexpr int S_TB = S_AD + 2 * 16 * A_LD * 4;   // T_00, T_11 (bf16) for the off-diagonal product
constexpr int S_SC = S_TB + 2 * 16 * A_LD * 2;
constexpr int S_DEC = S_SC + 2 * D * 4;       // chunk decays e^{G_L}: a ring of 3 chunks
constexpr int S_BETA = S_DEC + 3 * D * 4;     // beta: a ring of 3 chunks
constexpr int SMEM = S_BETA + 3 * C * 4;
// output norm: per-token partial sums of squares of the 4 consumer waves, and the norm weight
constexpr int S_NRM = SMEM;
constexpr int S_NW = S_NRM + C * 4 * 4;
constexpr int SMEM_NORM = S_NW + D * 4;
static_assert(SMEM_NORM <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
// capped concurrency: its packing scratch, after the norm's sums
constexpr int S_CAP = SMEM_NORM;
constexpr int SMEM_CAP = S_CAP + 4 * (3 * CAP_MAX_N + 2 * CAP_MAX_SLOTS + 4);
static_assert(SMEM_CAP <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
static_assert(4 * (LPT_MAX_SEQ + 1) <= B_SIZE, "longest-first scratch fits in operand buffer 0");
static_assert(B_SIZE % 16 == 0 && S_GRAW % 16 == 0 && S_X % 16 == 0 && S_A10 % 16 == 0 && S_AD % 16 == 0 && S_TB % 16 == 0 &&
              S_SC % 16 == 0 && S_DEC % 16 == 0 && S_BETA % 16 == 0, "16-byte aligned regions");

typedef Vec4<bf16> V4;
typedef Vec4<float> V4f;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Index of the sequence of rank r when the N sequences of a packed batch are ordered longest
// first (ties: lower index first), so that a launch with more chains than CUs starts its
// longest chains first and its short ones fill in behind them.  Every thread of the workgroup
// calls it (it holds three barriers) and gets the result.  Its scratch, the first 4 (N + 1)
// bytes of LDS, is written next only after the barriers that start the main loop.
__device__ int longest_first(const int32_t *cu, int N, int r, char *smem)
{
    int *sLen = (int *)smem;
    for (int i = threadIdx.x; i < N; i += NT) sLen[i] = cu[i + 1] - cu[i];
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += NT) {
        const int li = sLen[i];
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = sLen[j];
            rank += (lj > li) | ((lj == li) & (j < i));
        }
        if (rank == r) sLen[N] = i;     // the ranks are a permutation: exactly one writer
    }
    __syncthreads();
    const int n = sLen[N];
    __syncthreads();
    return n;
}

// Capped concurrency: the step time of this kernel hardly depends on how many chains run at
// once up to about 160 of 256 CUs and then climbs (the clock and HBM under full load), while a
// packed batch of mixed lengths ends with its longest chain.  So the sequences are packed,
// longest first, into groups of H workgroups (each into the least-loaded group; the
// per-sequence cost is its chunks plus 3 for the pipeline's fill): the fewest groups, from
// cap_slots up, with which the longest sequence alone still bounds the packing.  A workgroup
// whose sequence follows another one in its group then waits for that sequence's chain of the
// same head to finish before its main loop.
// Every chain is resident at once (chains <= CUs), so a predecessor is always running; the
// wait is bounded all the same, and it orders no data.  Every thread calls it at the same
// point of its prologue (after its first loads are issued, so their latency overlaps); thread
// i < N brings sequence i's length in tokens; sc is the dedicated scratch (S_CAP).
//
// A chain's flag holds the call's value (low word) and a count (high word).  Thread 0 returns
// the flag this chain stores when it finishes: the call's value with its previous count plus
// one when the flag already holds this call's value (a graph replaying the same captured call,
// whose chains all replay together), else with count 1.  A waiting workgroup waits for its
// predecessor's flag to reach that same value.
__device__ uint64_t cap_wait(const ChunkParams &p, int n, int h, int len_i, char *sc)
{
    const int N = p.N, S = p.cap_slots;
    int *sLen = (int *)sc, *sOrd = sLen + CAP_MAX_N, *sPred = sOrd + CAP_MAX_N, *sLoad = sPred + CAP_MAX_N;
    int *sLast = sLoad + CAP_MAX_SLOTS, *sOk = sLast + CAP_MAX_SLOTS;
    uint64_t next = 0;
    if (threadIdx.x == 0) {
        const uint64_t own = __hip_atomic_load(p.cap_flags + (int64_t)n * p.H + h, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t count = ((uint32_t)own == p.cap_epoch) ? (uint32_t)(own >> 32) + 1u : 1u;
        next = ((uint64_t)count << 32) | p.cap_epoch;
    }
    if ((int)threadIdx.x < N) sLen[threadIdx.x] = (len_i + C - 1) / C + 3;
    __syncthreads();
    if ((int)threadIdx.x < N) {
        const int i = threadIdx.x, li = sLen[i];
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = sLen[j];
            rank += (lj > li) | ((lj == li) & (j < i));
        }
        sOrd[rank] = i;                 // the ranks are a permutation
        if (i == n) sOk[0] = rank;
    }
    __syncthreads();
    // the S longest sequences open the groups: their workgroups (the ones that bound the call)
    // skip the packing.  The others pack with S groups, then S + 1, ... (fewer than N) until the
    // longest sequence alone still bounds the packing; none of those counts: no wait
    if (threadIdx.x == 0 && sOk[0] >= S) {
        int pred = -1;
        for (int G = S; G < N && G <= CAP_MAX_SLOTS; ++G) {
            for (int g = 0; g < G; ++g) {
                sLoad[g] = 0;
                sLast[g] = -1;
            }
            for (int r = 0; r < N; ++r) {
                const int i = sOrd[r];
                int best = 0;
                for (int g = 1; g < G; ++g) best = sLoad[g] < sLoad[best] ? g : best;
                sPred[i] = sLast[best];
                sLast[best] = i;
                sLoad[best] += sLen[i];
            }
            int most = 0;
            for (int g = 0; g < G; ++g) most = max(most, sLoad[g]);
            if (most <= sLen[sOrd[0]] + 2) {
                pred = sPred[n];
                break;
            }
        }
        if (pred >= 0) {
            // bound: the given one, else 8 us per chunk of the predecessor plus 2 ms (100 MHz ticks)
            const uint64_t limit = 100ull * (p.cap_wait_us > 0 ? (uint64_t)p.cap_wait_us
                                                                  : 8ull * (uint64_t)sLen[pred] + 2000ull);
            const uint64_t *f = p.cap_flags + (int64_t)pred * p.H + h;
            const uint64_t ts = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != next &&
                   __builtin_amdgcn_s_memrealtime() - ts < limit)
                __builtin_amdgcn_s_sleep(32);
        }
    }
    __syncthreads();
    return next;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane 4a+b receives
// 16-bit element b of the 8-byte words addressed by lanes a, a+4, a+8, a+12 of the group.
__device__ __forceinline__ uint2 lds_tr16(const bf16 *p)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
    return __builtin_bit_cast(uint2, v);
}

// x += a[lane J of this lane's 16-lane row] * t: one v_fmac with a DPP row broadcast of a.
// (The compiler does not fold a row-broadcast move into its FMA, and keeping the broadcast
// values in registers of their own would cost 120 of them.)  The DPP source a is only ever
// loaded from LDS, never written by a VALU instruction, so no DPP read-after-VALU-write wait
// states are needed.
template <int J>
__device__ __forceinline__ void fmac_row_bcast(float &x, float a, float t)
{
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(x) : "v"(a), "v"(t), "i"(J));
}

// Columns J, J-1, ..., 1 of the downward sweep of the 16x16 T solve: x is this lane's row
// of T, a this lane's row of A; row J of A comes from lane J of the block.
template <int J>
__device__ __forceinline__ void tsweep(float (&x)[16], const float (&a)[16])
{
    const float ntj = -x[J];
#pragma unroll
    for (int c = J - 1; c >= 0; --c) fmac_row_bcast<J>(x[c], a[c], ntj);   // column J-1 first: the next pivot
    if constexpr (J > 1) tsweep<J - 1>(x, a);
}

// The decay of one 32x32 state tile: accumulator element 4q + r (row 32M + 8q + 4g + r, g the
// lane's half) times element r of dd on lane 4M + q of the lane's 16-lane row, by DPP row
// broadcast -- every lane loads dd = decays 8 l16 + 4g + 0..3, so a 16-lane row holds the 64
// decays its half of the tile needs.  dd comes straight from LDS (no VALU write before the DPP
// read).  The closing s_nop gives the two wait states a matrix-core read of the tile needs after
// a VALU write, which the compiler does not insert after inline assembly.
template <int M>
__device__ __forceinline__ void decay_tile(f32x16 &s, const float4 dd)
{
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = s[k];
    asm(
        "v_mul_f32_dpp %0, %16, %0 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %1, %17, %1 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %2, %18, %2 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %3, %19, %3 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %4, %16, %4 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %5, %17, %5 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %6, %18, %6 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %7, %19, %7 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %8, %16, %8 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %9, %17, %9 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %10, %18, %10 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %11, %19, %11 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %12, %16, %12 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %13, %17, %13 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %14, %18, %14 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %15, %19, %15 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n"
        "s_nop 1"
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]),
          "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]), "+v"(x[14]), "+v"(x[15])
        : "v"(dd.x), "v"(dd.y), "v"(dd.z), "v"(dd.w), "i"(4 * M), "i"(4 * M + 1), "i"(4 * M + 2), "i"(4 * M + 3));
#pragma unroll
    for (int k = 0; k < 16; ++k) s[k] = x[k];
}

// OUT: the launch's roles store outputs (ROLE_OUT, ROLE_SEG_OUT); the segment-map roles do
// not, and skip everything that only feeds O: q, Qt, the P tiles and the O products.
// NORM (with OUT): the output rows pass through the gated RMS norm before they are written.
// A token's row spans the 4 consumer waves, so each wave leaves its partial sum of squares
// in LDS and keeps its O tile in registers across the step's barrier; the next interval 1
// (or, for the last chunk, the end of the chain) normalises and stores it.
// MC (without OUT): the segment-map role ROLE_SEG_MC -- the consumer waves carry both maps of
// the segment on their 32 value columns, C (start state 0, V as given) and M (start state I,
// V = 0), from the same operands: each fragment of Kt, T diag(beta) and Kh read from LDS feeds
// the product of both.  One workgroup then builds both maps of a segment.
template <bool STALL, bool OUT, bool NORM, bool MC>
__global__ __launch_bounds__(NT, 1) void chunk_pipe_kernel(const ChunkParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[(OUT && !MC) ? SMEM_CAP : SMEM];
    float *sG = (float *)(smem + S_G), *sGraw = (float *)(smem + S_GRAW);
    bf16 *sX = (bf16 *)(smem + S_X), *sY = (bf16 *)(smem + S_Y), *sZ = (bf16 *)(smem + S_Z);
    bf16 *sKb = (bf16 *)(smem + S_KB), *sA10 = (bf16 *)(smem + S_A10);
    float *sAd = (float *)(smem + S_AD);
    bf16 *sTb = (bf16 *)(smem + S_TB);
    float *sSc = (float *)(smem + S_SC), *sDec = (float *)(smem + S_DEC);
    float *sBeta = (float *)(smem + S_BETA);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l32 = lane & 31, g2 = lane >> 5, l16 = lane & 15, g4 = lane >> 4;
    const bool producer = wave >= 4;

    const int stall_iters = (STALL && wave == p.stall_wave) ? p.stall_iters : 0;   // wave-uniform
    auto sync = [&]() {
        __syncthreads();
        if constexpr (STALL) {
            for (int s = 0; s < stall_iters; ++s) __builtin_amdgcn_s_sleep(127);
        }
    };

    // T diag(beta) of one chunk from its A and beta, into pT, in two parts, each run by one
    // wave: the diagonal 16x16 blocks (from sAd; also leaves T_00 and T_11 in sTb) and, a
    // step later, the off-diagonal block (from sA10 and sTb).
    auto build_T_diag = [&](const int b, const float (&bt)[16], bf16 *pT) {
        // Diagonal 16x16 block b of T = (I + A)^-1, one row per lane (each 16-lane group
        // holds the whole block).  T = I - T A gives, for row i, T_ic = [i == c] -
        // sum_{j > c} T_ij A_jc, so column j of the row is final once the columns after it
        // are folded in: sweeping j downwards, each final T_ij is folded into the remaining
        // columns with row j of A.  Each lane keeps its own row of A in registers; row j
        // reaches the other lanes of the group by a DPP broadcast from lane j of the 16-lane
        // row, so the sweep makes no LDS access.
        const int i = l16;
        float a[16], x[16];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const float4 a4 = *(const float4 *)(sAd + (16 * b + i) * A_LD + 4 * c4);
            a[4 * c4] = a4.x; a[4 * c4 + 1] = a4.y; a[4 * c4 + 2] = a4.z; a[4 * c4 + 3] = a4.w;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) x[c] = (c == i) ? 1.f : 0.f;
        tsweep<15>(x, a);
        // One branch-free store sequence: lanes 0-31 write row 16b+i of T diag(beta) (its
        // diagonal block, and zeros over the other 16 columns -- block (0,1) is zero, block
        // (1,0) is written a step later); lanes 32-63 write the unscaled row to sTb.  Lanes
        // 16-31 and 48-63 repeat the stores of lanes 0-15 and 32-47.
        const bool hi = lane >= 32;
        bf16 *dst0 = hi ? sTb + (16 * b + i) * A_LD : pT + (16 * b + i) * P_LD + 16 * b;
        bf16 *dst1 = pT + (16 * b + i) * P_LD + 16 * (1 - b);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            float tb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) tb[e] = hi ? x[4 * c4 + e] : x[4 * c4 + e] * bt[4 * c4 + e];
            V4::store(dst0 + 4 * c4, V4::pack(tb));
            V4::store(dst1 + 4 * c4, V4::zero());
        }
    };
    auto build_T_off = [&](const float *betac, bf16 *pT) {
        // Off-diagonal block T_10 = -T_11 (A_10 T_00), formed transposed so that each lane
        // ends with four consecutive entries of one row: Y = A_10 T_00 (lane = column of Y),
        // then Y^T T_11^T = -T_10^T, whose accumulator puts row l16 of T_10 in lane l16.
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
        Frag4<bf16> fa, fb;
        fa.load4(sA10 + l16 * A_LD + 4 * g4);
        // T_00 columns: rows 4*g4..4*g4+3 of column l16, by one transposing read
        fb.v = __builtin_bit_cast(s16x4, lds_tr16(sTb + (4 * g4 + (l16 >> 2)) * A_LD + 4 * (l16 & 3)));
        mma16k16(Y, fa, fb);
        Frag4<bf16> fy, ft;
        {
            const float y4[4] = {Y[0], Y[1], Y[2], Y[3]};
            fy.set(y4);
        }
        ft.load4(sTb + (16 + l16) * A_LD + 4 * g4);
        f32x4 Z = {0.f, 0.f, 0.f, 0.f};
        mma16k16(Z, fy, ft);
        const float4 b4 = *(const float4 *)(betac + 4 * g4);
        const float z4[4] = {-Z[0] * b4.x, -Z[1] * b4.y, -Z[2] * b4.z, -Z[3] * b4.w};
        V4::store(pT + (16 + l16) * P_LD + 4 * g4, V4::pack(z4));
    };

    // ------------------------------------------------ chain / segment
    // chain: the (sequence, head) chain; lchain: its workspace slot among the segmented chains;
    // nseg: the segments of this chain (1 for a chain run whole)
    const int wg = blockIdx.x;
    int role = p.role, nseg = p.nseg, seg = 0, chain, lchain = 0;
    if (role == ROLE_SEG_MC) {          // maps of segments 0 .. nseg - 2 (COMBINE never reads the last's)
        lchain = wg / (nseg - 1);
        seg = wg % (nseg - 1);
        chain = p.seg_chain0 + lchain;
    } else if (role == ROLE_SEG_OUT && wg < p.n_segwg) {
        lchain = wg / nseg;
        seg = wg % nseg;
        chain = p.seg_chain0 + lchain;
    } else {                            // a whole chain (the launch's trailing workgroups in a split plan)
        chain = (role == ROLE_SEG_OUT) ? wg - p.n_segwg : wg;
        role = ROLE_OUT;
        nseg = 1;
    }
    const int h = chain % p.H;
    const int n = p.lpt ? longest_first(p.cu, p.N, chain / p.H, smem) : chain / p.H;
    const bool capped = OUT && !MC && role == ROLE_OUT && p.cap_slots > 0;
    int cap_len = 0;                    // capped: sequence tid's length (threads tid < N), for cap_wait
    if (capped && tid < p.N) cap_len = p.cu[tid + 1] - p.cu[tid];
    int64_t t0, bsel;
    int len;
    seq_range(p.cu, n, p.T, t0, len, bsel);
    const int nchunks = (len + C - 1) / C;
    const int cps = (nchunks + nseg - 1) / nseg;
    const int c_begin = min(seg * cps, nchunks);
    const int c_end = min(c_begin + cps, nchunks);
    const int nck = c_end - c_begin;
    constexpr bool has_out = OUT;

    // ------------------------------------------------ gate-factored operands (all waves)
    // Thread tid handles tokens 2*(tid>>5) and 2*(tid>>5)+1, channels 4*(tid&31)..+3 of a
    // chunk: the consumer waves gate sub-block 0, the producer waves sub-block 1.
    const int etp = tid >> 5, ech = 4 * (tid & 31);
    const char *qb = (const char *)p.q + 2 * (bsel * p.q_sb + h * p.q_sh + t0 * p.q_st);
    const char *kb = (const char *)p.k + 2 * (bsel * p.k_sb + h * p.k_sh + t0 * p.k_st);
    const char *vb = (const char *)p.v + 2 * (bsel * p.v_sb + h * p.v_sh + t0 * p.v_st);
    // Each load addresses a uniform chunk base plus a 32-bit per-lane byte offset (the host
    // keeps a chunk's rows within 2^31 bytes).  Rows past a short chunk's end re-read its last
    // row: with non-negative strides, min(row, L-1) * stride = min(row * stride, (L-1) * stride).
    const uint32_t qst = 2 * (uint32_t)p.q_st, kst = 2 * (uint32_t)p.k_st, vst = 2 * (uint32_t)p.v_st;
    const uint32_t qro = 2 * etp * qst + 2 * ech, kro = 2 * etp * kst + 2 * ech, vro = 2 * etp * vst + 2 * ech;
    uint2 rq[2], rk[2], rv[2];          // 2 tokens x 4 channels of q, k, v (bf16)
    auto prefetch_qkv = [&](int c) {
        const int tok0 = c * C, Lm1 = min(C, len - tok0) - 1;
        const char *qc = qb + (int64_t)tok0 * qst, *kc = kb + (int64_t)tok0 * kst, *vc = vb + (int64_t)tok0 * vst;
        const uint32_t ql = Lm1 * qst + 2 * ech, kl = Lm1 * kst + 2 * ech, vl = Lm1 * vst + 2 * ech;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if constexpr (OUT) rq[r] = *(const uint2 *)(qc + min(qro + r * qst, ql));
            rk[r] = *(const uint2 *)(kc + min(kro + r * kst, kl));
            rv[r] = *(const uint2 *)(vc + min(vro + r * vst, vl));
        }
    };
    // B1: sub-block 1.  Rows past a short chunk's end hold finite copies of token L-1: with
    // beta = 0 there, T diag(beta) has zero rows and columns, so they enter U, O and S only
    // through exact zeros and need no masking.
    auto operands = [&](auto b1_tag, char *PB) {
        constexpr bool B1 = decltype(b1_tag)::value;
        bf16 *pQt = (bf16 *)(PB + B_QT), *pKt = (bf16 *)(PB + B_KT), *pKh = (bf16 *)(PB + B_KH);
        bf16 *pV = (bf16 *)(PB + B_V);
        float4 E1 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (B1) E1 = *(const float4 *)(sG + 15 * G_LD + ech);
        const float4 e15 = *(const float4 *)(sSc + 0 * D + ech);
        const float4 sl = *(const float4 *)(sSc + 1 * D + ech);
        const float E1v[4] = {E1.x, E1.y, E1.z, E1.w}, e15v[4] = {e15.x, e15.y, e15.z, e15.w};
        const float slv[4] = {sl.x, sl.y, sl.z, sl.w};
        float kh[2][4];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = 2 * etp + r;
            const float4 Gv = *(const float4 *)(sG + i * G_LD + ech);
            const float G4[4] = {Gv.x, Gv.y, Gv.z, Gv.w};
            float qf[4] = {0.f, 0.f, 0.f, 0.f}, kf[4];
            if constexpr (OUT) V4::unpack(rq[r], qf);
            V4::unpack(rk[r], kf);
            float X[4], Y[4], Z[4], Kb[4], Qt[4], Kt[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = __builtin_amdgcn_exp2f(G4[e] - E1v[e]);   // e^{G_i - E_b}, in [e^-80, 1]
                const float rr = fast_rcp(f);                             // e^{E_b - G_i}, in [1, e^80]
                X[e] = kf[e] * f;
                Y[e] = qf[e] * f;
                Z[e] = kf[e] * rr;
                if (!B1) {
                    Kb[e] = Z[e] * e15v[e];              // k e^{G_15 - G_i} <= 1
                    kh[r][e] = Kb[e] * slv[e];           // k e^{G_L - G_i}
                    Kt[e] = -X[e];                       // -k e^{G_i}
                    Qt[e] = Y[e];                        // q e^{G_i}
                } else {
                    kh[r][e] = Z[e] * slv[e];
                    Qt[e] = Y[e] * e15v[e];
                    Kt[e] = -(X[e] * e15v[e]);
                }
            }
            const uint2 Xp = V4::pack(X);
            V4::store(sX + i * X_LD + ech, Xp);
            V4::store(sZ + i * X_LD + ech, V4::pack(Z));
            // sub-block 0: -Kt is X, negated exactly by flipping the bf16 sign bits
            V4::store(pKt + i * W_LD + ech, B1 ? V4::pack(Kt) : make_uint2(Xp.x ^ 0x80008000u, Xp.y ^ 0x80008000u));
            if constexpr (OUT) {
                V4::store(sY + i * X_LD + ech, V4::pack(Y));
                V4::store(pQt + i * W_LD + ech, V4::pack(Qt));
            }
            if (!B1) V4::store(sKb + i * X_LD + ech, V4::pack(Kb));
        }
        // Kh and V rows, row-major like Qt and Kt (the consumers read them transposed)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            V4::store(pKh + (2 * etp + r) * KR_LD + ech, V4::pack(kh[r]));
            V4::store(pV + (2 * etp + r) * KR_LD + ech, rv[r]);
        }
    };
    const int c_last = c_end - 1;

    if (producer) {
        // ============================================ producer waves
        const int pt = tid - 256, pw = wave - 4;
        const int sc = (pw == 1) ? lane : (pw == 3) ? 64 + lane : -1;   // scan threads (waves 5, 7): one key channel each
        const char *gb = (const char *)(p.g + bsel * p.g_sb + h * p.g_sh + t0 * p.g_st);
        const char *bb = (const char *)(p.beta + bsel * p.b_sb + h * p.b_sh + t0 * p.b_st);

        float rgv[16];                  // g of tokens 4*gq..4*gq+3 x channels 4*gc..4*gc+3
        float rbeta;                    // beta of token gc
        const int gq = pt >> 5, gc = pt & 31;
        const uint32_t gst = 4 * (uint32_t)p.g_st, bst = 4 * (uint32_t)p.b_st;
        const uint32_t gro = 4 * gq * gst + 16 * gc, bro = gc * bst;
        // Every thread of a role issues the same loads, from always in-bounds addresses (the
        // rows of a short last chunk re-read its last token; chunks past the segment's end
        // re-read its last chunk), all in interval 1, and consumes them at the start of the
        // next step's interval 1.  Whatever wait the compiler places before a use then only
        // covers loads issued a whole step earlier: its bookkeeping of outstanding loads
        // across the loop's branches is conservative, and a wait that also covered younger
        // loads would expose their full memory latency.
        auto prefetch_g = [&](int c) {
            const int tok0 = c * C, Lm1 = min(C, len - tok0) - 1;
            const char *gcb = gb + (int64_t)tok0 * gst, *bcb = bb + (int64_t)tok0 * bst;
            const uint32_t gl = Lm1 * gst + 16 * gc;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 v = *(const float4 *)(gcb + min(gro + k * gst, gl));
                rgv[4 * k] = v.x; rgv[4 * k + 1] = v.y; rgv[4 * k + 2] = v.z; rgv[4 * k + 3] = v.w;
            }
            rbeta = *(const float *)(bcb + min(bro, Lm1 * bst));
        };
        // Raw g of chunk c (the t-th of this segment) into the staging buffer, transposed: channel
        // row ch holds its 32 tokens as 8 groups of 4, group k at slot k ^ ((ch >> 4) & 7), which
        // keeps both these 16-byte stores and the scan's 16-byte row reads free of bank conflicts.
        // Beta goes into ring slot t % 3.
        auto stage_g = [&](int c, int t) {
            const int L = min(C, len - c * C);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = 4 * gc + e;
                *(float4 *)(sGraw + ch * GT_LD + 4 * (gq ^ ((ch >> 4) & 7))) =
                    make_float4(rgv[e], rgv[4 + e], rgv[8 + e], rgv[12 + e]);
            }
            if (pt < C) sBeta[(t % 3) * C + pt] = (pt < L) ? (p.beta_act ? sigmoid_act(rbeta) : rbeta) : 0.f;
        };
        // gate scan of the staged chunk c (the t-th of this segment) into Gamma * log2(e),
        // plus the per-channel scales and decay ring slot t % 3
        auto scan_load = [&](float4 (&gcol)[C / 4]) {
#pragma unroll
            for (int k = 0; k < C / 4; ++k) gcol[k] = *(const float4 *)(sGraw + sc * GT_LD + 4 * (k ^ ((sc >> 4) & 7)));
        };
        auto scan = [&](int c, int t, const float4 (&gcol)[C / 4]) {
            const int L = min(C, len - c * C);
            if (sc >= 0) {
                float rg[C];
#pragma unroll
                for (int k = 0; k < C / 4; ++k) {
                    const float4 v = gcol[k];
                    rg[4 * k] = v.x; rg[4 * k + 1] = v.y; rg[4 * k + 2] = v.z; rg[4 * k + 3] = v.w;
                }
                // logits in: the decays lb * sigmoid(x), before the sum
                if (p.gate_act && !p.g_is_gamma) {
#pragma unroll
                    for (int i = 0; i < C; ++i) rg[i] = gate_act(rg[i], p.gate_lb);
                }
                // tail rows re-read token L-1 (clamped loads), so a precomputed Gamma needs
                // no select there; the cumsum skips them so they hold Gamma_{L-1}
                if (p.g_is_gamma) {
#pragma unroll
                    for (int i = 0; i < C; ++i) rg[i] *= LOG2E;
                } else if (L == C) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < C; ++i) {
                        acc += rg[i];                                   // fp32 adds in token order
                        rg[i] = acc * LOG2E;
                    }
                } else {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < C; ++i) {
                        acc += (i < L) ? rg[i] : 0.f;
                        rg[i] = acc * LOG2E;
                    }
                }
#pragma unroll
                for (int i = 0; i < C; ++i) sG[i * G_LD + sc] = rg[i];
                sSc[0 * D + sc] = __builtin_amdgcn_exp2f(rg[15]);              // e^{G_15}
                sSc[1 * D + sc] = __builtin_amdgcn_exp2f(rg[31] - rg[15]);     // e^{G_L - G_15}
                sDec[(t % 3) * D + sc] = __builtin_amdgcn_exp2f(rg[31]);             // e^{G_L}
            }
        };
        if (nck > 0) {
            prefetch_g(c_begin);
            prefetch_qkv(c_begin);
            stage_g(c_begin, 0);
            prefetch_g(min(c_begin + 1, c_last));
        }
        if (capped) cap_wait(p, n, h, cap_len, smem + S_CAP);
        sync();
        if (nck > 0 && sc >= 0) {
            float4 gcol[C / 4];
            scan_load(gcol);
            scan(c_begin, 0, gcol);
        }
        sync();
        for (int t = 0; nck > 0 && t <= nck; ++t) {
            const bool pact = t < nck;                           // builds chunk c_begin + t into buffer t % 2
            const int cur = t & 1;
            char *PB = smem + cur * B_SIZE;
            bf16 *pP = (bf16 *)(PB + B_P), *pT = (bf16 *)(PB + B_T);
            const int pc = c_begin + t;
            const bool more = t + 1 < nck;
            const float *betac = sBeta + (t % 3) * C;
            // ---------------- interval 1: gate-factored operands of chunk t; g of t+1 staged
            stage_g(min(pc + 1, c_last), t + 1);
            prefetch_g(min(pc + 2, c_last));
            if (pact) operands(std::true_type{}, PB);
            prefetch_qkv(min(pc + 1, c_last));
            sync();
            // ---------------- interval 2: A^T and P^T sub-tiles (16x16, k = 128), diagonal T blocks
            //                  of chunk t; gate scan of chunk t+1
            // 16x16 tile of A^T (mat 0: rows i scaled by beta_i, strictly lower) or P^T (mat 1:
            // lower including the diagonal) for row block ib, column block jb.  A wave first issues
            // every LDS read of its interval-2 work, then computes: its reads then wait in the
            // LDS queue once, not once per dependent step.
            struct TileOps { Frag8<bf16> fa[D / 32], fb[D / 32]; };
            auto tile_load = [&](int mat, int ib, int jb, TileOps &o) {
                const bf16 *arow = ((ib == jb) ? sZ : sKb) + (16 * jb + l16) * X_LD;
                const bf16 *brow = (mat ? sY : sX) + (16 * ib + l16) * X_LD;
#pragma unroll
                for (int s = 0; s < D / 32; ++s) {
                    o.fa[s].load8(arow + 32 * s + 8 * g4);
                    o.fb[s].load8(brow + 32 * s + 8 * g4);
                }
            };
            auto tile = [&](int mat, int ib, int jb, const TileOps &o, float sc_i, float (&vals)[4]) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < D / 32; ++s) mma16(acc, o.fa[s], o.fb[s]);
                const int i = 16 * ib + l16, j0 = 16 * jb + 4 * g4;
#pragma unroll
                for (int r = 0; r < 4; ++r) vals[r] = (j0 + r < i + mat) ? acc[r] * sc_i : 0.f;
            };
            if (pw == 0 || pw == 2) {
                // wave 0 -> A (0,0) then T_00, wave 2 -> A (1,1) then T_11
                if (pact) {
                    const int b = pw >> 1;
                    TileOps o;
                    tile_load(0, b, b, o);
                    float bt[16];
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const float4 b4 = *(const float4 *)(betac + 16 * b + 4 * c4);
                        bt[4 * c4] = b4.x; bt[4 * c4 + 1] = b4.y; bt[4 * c4 + 2] = b4.z; bt[4 * c4 + 3] = b4.w;
                    }
                    const float sc_i = betac[16 * b + l16];
                    __builtin_amdgcn_sched_barrier(0);
                    float vals[4];
                    tile(0, b, b, o, sc_i, vals);
                    *(float4 *)(sAd + (b * 16 + l16) * A_LD + 4 * g4) = make_float4(vals[0], vals[1], vals[2], vals[3]);
                    lds_fence();          // this wave's A rows, written above by other lanes
                    build_T_diag(b, bt, pT);
                }
            } else {
                // wave 1 -> A (1,0) and P (1,0), wave 3 -> P (0,0) and P (1,1); both write the zero
                // P block (0,1); then the gate scan of chunk t+1.  One straight-line block (past the
                // last chunk its results are never read), so the scan can overlap the MFMAs.
                if constexpr (OUT) {
                    const bool w1 = pw == 1;
                    TileOps o[2];
#pragma unroll
                    for (int it = 0; it < 2; ++it) tile_load(w1 ? it : 1, w1 ? 1 : it, w1 ? 0 : it, o[it]);
                    float4 gcol[C / 4];
                    scan_load(gcol);
                    const float sc_a = betac[16 + l16];
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int it = 0; it < 2; ++it) {
                        const int mat = w1 ? it : 1;
                        const int ib = w1 ? 1 : it, jb = w1 ? 0 : it;
                        float vals[4];
                        tile(mat, ib, jb, o[it], mat ? 1.f : sc_a, vals);
                        bf16 *dst = (mat == 0) ? sA10 + l16 * A_LD + 4 * g4 : pP + (16 * ib + l16) * P_LD + 16 * jb + 4 * g4;
                        V4::store(dst, V4::pack(vals));
                    }
                    V4::store(pP + l16 * P_LD + 16 + 4 * g4, V4::zero());   // P block (0,1)
                    scan(pc + 1, t + 1, gcol);
                } else {
                    // no outputs: wave 1 -> A (1,0) only, wave 3 -> the scan only
                    float4 gcol[C / 4];
                    if (pw == 1) {
                        TileOps o;
                        tile_load(0, 1, 0, o);
                        scan_load(gcol);
                        const float sc_a = betac[16 + l16];
                        __builtin_amdgcn_sched_barrier(0);
                        float vals[4];
                        tile(0, 1, 0, o, sc_a, vals);
                        V4::store(sA10 + l16 * A_LD + 4 * g4, V4::pack(vals));
                    } else {
                        scan_load(gcol);
                    }
                    scan(pc + 1, t + 1, gcol);
                }
            }
            sync();
        }
    } else {
        // ============================================ consumer waves
        const int cw = wave;
        // transposed reads: lane k of each 16-lane group addresses row k/4 and channel
        // 4*(k%4) of a 16-channel slice; it receives 4 rows of channel (its slice) + (lane%16)
        const int tr_row = (lane & 15) >> 2, tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        char *ob = has_out ? (char *)p.o + 2 * (bsel * p.o_sb + h * p.o_sh + t0 * p.o_st) : nullptr;
        const uint32_t ost = 2 * (uint32_t)p.o_st, oro = l32 * ost + 2 * (32 * cw + 4 * g2);
        f32x16 S[4];
        const int vcol = 32 * cw + l32;
        // output norm: the pending O tile of the previous chunk, its gate factors w * sigmoid(z),
        // its token range, and the gate rows of the chunk after it (loaded a step ahead)
        float *sNrm = (float *)(smem + S_NRM), *sNw = (float *)(smem + S_NW);
        f32x16 Opend = {}, gw = {};
        uint2 zr[4];
        int pend_tok0 = 0, pend_L = 0;
        const char *zb = nullptr;
        uint32_t zst = 0;
        // gate rows of chunk c: row l32 (rows past the chunk's end re-read its last row), this
        // lane's 16 columns
        auto load_gate = [&](int c) {
            const int L = min(C, len - c * C);
            const char *zc = zb + (int64_t)(c * C) * zst + min(l32, L - 1) * zst + 2 * (32 * cw + 4 * g2);
#pragma unroll
            for (int q = 0; q < 4; ++q) zr[q] = *(const uint2 *)(zc + 16 * q);
        };
        if constexpr (NORM) {
            zb = (const char *)p.z + 2 * (bsel * p.z_sb + h * p.z_sh + t0 * p.z_st);
            zst = 2 * (uint32_t)p.z_st;
            if (tid < D) sNw[tid] = p.nw[tid];
            if (nck > 0) load_gate(c_begin);
        }
        // O row l32 of the pending chunk: o * rsqrt(mean(o^2) + eps) * (w * sigmoid(z))
        auto norm_store = [&]() {
            const float4 nr = *(const float4 *)(sNrm + 4 * l32);
            const float rn = __builtin_amdgcn_rsqf(((nr.x + nr.y) + (nr.z + nr.w)) * (1.f / D) + p.eps);
            if (l32 < pend_L) {
                bf16 *dst = (bf16 *)(ob + (int64_t)pend_tok0 * ost + oro);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float o4[4] = {Opend[4 * q] * rn * gw[4 * q], Opend[4 * q + 1] * rn * gw[4 * q + 1],
                                         Opend[4 * q + 2] * rn * gw[4 * q + 2], Opend[4 * q + 3] * rn * gw[4 * q + 3]};
                    V4::store(dst + 8 * q, V4::pack(o4));
                }
            }
        };
        {
            const float *src = nullptr;
            int64_t rs = D;
            if (role == ROLE_OUT && p.s0) {
                src = p.s0 + n * p.s0_sn + h * p.s0_sh;
                rs = p.s0_sr;
            } else if (role == ROLE_SEG_OUT) {
                src = p.ws_start + ((int64_t)lchain * nseg + seg) * D * D;
            }
            const bf16 *srch = (role == ROLE_OUT && p.s0h) ? p.s0h + n * p.s0_sn + h * p.s0_sh : nullptr;
            if (src) {              // one straight-line block of 64 loads
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[m][4 * q + r] = src[(32 * m + 8 * q + 4 * g2 + r) * rs + vcol];
            } else if (srch) {        // bf16 initial state, widened
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[m][4 * q + r] = (float)srch[(32 * m + 8 * q + 4 * g2 + r) * p.s0_sr + vcol];
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[m][4 * q + r] = 0.f;     // C map, or no initial state
            }
        }
        // MC: the M map of this wave's columns, from the identity
        f32x16 SM[4];
        if constexpr (MC) {
            const int diag = vcol - 4 * g2;     // row 32m + 8q + 4 g2 + r is this lane's column
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) SM[m][4 * q + r] = (32 * m + 8 * q + r == diag) ? 1.f : 0.f;
        }
        // V enters R = V - Kt S on the matrix cores: IdV[j] is the A operand of an identity
        // over tokens 16j..16j+15 (element e of lane (i, g) is 1 where token 16j + 8(e/4) + 4g +
        // e%4 is row i)
        auto make_idv = [&](Frag8<bf16> (&id)[2]) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float t8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = (l32 == 16 * j + 8 * (e >> 2) + 4 * g2 + (e & 3)) ? 1.f : 0.f;
                id[j].set(t8);
            }
        };
        // held across the loop, except in the map role (two states): rebuilt there each step
        Frag8<bf16> IdV[2];
        if constexpr (!MC) make_idv(IdV);
        if (nck > 0) prefetch_qkv(c_begin);
        uint64_t cap_next = 0;          // thread 0: the flag value this chain stores when it is done
        if (capped) cap_next = cap_wait(p, n, h, cap_len, smem + S_CAP);
        sync();
        sync();
        for (int t = 0; nck > 0 && t <= nck; ++t) {
            const bool cact = t >= 1;                       // runs chunk c_begin + t - 1 from buffer (t-1) % 2
            char *CB = smem + ((t + 1) & 1) * B_SIZE;
            const bf16 *cQt = (const bf16 *)(CB + B_QT), *cKt = (const bf16 *)(CB + B_KT);
            const bf16 *cKh = (const bf16 *)(CB + B_KH), *cV = (const bf16 *)(CB + B_V);
            const bf16 *cP = (const bf16 *)(CB + B_P), *cT = (const bf16 *)(CB + B_T);
            const float *cDec = sDec + ((t + 2) % 3) * D;   // ring slot (t - 1) % 3
            const int cc = c_begin + t - 1, ctok0 = cc * C, cL = min(C, len - ctok0);
            Frag8<bf16> SB[8], UB[2];
            // ---------------- interval 1: sub-block 0 operands of chunk t into buffer t % 2;
            //                  R = V - Kt S; wave 0 also finishes T diag(beta) of the chunk
            // One straight-line block, so that the R products can overlap the operand arithmetic:
            // the operands of the step past the last chunk, and R before the first one, are
            // computed on stale data and never read.
            operands(std::false_type{}, smem + (t & 1) * B_SIZE);
            prefetch_qkv(min(c_begin + t + 1, c_last));
            // two maps hold twice the state: keep the operand arithmetic and the R products apart
            if constexpr (MC) __builtin_amdgcn_sched_barrier(0);
            Frag8<bf16> RB[2], RBM[2];
            {
                f32x16 R = {}, RM = {};
                if constexpr (MC) make_idv(IdV);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    Frag8<bf16> fv;
                    const bf16 *p0 = cV + (16 * j + 4 * g2 + tr_row) * KR_LD + 32 * cw + tr_col;
                    fv.load44_tr(p0, p0 + 8 * KR_LD);
                    mma32(R, IdV[j], fv);
                }
                if constexpr (OUT) {        // the bf16 state feeds O too: all 8 fragments, up front
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        float t8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) t8[e] = S[s >> 1][8 * (s & 1) + e];
                        SB[s].set(t8);
                    }
                }
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    Frag8<bf16> fa;
                    const bf16 *row = cKt + l32 * W_LD + 16 * s + 4 * g2;
                    fa.load44(row, row + 8);
                    if constexpr (!OUT) {       // maps: each fragment converted where it is used
                        float t8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) t8[e] = S[s >> 1][8 * (s & 1) + e];
                        SB[s].set(t8);
                    }
                    mma32(R, fa, SB[s]);
                    if constexpr (MC) {           // R_M = -Kt M (V = 0), from the same Kt fragment
                        float t8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) t8[e] = SM[s >> 1][8 * (s & 1) + e];
                        Frag8<bf16> sbm;
                        sbm.set(t8);
                        mma32(RM, fa, sbm);
                    }
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float t8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t8[e] = R[8 * s + e];
                    RB[s].set(t8);
                    if constexpr (MC) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) t8[e] = RM[8 * s + e];
                        RBM[s].set(t8);
                    }
                }
            }
            if (cact && cw == 0) build_T_off(sBeta + ((t + 2) % 3) * C, (bf16 *)(CB + B_T));
            if constexpr (NORM) {
                if (t >= 2) norm_store();     // O of chunk t-2, formed in the last interval 2
            }
            sync();
            // ---------------- interval 2: U = (T diag(beta)) R; O = Qt S + P U, stored
            if (cact) {
                // the decay of the state update first: S is not read again before it (O uses SB)
                {
                    const float4 dd = *(const float4 *)(cDec + 8 * l16 + 4 * g2);
                    decay_tile<0>(S[0], dd);
                    decay_tile<1>(S[1], dd);
                    decay_tile<2>(S[2], dd);
                    decay_tile<3>(S[3], dd);
                    if constexpr (MC) {
                        decay_tile<0>(SM[0], dd);
                        decay_tile<1>(SM[1], dd);
                        decay_tile<2>(SM[2], dd);
                        decay_tile<3>(SM[3], dd);
                    }
                }
                f32x16 U = {}, UM = {};
                Frag8<bf16> UBM[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    Frag8<bf16> fa;
                    const bf16 *row = cT + l32 * P_LD + 16 * s + 4 * g2;
                    fa.load44(row, row + 8);
                    mma32(U, fa, RB[s]);
                    if constexpr (MC) mma32(UM, fa, RBM[s]);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float t8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t8[e] = U[8 * s + e];
                    UB[s].set(t8);
                    if constexpr (MC) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) t8[e] = UM[8 * s + e];
                        UBM[s].set(t8);
                    }
                }
                // O = Qt S + P U (always formed: without outputs it is discarded), then the
                // state update, in one block so the three MFMA chains and the conversions can
                // interleave; the stores come last
                f32x16 O = {};
                if constexpr (OUT) {
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        Frag8<bf16> fb;
                        const bf16 *row = cQt + l32 * W_LD + 16 * s + 4 * g2;
                        fb.load44(row, row + 8);
                        mma32(O, SB[s], fb);
                    }
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        Frag8<bf16> fb;
                        const bf16 *row = cP + l32 * P_LD + 16 * s + 4 * g2;
                        fb.load44(row, row + 8);
                        mma32(O, UB[s], fb);
                    }
                }
                // ---------------- state update: S <- Diag(e^{G_L}) S + Kh^T U
#pragma unroll
                for (int m = 0; m < 4; ++m) {
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        Frag8<bf16> fa;
                        const bf16 *p0 = cKh + (16 * s + 4 * g2 + tr_row) * KR_LD + 32 * m + tr_col;
                        fa.load44_tr(p0, p0 + 8 * KR_LD);
                        mma32(S[m], fa, UB[s]);
                        if constexpr (MC) mma32(SM[m], fa, UBM[s]);
                    }
                }
                if constexpr (NORM) {
                    // this wave's 32 columns of each token's sum of squares; the gate factors of
                    // this chunk, then the gate rows of the next
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) ss += O[e] * O[e];
                    ss += __shfl_xor(ss, 32);
                    if (g2 == 0) sNrm[4 * l32 + cw] = ss;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float zf[4];
                        V4::unpack(zr[q], zf);
                        const float4 w4 = *(const float4 *)(sNw + 32 * cw + 4 * g2 + 8 * q);
                        gw[4 * q] = w4.x * sigmoid_act(zf[0]);
                        gw[4 * q + 1] = w4.y * sigmoid_act(zf[1]);
                        gw[4 * q + 2] = w4.z * sigmoid_act(zf[2]);
                        gw[4 * q + 3] = w4.w * sigmoid_act(zf[3]);
                    }
                    load_gate(min(cc + 1, c_last));
                    Opend = O;
                    pend_tok0 = ctok0;
                    pend_L = cL;
                } else if (OUT && l32 < cL) {
                    bf16 *dst = (bf16 *)(ob + (int64_t)ctok0 * ost + oro);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float o4[4] = {O[4 * q], O[4 * q + 1], O[4 * q + 2], O[4 * q + 3]};
                        V4::store(dst + 8 * q, V4::pack(o4));
                    }
                }
            }
            sync();
        }
        if constexpr (NORM) {
            if (nck > 0) norm_store();        // O of the last chunk
        }
        float *dst = nullptr;
        bf16 *dsth = nullptr;         // bf16 final state (rounded to nearest even)
        int64_t rs = D;
        if (role == ROLE_OUT || (role == ROLE_SEG_OUT && seg == nseg - 1)) {
            if (p.sT) { dst = p.sT + n * p.sT_sn + h * p.sT_sh; rs = p.sT_sr; }
            if (p.sTh) dsth = p.sTh + n * p.sT_sn + h * p.sT_sh;
        } else if (role == ROLE_SEG_MC) {
            dst = p.ws_maps + map_offset(lchain, nseg, seg, 1, D);   // C
        }
        if (dst) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(32 * m + 8 * q + 4 * g2 + r) * rs + vcol] = S[m][4 * q + r];
        }
        if constexpr (MC) {     // M (an empty segment -- a chain shorter than nseg segments -- leaves I)
            store_map_m<true>(p.ws_maps + map_offset(lchain, nseg, seg, 0, D), SM, lane, vcol, D);
        }
        if (dsth) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dsth[(32 * m + 8 * q + 4 * g2 + r) * p.sT_sr + vcol] = (bf16)S[m][4 * q + r];
        }
        // capped concurrency: this chain is done (its last stores are issued); a workgroup
        // queued behind its sequence may start
        if (capped && tid == 0)
            __hip_atomic_store(p.cap_flags + (int64_t)n * p.H + h, cap_next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace pipe

hipError_t launch_chunk_pipe(const ChunkParams &p, int grid, bool stall, hipStream_t st)
{
    if (grid <= 0) return hipSuccess;
    const bool out = p.role == ROLE_OUT || p.role == ROLE_SEG_OUT;
    if (!out && p.role != ROLE_SEG_MC) return hipErrorInvalidValue;   // maps: the merged role only
    const bool norm = out && p.z;
#define KDA_PIPE(S, O, N, M) hipLaunchKernelGGL((pipe::chunk_pipe_kernel<S, O, N, M>), dim3(grid), dim3(pipe::NT), 0, st, p)
    if (stall && norm) KDA_PIPE(true, true, true, false);
    else if (stall && out) KDA_PIPE(true, true, false, false);
    else if (stall) KDA_PIPE(true, false, false, true);
    else if (norm) KDA_PIPE(false, true, true, false);
    else if (out) KDA_PIPE(false, true, false, false);
    else KDA_PIPE(false, false, false, true);
#undef KDA_PIPE
    return hipGetLastError();
}

}  // namespace kda
