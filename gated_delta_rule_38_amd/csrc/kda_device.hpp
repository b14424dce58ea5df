// Device-side building blocks for the gfx950 KDA prefill kernels: element
// types, MFMA wrappers, LDS fragment loaders and the kernel parameter blocks.
//
// Matrix-core conventions used by every kernel (CDNA3/CDNA4 wave64 MFMA):
//   32x32 tiles  (v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x2_f32)
//       accumulator: lane l holds column l%32, register 4q+r holds row
//       8q + 4(l/32) + r  (q = 0..3, r = 0..3).
//   16x16 tiles  (v_mfma_f32_16x16x32_bf16, _16x16x16_bf16, _16x16x4_f32)
//       accumulator: lane l holds column l%16, register r holds row 4(l/16) + r.
//   Operands: lane l holds A[row = l%M][k in kset(l)] and B[k in kset(l)][col = l%N].
// A contraction only needs A and B to agree on kset, so a kernel may pick any
// k-assignment per lane group.  Two are used:
//   * contiguous: kset = 8*(l/32) + 0..7 (32x32) -- one 16-byte LDS read;
//   * acc-compatible: kset = {4g+0..3, 8+4g+0..3}, g = l/32, within each
//     16-wide k step -- exactly the rows an accumulator lane already holds, so
//     an fp32 accumulator converts in registers into the next MFMA's B operand
//     (as itself) or A operand (as its transpose) with no LDS round trip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CHUNK = 64;     // tokens per chunk
constexpr int SUB = 16;       // tokens per gate sub-block (factorisation reference span)
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// lb * sigmoid(x) and sigmoid(x) = 1 / (1 + e^-x): the fused gate and beta activations.  The
// multiply is kept out of FMA contraction so that a sum of these values has the same bits in
// every kernel that forms it (the standalone PREP and the chunk kernels' in-chunk scans).
__device__ __forceinline__ float sigmoid_act(float x)
{
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * LOG2E));
}
__device__ __forceinline__ float gate_act(float x, float lb)
{
#pragma clang fp contract(off)
    return lb * sigmoid_act(x);
}

// ---------------------------------------------------------------- element IO
template <typename ET> struct Elem;
template <> struct Elem<bf16> {
    static __device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
    static __device__ __forceinline__ bf16 from_f(float x) { return (bf16)x; }
};
template <> struct Elem<float> {
    static __device__ __forceinline__ float to_f(float x) { return x; }
    static __device__ __forceinline__ float from_f(float x) { return x; }
};

// Two fp32 values rounded to bf16 (nearest-even) as one packed word, low half first: a
// two-wide conversion, which maps onto one packed-convert instruction.
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 4 consecutive elements, loaded/stored as one 8-byte (bf16) or 16-byte (fp32) access.
template <typename ET> struct Vec4;
template <> struct Vec4<bf16> {
    typedef uint2 raw;
    static __device__ __forceinline__ raw load(const bf16 *p) { return *(const uint2 *)p; }
    static __device__ __forceinline__ void store(bf16 *p, raw v) { *(uint2 *)p = v; }
    static __device__ __forceinline__ void unpack(raw v, float *f) {
        f[0] = __builtin_bit_cast(float, v.x << 16);
        f[1] = __builtin_bit_cast(float, v.x & 0xffff0000u);
        f[2] = __builtin_bit_cast(float, v.y << 16);
        f[3] = __builtin_bit_cast(float, v.y & 0xffff0000u);
    }
    static __device__ __forceinline__ raw pack(const float *f) {
        return make_uint2(pack2(f[0], f[1]), pack2(f[2], f[3]));
    }
    static __device__ __forceinline__ raw zero() { return make_uint2(0u, 0u); }
};
template <> struct Vec4<float> {
    typedef float4 raw;
    static __device__ __forceinline__ raw load(const float *p) { return *(const float4 *)p; }
    static __device__ __forceinline__ void store(float *p, raw v) { *(float4 *)p = v; }
    static __device__ __forceinline__ void unpack(raw v, float *f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
    static __device__ __forceinline__ raw pack(const float *f) { return make_float4(f[0], f[1], f[2], f[3]); }
    static __device__ __forceinline__ raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// ------------------------------------------------------------- fragments
// An 8-value operand fragment: for bf16 one MFMA (k = 16 / 32 wide), for fp32
// eight MFMAs, MFMA m consuming value m of every lane.
template <typename ET> struct Frag8;
template <> struct Frag8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void set(const float *f) {
        v = __builtin_bit_cast(bf16x8, make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])));
    }
    // 8 contiguous elements
    __device__ __forceinline__ void load8(const bf16 *p) { v = *(const bf16x8 *)p; }
    // elements p[0..3] then p2[0..3]
    __device__ __forceinline__ void load44(const bf16 *p, const bf16 *p2) {
        uint2 a = *(const uint2 *)p, b = *(const uint2 *)p2;
        uint4 u = make_uint4(a.x, a.y, b.x, b.y);
        v = __builtin_bit_cast(bf16x8, u);
    }
    // two transposing LDS reads (ds_read_b64_tr_b16): 4 rows of one column each
    __device__ __forceinline__ void load44_tr(const bf16 *p, const bf16 *p2) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p2);
        const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
        v = __builtin_bit_cast(bf16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
    }
};
template <> struct Frag8<float> {
    float v[8];
    __device__ __forceinline__ void set(const float *f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f[e];
    }
    __device__ __forceinline__ void load8(const float *p) {
        float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ __forceinline__ void load44(const float *p, const float *p2) {
        float4 a = *(const float4 *)p, b = *(const float4 *)p2;
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// C(32x32) += A(32 x 16) * B(16 x 32)
__device__ __forceinline__ void mma32(f32x16 &c, const Frag8<bf16> &a, const Frag8<bf16> &b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16 &c, const Frag8<float> &a, const Frag8<float> &b) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[m], b.v[m], c, 0, 0, 0);
}
// C(16x16) += A(16 x 32) * B(32 x 16)
__device__ __forceinline__ void mma16(f32x4 &c, const Frag8<bf16> &a, const Frag8<bf16> &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4 &c, const Frag8<float> &a, const Frag8<float> &b) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[m], b.v[m], c, 0, 0, 0);
}

// 4-value fragments for 16x16 tiles with a 16-wide k (kset = 4*(l/16) + 0..3),
// matching the 16x16 accumulator rows of a lane.
template <typename ET> struct Frag4;
template <> struct Frag4<bf16> {
    s16x4 v;
    __device__ __forceinline__ void set(const float *f) {
        v = __builtin_bit_cast(s16x4, make_uint2(pack2(f[0], f[1]), pack2(f[2], f[3])));
    }
    __device__ __forceinline__ void load4(const bf16 *p) { v = __builtin_bit_cast(s16x4, *(const uint2 *)p); }
};
template <> struct Frag4<float> {
    float v[4];
    __device__ __forceinline__ void set(const float *f) { v[0] = f[0]; v[1] = f[1]; v[2] = f[2]; v[3] = f[3]; }
    __device__ __forceinline__ void load4(const float *p) {
        float4 a = *(const float4 *)p;
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
};
__device__ __forceinline__ void mma16k16(f32x4 &c, const Frag4<bf16> &a, const Frag4<bf16> &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma16k16(f32x4 &c, const Frag4<float> &a, const Frag4<float> &b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[m], b.v[m], c, 0, 0, 0);
}

// ------------------------------------------------------- kernel parameters
// Roles of the chunk kernel.
enum Role : int32_t {
    ROLE_OUT = 0,      // one chain per workgroup: start state -> outputs + final state
    ROLE_SEG_M = 1,    // segment operator M: V = 0, start state = I, no outputs
    ROLE_SEG_C = 2,    // segment offset C: start state = 0, no outputs
    ROLE_SEG_OUT = 3,  // one segment: start state from workspace -> outputs (+ final state)
    ROLE_SEG_MC = 4    // both maps of one segment in one workgroup (pipelined kernel): the
                       // consumer waves carry M and C on their value columns
};
// Segment maps are built for segments 0 .. nseg - 2 only: COMBINE never reads the last one's.
// Map (M or C) `which` (0 = M, 1 = C) of segment seg of chain `chain`, in a workspace of
// [chain][nseg - 1][2][D][D] fp32.
__device__ __forceinline__ int64_t map_offset(int chain, int nseg, int seg, int which, int D)
{
    return (((int64_t)chain * (nseg - 1) + seg) * 2 + which) * D * D;
}

// C is row-major ([key channel][value column], like a state).  M is stored in the order COMBINE
// feeds it to the matrix cores, so that each of a wave's loads is one contiguous 1 KB run of 64
// lanes x 16 bytes instead of 16 rows x 64 bytes (on MI355X a COMBINE step took 30% less time).
// The wave that forms rows 16w .. 16w + 15 of a start state holds, in lane l, row 16w + l % 16:
//   * fp32 maps (fp32 I/O): run j of the wave holds columns k = 16j + 4(l / 16) + 0..3;
//   * split maps (bf16 I/O): M = Mh + Ml, both bf16 (Mh = M rounded to nearest even, Ml = the
//     remainder rounded), so the product M S runs as Mh Sh + Mh Sl + Ml Sh on the bf16 matrix
//     cores with a relative error near 2^-16; for each 32-column block b, run 2b holds Mh and
//     run 2b + 1 Ml of columns k = 32b + 8(l / 16) + 0..7.
// Element (row, k) of a D x D fp32 map, in floats:
__device__ __forceinline__ int map_m_index(int row, int k, int D)
{
    return (((row >> 4) * (D >> 4) + (k >> 4)) * 64 + ((k & 15) >> 2) * 16 + (row & 15)) * 4 + (k & 3);
}
// Element (row, k) of Mh of a split map, in bf16 elements (Ml's is 512 further).
__device__ __forceinline__ int map_m_split_index(int row, int k, int D)
{
    return (((row >> 4) * (D >> 4) + 2 * (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (row & 15)) * 8 + (k & 7);
}

// x = hi + lo to about 16 significant bits, two values at a time: hi = x rounded to bf16 (nearest
// even), lo = the remainder x - hi (exact in fp32) rounded to bf16; each as a packed word.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = pack2(a, b);
    lo = pack2(a - __builtin_bit_cast(float, hi << 16), b - __builtin_bit_cast(float, hi & 0xffff0000u));
}

// Store a map M held in 32x32 MFMA accumulators -- tile m, element 4q + r at row
// 32m + 8q + 4(lane / 32) + r, column `vcol` -- in COMBINE's order (SPLIT: as Mh and Ml).
// Lanes 2a and 2a + 1 (columns c, c + 1) first swap two of their four rows (a quad permute
// [1,0,3,2]), so each lane holds two consecutive columns of two rows and stores them as pairs.
template <bool SPLIT, int NM>
__device__ __forceinline__ void store_map_m(float *dm, const f32x16 (&S)[NM], int lane, int vcol, int D)
{
    const bool odd = lane & 1;
    const int k0 = vcol & ~1, rb = 4 * (lane >> 5) + (odd ? 1 : 0);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // an even lane keeps rows 0 and 2 of its column and takes those of its odd
            // neighbour; an odd lane rows 1 and 3
            const float a0 = S[m][4 * q], a1 = S[m][4 * q + 1], a2 = S[m][4 * q + 2], a3 = S[m][4 * q + 3];
            const float s0 = odd ? a0 : a1, s1 = odd ? a2 : a3;
            const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0), 0xB1, 0xf, 0xf, false));
            const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1), 0xB1, 0xf, 0xf, false));
            // even lane: row 0 = (a0, r0), row 2 = (a2, r1); odd lane: row 1 = (r0, a1), row 3 = (r1, a3)
            const float2 lo = odd ? make_float2(r0, a1) : make_float2(a0, r0);
            const float2 hi = odd ? make_float2(r1, a3) : make_float2(a2, r1);
            const int row = 32 * m + 8 * q + rb;
            if constexpr (SPLIT) {
                // lanes l and l ^ 2 hold the same rows for columns k0 .. k0 + 1 and k0 ^ 2 ..:
                // a lane with bit 1 clear keeps row `row` and takes its partner's, the other
                // keeps row + 2, so each stores 4 consecutive columns of one row (8 bytes of
                // Mh, 8 of Ml)
                uint32_t ha, la, hb, lb;
                split2(lo.x, lo.y, ha, la);         // row
                split2(hi.x, hi.y, hb, lb);         // row + 2
                const bool up = lane & 2;
                const uint32_t sh = up ? ha : hb, sl = up ? la : lb;
                const uint32_t rh = __builtin_amdgcn_mov_dpp(sh, 0x4E, 0xf, 0xf, false);
                const uint32_t rl = __builtin_amdgcn_mov_dpp(sl, 0x4E, 0xf, 0xf, false);
                // bit 1 clear: row, columns (k0, k0 + 1) then the partner's (k0 + 2, k0 + 3);
                // bit 1 set: row + 2, the partner's (k0 - 2, k0 - 1) then its own
                const uint2 h2 = up ? make_uint2(rh, hb) : make_uint2(ha, rh);
                const uint2 l2 = up ? make_uint2(rl, lb) : make_uint2(la, rl);
                const int i = map_m_split_index(up ? row + 2 : row, k0 & ~3, D);
                *(uint2 *)((bf16 *)dm + i) = h2;
                *(uint2 *)((bf16 *)dm + i + 512) = l2;
            } else {
                *(float2 *)(dm + map_m_index(row, k0, D)) = lo;
                *(float2 *)(dm + map_m_index(row + 2, k0, D)) = hi;
            }
        }
}

struct ChunkParams {
    const void *q, *k, *v;     // ET
    const float *g;            // raw log decays, or in-chunk cumsums (g_is_gamma)
    const float *beta;
    const float *s0;           // initial state or NULL (fp32)
    const bf16 *s0h;           // initial state or NULL (bf16; s0 is then NULL)
    void *o;                   // ET
    float *sT;                 // final state or NULL (fp32)
    bf16 *sTh;                 // final state or NULL (bf16; sT is then NULL)
    const int32_t *cu;         // NULL: dense layout
    float *ws_maps;            // [chain][nseg - 1][2][D x D] segment operators (M, C) of segments 0 .. nseg - 2
                               // (M in COMBINE's order, split on bf16 I/O; C row-major)
    const float *ws_start;     // [chain][seg][D][D] segment start states
    // strides in elements: batch, token, head
    int64_t q_sb, q_st, q_sh, k_sb, k_st, k_sh, v_sb, v_st, v_sh, g_sb, g_st, g_sh;
    int64_t b_sb, b_st, b_sh, o_sb, o_st, o_sh;
    int64_t s0_sn, s0_sh, s0_sr, sT_sn, sT_sh, sT_sr;   // state: sequence, head, row
    int32_t N, H, T;           // T: tokens per sequence in the dense layout
    int32_t nseg;
    int32_t role;
    int32_t g_is_gamma;
    int32_t stall_wave;        // wave index to stall, or -1
    int32_t stall_iters;       // s_sleep(127) repetitions per stall
    int32_t gate_act;          // g holds logits: log decay = gate_lb * sigmoid(g)
    float gate_lb;
    int32_t beta_act;          // beta holds logits: beta = sigmoid(beta)
    const void *z;             // output gate (out's layout and dtype), or NULL: no output norm
    int64_t z_sb, z_st, z_sh;
    const float *nw;           // norm weight [D]
    float eps;
    int32_t lpt;               // packed layout, one segment: workgroup rank r runs the r-th
                               // longest sequence (ties: lower index first); N <= LPT_MAX_SEQ
    // Segmented plans cut chains seg_chain0 .. N*H - 1 into nseg segments (workspace slots are
    // indexed from seg_chain0); chains below seg_chain0 run whole.  In a ROLE_SEG_OUT launch,
    // workgroups 0 .. n_segwg - 1 run the segments and the ones after them run chains
    // 0 .. seg_chain0 - 1 whole (ROLE_OUT).
    int32_t seg_chain0;
    int32_t n_segwg;
    // Capped concurrency (packed layout, one segment, every chain resident at once): the
    // sequences, longest first, are packed into cap_slots groups of H workgroups, each
    // sequence into the least-loaded group; a workgroup whose sequence follows another one in
    // its group first waits until the chain of the same head of that sequence has stored the
    // value its own flag will take (cap_epoch, with a count that tells replays of one captured
    // call apart), or until cap_wait_us (0: a bound from the predecessor's length) has passed.
    // The wait orders no data: it only keeps fewer chains running at once.  0 = off.
    int32_t cap_slots;
    uint32_t cap_epoch;
    int32_t cap_wait_us;
    uint64_t *cap_flags;       // [N * H] in the workspace, chain n * H + h: the call's value
                               // (low word) and a count of replays of that call (high word)
};

// Longest-first chain order: at most this many sequences (one launch ranks them all in LDS).
constexpr int LPT_MAX_SEQ = 512;
// Capped concurrency: at most this many groups, and N * groups <= CAP_MAX_WORK (one thread
// packs the sequences at the start of every workgroup).
constexpr int CAP_MAX_SLOTS = 16;
constexpr int CAP_MAX_WORK = 4096;
constexpr int CAP_MAX_N = 128;     // sequences

struct PrepParams {
    const float *g;
    float *gamma;
    const int32_t *cu;
    int64_t g_sb, g_st, g_sh, y_sb, y_st, y_sh;
    int32_t N, H, T, D;
    int32_t chunk;             // tokens per chunk (32 or 64)
    int32_t chunks_per_seq;    // dense layout: ceil(T / chunk); packed: unused
    int32_t gate_act;          // g holds logits: log decay = gate_lb * sigmoid(g)
    float gate_lb;
};

constexpr int DECODE_MAX_TOKENS = 8;

struct DecodeParams {
    const void *q, *k, *v;     // [R][T][H][D], bf16 or fp32
    const float *g, *beta;     // [R][T][H][D], [R][T][H]
    void *pool;                // [P][H][D][D], fp32 or bf16
    const int32_t *idx;        // [R] pool slot per request (outside [0, P): skipped)
    const int32_t *ntok;       // [R] tokens per request (clamped to [0, T]), or NULL for T
    void *o;                   // [R][T][H][D] or NULL
    int64_t q_sr, q_st, q_sh, k_sr, k_st, k_sh, v_sr, v_st, v_sh, g_sr, g_st, g_sh;
    int64_t b_sr, b_st, b_sh, o_sr, o_st, o_sh;
    int64_t p_sn, p_sh, p_sr;  // pool: slot, head, row
    int32_t R, T, H, P;
    int32_t update;
    int32_t gate_act;
    float gate_lb;
    int32_t beta_act;
    int32_t stall_wave;        // test hook: wave index to stall after every barrier, or -1
    int32_t stall_iters;       // s_sleep(127) repetitions per stall
    const void *z;             // output gate [R][T][H][D] (out's dtype), or NULL: no output norm
    int64_t z_sr, z_st, z_sh;
    const float *nw;           // norm weight [D]
    float eps;
};

struct CombineParams {
    const float *maps;         // [chain - seg_chain0][nseg - 1][2][D x D] (M in COMBINE's order)
    float *start;              // [chain - seg_chain0][seg][D][D]
    const float *s0;           // initial state (fp32), or NULL
    const bf16 *s0h;           // initial state (bf16), or NULL
    int64_t s0_sn, s0_sh, s0_sr;
    int32_t N, H, nseg;
    int32_t seg_chain0;        // workgroup x runs chain seg_chain0 + x
};

// A token-major fp32 view for the debug-mode range check of g: element (row r, head h,
// channel c) at g[b sb + t st + h sh + c] with r = b rows_per_b + t.
struct CheckG {
    const float *g;
    int64_t rows, rows_per_b, sb, st, sh;
    int64_t H, D;
    float lo, hi;
};

// Sequence n's token range in the dense ([B,T,...]) or packed (cu_seqlens) layout.
__device__ __forceinline__ void seq_range(const int32_t *cu, int n, int T, int64_t &t0, int &len, int64_t &bofs_sel) {
    if (cu) {
        t0 = cu[n];
        len = cu[n + 1] - cu[n];
        bofs_sel = 0;
    } else {
        t0 = 0;
        len = T;
        bofs_sel = n;
    }
}

}  // namespace kda
