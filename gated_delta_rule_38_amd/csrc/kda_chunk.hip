// CHUNK kernel: the KDA chunked prefill of one (sequence, head) chain -- or one
// segment of it -- per workgroup, on gfx950 matrix cores.
//
// Per 64-token chunk with start state S0 (d_k x d_v fp32, row = key channel),
// in-chunk inclusive log-decay cumsum Gamma (vector over key channels), the WY/UT
// form of the gated delta rule (derived from the recurrence; the pages name the
// WY-form chunk in TensorRT-LLM PR #19960 and use 64-token chunks (v64) in
// the cudnn-frontend Hopper kernel of PR #1056):
//     A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}  (j < i),   T = (I + A)^-1
//     P_ij =        sum_c q_ic k_jc e^{G_ic - G_jc}  (j <= i)
//     W = T diag(beta) (K o e^G),   Ut = T diag(beta) V
//     U = Ut - W S0,   O = (Q o e^G) S0 + P U,   S_L = Diag(e^{G_L}) S0 + (K o e^{G_L - G})^T U
//
// Gate safety.  At the production gate floor of -5 (cudnn-frontend PR #1056:
// a kernel correct at gate -1 returned all-NaN at -5) Gamma spans up to 320
// nats per chunk, so a chunk-wide factor e^{-Gamma} overflows fp32.  A and P are
// built from 16-token sub-blocks b instead: with E_b = Gamma at the token before
// block b (0 for b = 0) and Gend_b = Gamma at the block's last token,
//   diagonal blocks:     (k_i e^{G_i - E_b}) . (k_j e^{E_b - G_j})    factors in [e^-80, e^80]
//   off-diagonal (b'<b): (k_i e^{G_i - E_b}) . (k_j e^{Gend_b' - G_j}) e^{E_b - Gend_b'}
// where every off-diagonal factor is <= 1, so an underflow to zero only drops a
// term that is itself below fp32 range.  Every other operand is a product of
// factors <= 1 in the same way.  One exp and one reciprocal per element.
//
// Work split.  The workgroup has D/32 waves; wave w owns value columns
// [32w, 32w + 32) of the state for the whole chain and keeps that slab in MFMA
// accumulators across chunks (the register-resident state of the cudnn-frontend
// kernel's description, here as the accumulator of v_mfma_f32_32x32x16_bf16).
// The accumulator layout feeds the next contraction directly (see
// kda_device.hpp), so the state never passes through LDS.  The chunk-local
// operators (A, P, T, W) are built cooperatively in LDS; every LDS buffer that
// is rewritten within a chunk or by the next chunk has a workgroup barrier
// between its last reader and its next writer (the inter-chunk shared-memory
// race fixed in TensorRT-LLM PR #19826 is exactly a missing one).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D, typename ET> struct ChunkCfg {
    static constexpr int NW = D / 32;          // waves = value slabs = key row tiles
    static constexpr int NT = 64 * NW;
    static constexpr int HALF = D / 2;         // channels per elementwise half pass
    static constexpr int CG = HALF / 4;        // 4-channel groups per half
    static constexpr int ES = (int)sizeof(ET);
    static constexpr int PH = 16 / ES;         // pad of the sub-block operand tiles
    // leading dimensions (elements)
    static constexpr int G_LD = D + 4;         // Gamma, fp32 [64][D]
    static constexpr int H_LD = HALF + PH;     // X, Y, Z, Kb  [rows][HALF]
    static constexpr int QT_LD = D + 4;        // Qt, W [64][D]
    static constexpr int TT_LD = CHUNK + 4;    // Kh^T [D][64], read 8 bytes per lane
    static constexpr int TW_LD = CHUNK + PH;   // (beta Kt)^T, (beta V)^T [D][64], read 16 bytes per lane
    static constexpr int SQ_LD = CHUNK + 4;    // A, P [64][64]
    static constexpr int TQ_LD = CHUNK + PH;   // T [64][64], read 16 bytes per lane
    static constexpr int AD_LD = 20;           // fp32 diagonal blocks of A (bf16 mode): rows 16-byte aligned
    static constexpr int AD_BS = 16 * AD_LD + 4;
    static constexpr int TD_LD = 16 + 4;       // transposed diagonal blocks of T
    static constexpr int KB_ROWS = 96;         // K-bar blocks 0..2 + three scaled copies
    // region G: Gamma, later A (+ fp32 diagonal), T, T-diag^T
    static constexpr int SZ_GAM = CHUNK * G_LD * 4;
    static constexpr int SZ_A = CHUNK * SQ_LD * ES;
    static constexpr int SZ_AD = (ES == 2) ? 4 * AD_BS * 4 : 0;
    static constexpr int SZ_T = CHUNK * TQ_LD * ES;
    static constexpr int SZ_TD = 4 * 16 * TD_LD * ES;
    static constexpr int SZ_G2 = SZ_A + SZ_AD + SZ_T + SZ_TD;
    static constexpr int SZ_G = ((SZ_GAM > SZ_G2 ? SZ_GAM : SZ_G2) + 15) / 16 * 16;
    // region H: X, Y, Z, Kb half tiles, later W and P
    static constexpr int SZ_H1 = (3 * CHUNK + KB_ROWS) * H_LD * ES;
    static constexpr int SZ_W = CHUNK * QT_LD * ES;
    static constexpr int SZ_P = CHUNK * SQ_LD * ES;
    static constexpr int SZ_H = ((SZ_H1 > SZ_W + SZ_P ? SZ_H1 : SZ_W + SZ_P) + 15) / 16 * 16;
    // region E: Qt, Kh^T, (beta Kt)^T, (beta V)^T
    static constexpr int SZ_QT = CHUNK * QT_LD * ES;
    static constexpr int SZ_TT = D * TT_LD * ES;
    static constexpr int SZ_TW = D * TW_LD * ES;
    static constexpr int SZ_E = (SZ_QT + SZ_TT + 2 * SZ_TW + 15) / 16 * 16;
    static constexpr int NSC = 16;             // per-channel scale rows
    static constexpr int SZ_SC = NSC * D * 4;
    static constexpr int OFF_G = 0, OFF_H = SZ_G, OFF_E = OFF_H + SZ_H, OFF_SC = OFF_E + SZ_E;
    static constexpr int OFF_BETA = OFF_SC + SZ_SC;
    static constexpr int SMEM = OFF_BETA + CHUNK * 4;
    static_assert(SMEM <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
};

// scale rows (fp32 [NSC][D]):
//  0..3  e^{E_b}            4..7  tau_b = e^{Gend_b - E_b}     8..11 e^{G_L - Gend_b}
//  12    e^{Gend_1 - Gend_0} 13   e^{Gend_2 - Gend_0}          14    e^{Gend_2 - Gend_1}
//  15    e^{G_L}  (the chunk's state decay)
enum { SC_EE = 0, SC_TAU = 4, SC_SL = 8, SC_S20 = 12, SC_S30 = 13, SC_S31 = 14, SC_DEC = 15 };

template <int D, typename ET, bool STALL>
__global__ __launch_bounds__(64 * (D / 32), 1) void chunk_kernel(const ChunkParams p)
{
    using Cf = ChunkCfg<D, ET>;
    using V4 = Vec4<ET>;
    using EL = Elem<ET>;
    constexpr int NW = Cf::NW, HALF = Cf::HALF, CG = Cf::CG;
    constexpr int G_LD = Cf::G_LD, H_LD = Cf::H_LD, QT_LD = Cf::QT_LD, TT_LD = Cf::TT_LD,
                  SQ_LD = Cf::SQ_LD, TW_LD = Cf::TW_LD, TQ_LD = Cf::TQ_LD;
    constexpr int NMT = D / 32;            // 32-row tiles of the state
    constexpr int NITEM = 20 / NW;         // A/P sub-tiles per wave

    __shared__ __attribute__((aligned(16))) char smem[Cf::SMEM];
    float *sG = (float *)(smem + Cf::OFF_G);
    ET *sA = (ET *)(smem + Cf::OFF_G);
    float *sAd = (float *)(smem + Cf::OFF_G + Cf::SZ_A);
    ET *sT = (ET *)(smem + Cf::OFF_G + Cf::SZ_A + Cf::SZ_AD);
    ET *sTdT = (ET *)(smem + Cf::OFF_G + Cf::SZ_A + Cf::SZ_AD + Cf::SZ_T);
    ET *sX = (ET *)(smem + Cf::OFF_H);
    ET *sY = sX + CHUNK * H_LD;
    ET *sZ = sY + CHUNK * H_LD;
    ET *sKb = sZ + CHUNK * H_LD;
    ET *sW = (ET *)(smem + Cf::OFF_H);
    ET *sP = sW + CHUNK * QT_LD;
    ET *sQt = (ET *)(smem + Cf::OFF_E);
    ET *sKhT = sQt + CHUNK * QT_LD;
    ET *sKtT = sKhT + D * TT_LD;
    ET *sVT = sKtT + D * Cf::TW_LD;
    float *sSc = (float *)(smem + Cf::OFF_SC);
    float *sBeta = (float *)(smem + Cf::OFF_BETA);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, g2 = lane >> 5;      // 32x32 tiles
    const int l16 = lane & 15, g4 = lane >> 4;      // 16x16 tiles
    const int cg = tid % CG, tg = tid / CG;         // elementwise: 4 channels x 4 tokens
    const int blk = tg >> 2;                        // 16-token sub-block of this thread

    auto sync = [&]() {
        __syncthreads();
        if constexpr (STALL) {
            if (wave == p.stall_wave)
                for (int s = 0; s < p.stall_iters; ++s) __builtin_amdgcn_s_sleep(127);
        }
    };

    // ------------------------------------------------ which chain / segment
    int wg = blockIdx.x;
    int role = p.role;
    int per_chain = p.nseg;             // workgroups' segments per chain in this launch
    if (role == ROLE_SEG_M) {           // two workgroups (M, C) per segment 0 .. nseg - 2
        role = (wg & 1) ? ROLE_SEG_C : ROLE_SEG_M;
        wg >>= 1;
        per_chain = p.nseg - 1;
    }
    const int seg = wg % per_chain;
    const int chain = wg / per_chain;
    const int n = chain / p.H, h = chain % p.H;
    int64_t t0, bsel;
    int len;
    seq_range(p.cu, n, p.T, t0, len, bsel);
    const int nchunks = (len + CHUNK - 1) / CHUNK;
    const int cps = (nchunks + p.nseg - 1) / p.nseg;
    const int c_begin = min(seg * cps, nchunks);
    const int c_end = min(c_begin + cps, nchunks);
    const bool has_out = (role == ROLE_OUT || role == ROLE_SEG_OUT);
    const bool has_v = (role != ROLE_SEG_M);

    const ET *qb = (const ET *)p.q + bsel * p.q_sb + h * p.q_sh + t0 * p.q_st;
    const ET *kb = (const ET *)p.k + bsel * p.k_sb + h * p.k_sh + t0 * p.k_st;
    const ET *vb = (const ET *)p.v + bsel * p.v_sb + h * p.v_sh + t0 * p.v_st;
    const float *gb = p.g + bsel * p.g_sb + h * p.g_sh + t0 * p.g_st;
    const float *bb = p.beta + bsel * p.b_sb + h * p.b_sh + t0 * p.b_st;
    ET *ob = has_out ? (ET *)p.o + bsel * p.o_sb + h * p.o_sh + t0 * p.o_st : nullptr;

    // ------------------------------------------------ start state
    f32x16 S[NMT];
    const int vcol = 32 * wave + l32;               // value column owned by this lane
    {
        const float *src = nullptr;
        int64_t rs = D;
        if (role == ROLE_OUT && p.s0) {
            src = p.s0 + n * p.s0_sn + h * p.s0_sh;
            rs = p.s0_sr;
        } else if (role == ROLE_SEG_OUT) {
            src = p.ws_start + ((int64_t)chain * p.nseg + seg) * D * D;
        }
        const bf16 *srch = (role == ROLE_OUT && p.s0h) ? p.s0h + n * p.s0_sn + h * p.s0_sh : nullptr;
        const float one = (role == ROLE_SEG_M) ? 1.f : 0.f;
        if (src) {                  // one straight-line block of loads
#pragma unroll
            for (int m = 0; m < NMT; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[m][4 * q + r] = src[(32 * m + 8 * q + 4 * g2 + r) * rs + vcol];
        } else if (srch) {        // bf16 initial state, widened
#pragma unroll
            for (int m = 0; m < NMT; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[m][4 * q + r] = (float)srch[(32 * m + 8 * q + 4 * g2 + r) * p.s0_sr + vcol];
        } else {
#pragma unroll
            for (int m = 0; m < NMT; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[m][4 * q + r] = (32 * m + 8 * q + 4 * g2 + r == vcol) ? one : 0.f;
        }
    }

    // ------------------------------------------------ register prefetch
    typename V4::raw rq[2][4], rk[2][4], rv[2][4];
    float4 rg[2][4];
    float rbeta = 0.f;
    // Loads are unconditional from clamped, always in-bounds addresses (tail rows
    // re-read the chunk's last token) so no load sits in a branch whose merge would
    // force a wait; tail rows are zeroed where the data is used.
    auto load_g = [&](int c) {
        const int tok0 = c * CHUNK, Lm1 = min(CHUNK, len - tok0) - 1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = hh * HALF + 4 * cg;
                rg[hh][r] = *(const float4 *)(gb + (int64_t)(tok0 + min(4 * tg + r, Lm1)) * p.g_st + ch);
            }
        if (tid < CHUNK) rbeta = bb[(int64_t)(tok0 + min(tid, Lm1)) * p.b_st];
    };
    auto load_qkv = [&](int c, int hh) {
        const int tok0 = c * CHUNK, Lm1 = min(CHUNK, len - tok0) - 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ch = hh * HALF + 4 * cg;
            const int64_t tk = tok0 + min(4 * tg + r, Lm1);
            rq[hh][r] = V4::load(qb + tk * p.q_st + ch);
            rk[hh][r] = V4::load(kb + tk * p.k_st + ch);
            rv[hh][r] = V4::load(vb + tk * p.v_st + ch);
        }
    };
    if (c_begin < c_end) {
        load_g(c_begin);
        load_qkv(c_begin, 0);
        load_qkv(c_begin, 1);
    }

    // A/P sub-tile list: pair pr = 0..9 enumerates the lower 16-block triangle
    // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3).
    auto ib_of = [](int pr) { return pr >= 6 ? 3 : pr >= 3 ? 2 : pr >= 1 ? 1 : 0; };

    for (int c = c_begin; c < c_end; ++c) {
        const int tok0 = c * CHUNK;
        const int L = min(CHUNK, len - tok0);

        // ---------------- stage 1: raw g (or Gamma) and beta into LDS; logits in: the decays
        //                  lb * sigmoid(x) (tail rows stay zero, so the scan skips them)
        if (p.gate_act && !p.g_is_gamma) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float4 &x = rg[hh][r];
                    x = make_float4(gate_act(x.x, p.gate_lb), gate_act(x.y, p.gate_lb), gate_act(x.z, p.gate_lb),
                                    gate_act(x.w, p.gate_lb));
                }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *(float4 *)(sG + (4 * tg + r) * G_LD + hh * HALF + 4 * cg) =
                    (4 * tg + r < L) ? rg[hh][r] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < CHUNK) sBeta[tid] = (tid < L) ? (p.beta_act ? sigmoid_act(rbeta) : rbeta) : 0.f;
        if (c + 1 < c_end) load_g(c + 1);
        sync();

        // ---------------- stage 2: in-chunk gate scan (PREP's device step) + scales
        if (tid < D) {
            // one thread per key channel: the column into registers, the 64 adds in
            // token order (fp32, sequential), the column back
            float col[CHUNK], gend[4];
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) col[i] = sG[i * G_LD + tid];
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) {
                if (p.g_is_gamma) acc = (i < L) ? col[i] : acc;   // tail rows hold Gamma_{L-1}
                else acc = acc + col[i];
                col[i] = acc;
                if ((i & 15) == 15) gend[i >> 4] = acc;
            }
#pragma unroll
            for (int i = 0; i < CHUNK; ++i) sG[i * G_LD + tid] = col[i];
            const float GL = gend[3];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float Eb = b ? gend[b - 1] : 0.f;
                sSc[(SC_EE + b) * D + tid] = fast_exp(Eb);
                sSc[(SC_TAU + b) * D + tid] = fast_exp(gend[b] - Eb);
                sSc[(SC_SL + b) * D + tid] = fast_exp(GL - gend[b]);
            }
            sSc[SC_S20 * D + tid] = fast_exp(gend[1] - gend[0]);
            sSc[SC_S30 * D + tid] = fast_exp(gend[2] - gend[0]);
            sSc[SC_S31 * D + tid] = fast_exp(gend[2] - gend[1]);
            sSc[SC_DEC * D + tid] = fast_exp(GL);
        }
        sync();

        // ---------------- stages 3/4: elementwise operands + A/P sub-tiles, per channel half
        f32x4 apacc[NITEM];
#pragma unroll
        for (int it = 0; it < NITEM; ++it) apacc[it] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            {   // elementwise
                const int ch = hh * HALF + 4 * cg;
                const float4 Eb = blk ? *(const float4 *)(sG + (16 * blk - 1) * G_LD + ch)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                const float4 eE = *(const float4 *)(sSc + (SC_EE + blk) * D + ch);
                const float4 tau = *(const float4 *)(sSc + (SC_TAU + blk) * D + ch);
                const float4 sL = *(const float4 *)(sSc + (SC_SL + blk) * D + ch);
                const float4 s20 = *(const float4 *)(sSc + SC_S20 * D + ch);
                const float4 s30 = *(const float4 *)(sSc + SC_S30 * D + ch);
                const float4 s31 = *(const float4 *)(sSc + SC_S31 * D + ch);
                const float Ebv[4] = {Eb.x, Eb.y, Eb.z, Eb.w}, eEv[4] = {eE.x, eE.y, eE.z, eE.w};
                const float tauv[4] = {tau.x, tau.y, tau.z, tau.w}, sLv[4] = {sL.x, sL.y, sL.z, sL.w};
                const float s20v[4] = {s20.x, s20.y, s20.z, s20.w}, s30v[4] = {s30.x, s30.y, s30.z, s30.w};
                const float s31v[4] = {s31.x, s31.y, s31.z, s31.w};
                float kh[4][4], bkt[4][4], bv[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * tg + r;
                    const float4 Gv = *(const float4 *)(sG + i * G_LD + ch);
                    const float G4[4] = {Gv.x, Gv.y, Gv.z, Gv.w};
                    const float bi = sBeta[i];
                    float qf[4], kf[4], vf[4];
                    V4::unpack(rq[hh][r], qf);
                    V4::unpack(rk[hh][r], kf);
                    V4::unpack(rv[hh][r], vf);
                    if (i >= L || !has_v) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) vf[e] = 0.f;
                    }
                    if (i >= L) {                       // tail rows: no token
#pragma unroll
                        for (int e = 0; e < 4; ++e) { qf[e] = 0.f; kf[e] = 0.f; }
                    }
                    float X[4], Y[4], Z[4], Kb[4], Qt[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float f = fast_exp(G4[e] - Ebv[e]);   // e^{G_i - E_b} in [e^-80, 1]
                        const float rr = fast_rcp(f);                // e^{E_b - G_i} in [1, e^80]
                        X[e] = kf[e] * f;
                        Y[e] = qf[e] * f;
                        Z[e] = kf[e] * rr;
                        Kb[e] = Z[e] * tauv[e];                      // k e^{Gend_b - G_i}
                        Qt[e] = Y[e] * eEv[e];                       // q e^{G_i}
                        bkt[r][e] = bi * (X[e] * eEv[e]);            // beta k e^{G_i}
                        kh[r][e] = Kb[e] * sLv[e];                   // k e^{G_L - G_i}
                        bv[r][e] = bi * vf[e];
                    }
                    const int hc = 4 * cg;
                    V4::store(sX + i * H_LD + hc, V4::pack(X));
                    V4::store(sZ + i * H_LD + hc, V4::pack(Z));
                    if (has_out) {
                        V4::store(sY + i * H_LD + hc, V4::pack(Y));
                        V4::store(sQt + i * QT_LD + ch, V4::pack(Qt));
                    }
                    if (blk <= 2) V4::store(sKb + i * H_LD + hc, V4::pack(Kb));
                    if (blk == 0) {
                        float t1[4], t2[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) { t1[e] = Kb[e] * s20v[e]; t2[e] = Kb[e] * s30v[e]; }
                        V4::store(sKb + (48 + i) * H_LD + hc, V4::pack(t1));
                        V4::store(sKb + (64 + i) * H_LD + hc, V4::pack(t2));
                    } else if (blk == 1) {
                        float t1[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) t1[e] = Kb[e] * s31v[e];
                        V4::store(sKb + (80 + i - 16) * H_LD + hc, V4::pack(t1));
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a0[4] = {kh[0][e], kh[1][e], kh[2][e], kh[3][e]};
                    const float a1[4] = {bkt[0][e], bkt[1][e], bkt[2][e], bkt[3][e]};
                    V4::store(sKhT + (ch + e) * TT_LD + 4 * tg, V4::pack(a0));
                    V4::store(sKtT + (ch + e) * TW_LD + 4 * tg, V4::pack(a1));
                    if (has_v) {
                        const float a2[4] = {bv[0][e], bv[1][e], bv[2][e], bv[3][e]};
                        V4::store(sVT + (ch + e) * TW_LD + 4 * tg, V4::pack(a2));
                    }
                }
            }
            if (c + 1 < c_end) load_qkv(c + 1, hh);
            sync();
            // A^T / P^T sub-tiles: rows j (block jb), columns i (block ib), k = this half's channels
#pragma unroll
            for (int it = 0; it < NITEM; ++it) {
                const int item = wave + NW * it;
                const int mat = item / 10, pr = item % 10;   // mat 0: A, 1: P
                if (mat == 1 && !has_out) continue;
                const int ib = ib_of(pr), jb = pr - ib * (ib + 1) / 2;
                const ET *arow;
                if (ib == jb) arow = sZ + (16 * jb + l16) * H_LD;
                else if (ib == jb + 1) arow = sKb + (16 * jb + l16) * H_LD;
                else if (jb == 0) arow = sKb + ((ib == 2 ? 48 : 64) + l16) * H_LD;
                else arow = sKb + (80 + l16) * H_LD;
                const ET *brow = (mat ? sY : sX) + (16 * ib + l16) * H_LD;
#pragma unroll
                for (int s = 0; s < HALF / 32; ++s) {
                    Frag8<ET> fa, fb;
                    fa.load8(arow + 32 * s + 8 * g4);
                    fb.load8(brow + 32 * s + 8 * g4);
                    mma16(apacc[it], fa, fb);
                }
            }
            sync();
        }

        // ---------------- stage 5: masked A (beta-scaled), P into LDS; zero upper blocks
#pragma unroll
        for (int it = 0; it < NITEM; ++it) {
            const int item = wave + NW * it;
            const int mat = item / 10, pr = item % 10;
            if (mat == 1 && !has_out) continue;
            const int ib = ib_of(pr), jb = pr - ib * (ib + 1) / 2;
            const int i = 16 * ib + l16, j0 = 16 * jb + 4 * g4;
            float vals[4];
            if (mat == 0) {
                const float bi = sBeta[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) vals[r] = (j0 + r < i) ? apacc[it][r] * bi : 0.f;
                if (ib == jb) {
                    if constexpr (Cf::ES == 2) {
                        *(float4 *)(sAd + ib * Cf::AD_BS + l16 * Cf::AD_LD + 4 * g4) = make_float4(vals[0], vals[1], vals[2], vals[3]);
                    } else {
                        V4::store(sA + i * SQ_LD + j0, V4::pack(vals));
                    }
                } else {
                    V4::store(sA + i * SQ_LD + j0, V4::pack(vals));
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) vals[r] = (j0 + r <= i) ? apacc[it][r] : 0.f;
                V4::store(sP + i * SQ_LD + j0, V4::pack(vals));
            }
        }
        if (tid < 128) {
            // P and T are zero in the 16-blocks (0,1) and (2,3) that the 32-wide MFMA steps read
            const int bsel2 = tid >> 6, rem = tid & 63;
            const int ib = 2 * bsel2, i = 16 * ib + (rem >> 2), j = 16 * (ib + 1) + 4 * (rem & 3);
            if (has_out) V4::store(sP + i * SQ_LD + j, V4::zero());
            V4::store(sT + i * TQ_LD + j, V4::zero());
        }
        sync();

        // ---------------- stage 6: T = (I + A)^-1.  Diagonal 16x16 blocks by forward substitution
        {
            // block b of this lane: D = 128 gives one block per wave, D = 64 two per wave
            constexpr int PER = 4 / NW;
            const int b = wave + NW * (g4 % PER), col = l16;
            const float *Ab;
            int ld;
            if constexpr (Cf::ES == 2) { Ab = sAd + b * Cf::AD_BS; ld = Cf::AD_LD; }
            else { Ab = (const float *)sA + (16 * b) * SQ_LD + 16 * b; ld = SQ_LD; }
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float arow[16];
#pragma unroll
                for (int j4 = 0; j4 < (i + 3) / 4; ++j4) {
                    const float4 a4 = *(const float4 *)(Ab + i * ld + 4 * j4);
                    arow[4 * j4] = a4.x; arow[4 * j4 + 1] = a4.y; arow[4 * j4 + 2] = a4.z; arow[4 * j4 + 3] = a4.w;
                }
                float s = (i == col) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s = fmaf(-arow[j], x[j], s);
                x[i] = s;
            }
            if (g4 < PER) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sT[(16 * b + i) * TQ_LD + 16 * b + col] = EL::from_f(x[i]);
                    sTdT[(16 * b + col) * Cf::TD_LD + i] = EL::from_f(x[i]);
                }
            }
        }
        sync();
        // off-diagonal blocks, one block column per wave: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
        for (int jc = wave; jc < 3; jc += NW) {
            f32x4 Tp[4];
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                if (i <= jc) continue;
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 3; ++kk) {
                    if (kk < jc || kk >= i) continue;
                    Frag4<ET> fa, fb;
                    fa.load4(sA + (16 * i + l16) * SQ_LD + 16 * kk + 4 * g4);
                    if (kk == jc) fb.load4(sTdT + (16 * jc + l16) * Cf::TD_LD + 4 * g4);
                    else {
                        const float t4[4] = {Tp[kk][0], Tp[kk][1], Tp[kk][2], Tp[kk][3]};
                        fb.set(t4);
                    }
                    mma16k16(Y, fa, fb);
                }
                Frag4<ET> fa2, fy;
                fa2.load4(sT + (16 * i + l16) * TQ_LD + 16 * i + 4 * g4);
                const float y4[4] = {Y[0], Y[1], Y[2], Y[3]};
                fy.set(y4);
                f32x4 Tij = {0.f, 0.f, 0.f, 0.f};
                mma16k16(Tij, fa2, fy);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Tij[r] = -Tij[r];
                    sT[(16 * i + 4 * g4 + r) * TQ_LD + 16 * jc + l16] = EL::from_f(Tij[r]);
                }
                Tp[i] = Tij;
            }
        }
        sync();

        // ---------------- stage 7: W^T = (beta Kt)^T T^T into LDS (negated); Ut = T (beta V) in registers
        f32x16 U[2];
        {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16 acc = {};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (nt == 0 && s >= 2) continue;
                    Frag8<ET> fa, fb;
                    fa.load8(sKtT + (32 * wave + l32) * TW_LD + 16 * s + 8 * g2);
                    fb.load8(sT + (32 * nt + l32) * TQ_LD + 16 * s + 8 * g2);
                    mma32(acc, fa, fb);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float w4[4] = {-acc[4 * q], -acc[4 * q + 1], -acc[4 * q + 2], -acc[4 * q + 3]};
                    V4::store(sW + (32 * nt + l32) * QT_LD + 32 * wave + 8 * q + 4 * g2, V4::pack(w4));
                }
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                U[mt] = f32x16{};
                if (!has_v) continue;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (mt == 0 && s >= 2) continue;
                    Frag8<ET> fa, fb;
                    fa.load8(sT + (32 * mt + l32) * TQ_LD + 16 * s + 8 * g2);
                    fb.load8(sVT + (32 * wave + l32) * TW_LD + 16 * s + 8 * g2);
                    mma32(U[mt], fa, fb);
                }
            }
        }
        sync();

        // ---------------- stage 8: the state path (this wave's value slab)
        Frag8<ET> SB[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            float t8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) t8[e] = S[s >> 1][8 * (s & 1) + e];
            SB[s].set(t8);
        }
        // U = Ut - W S0
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                Frag8<ET> fa;
                const ET *row = sW + (32 * mt + l32) * QT_LD + 16 * s + 4 * g2;
                fa.load44(row, row + 8);
                mma32(U[mt], fa, SB[s]);
            }
        Frag8<ET> UB[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float t8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) t8[e] = U[s >> 1][8 * (s & 1) + e];
            UB[s].set(t8);
        }
        // O^T = S0^T Qt^T + U^T P^T, stored to out[token][value]
        if (has_out) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16 O = {};
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    Frag8<ET> fb;
                    const ET *row = sQt + (32 * nt + l32) * QT_LD + 16 * s + 4 * g2;
                    fb.load44(row, row + 8);
                    mma32(O, SB[s], fb);
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (nt == 0 && s >= 2) continue;
                    Frag8<ET> fb;
                    const ET *row = sP + (32 * nt + l32) * SQ_LD + 16 * s + 4 * g2;
                    fb.load44(row, row + 8);
                    mma32(O, UB[s], fb);
                }
                const int tok = 32 * nt + l32;
                if (tok < L) {
                    ET *dst = ob + (int64_t)(tok0 + tok) * p.o_st + 32 * wave + 4 * g2;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float o4[4] = {O[4 * q], O[4 * q + 1], O[4 * q + 2], O[4 * q + 3]};
                        V4::store(dst + 8 * q, V4::pack(o4));
                    }
                }
            }
        }
        // S <- Diag(e^{G_L}) S0 + Kh^T U
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 d = *(const float4 *)(sSc + SC_DEC * D + 32 * m + 8 * q + 4 * g2);
                S[m][4 * q + 0] *= d.x;
                S[m][4 * q + 1] *= d.y;
                S[m][4 * q + 2] *= d.z;
                S[m][4 * q + 3] *= d.w;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                Frag8<ET> fa;
                const ET *row = sKhT + (32 * m + l32) * TT_LD + 16 * s + 4 * g2;
                fa.load44(row, row + 8);
                mma32(S[m], fa, UB[s]);
            }
        }
        sync();
    }

    // ------------------------------------------------ end state
    float *dst = nullptr;
    bf16 *dsth = nullptr;         // bf16 final state (rounded to nearest even)
    int64_t rs = D;
    if (role == ROLE_OUT || (role == ROLE_SEG_OUT && seg == p.nseg - 1)) {
        if (p.sT) { dst = p.sT + n * p.sT_sn + h * p.sT_sh; rs = p.sT_sr; }
        if (p.sTh) dsth = p.sTh + n * p.sT_sn + h * p.sT_sh;
    } else if (role == ROLE_SEG_M || role == ROLE_SEG_C) {
        dst = p.ws_maps + map_offset(chain, p.nseg, seg, role == ROLE_SEG_C, D);
    }
    if (dst && role == ROLE_SEG_M) {
        store_map_m<std::is_same<ET, bf16>::value>(dst, S, lane, vcol, D);
    } else if (dst) {
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(32 * m + 8 * q + 4 * g2 + r) * rs + vcol] = S[m][4 * q + r];
    }
    if (dsth) {
#pragma unroll
        for (int m = 0; m < NMT; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dsth[(32 * m + 8 * q + 4 * g2 + r) * p.sT_sr + vcol] = (bf16)S[m][4 * q + r];
    }
}

template <int D, typename ET>
static hipError_t launch_chunk_t(const ChunkParams &p, int grid, bool stall, hipStream_t st)
{
    constexpr int NT = 64 * (D / 32);
    if (stall) hipLaunchKernelGGL((chunk_kernel<D, ET, true>), dim3(grid), dim3(NT), 0, st, p);
    else hipLaunchKernelGGL((chunk_kernel<D, ET, false>), dim3(grid), dim3(NT), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_chunk(const ChunkParams &p, int D, bool fp32, int grid, bool stall, hipStream_t st)
{
    if (grid <= 0) return hipSuccess;
    if (D == 128 && !fp32) return launch_chunk_t<128, bf16>(p, grid, stall, st);
    if (D == 64 && !fp32) return launch_chunk_t<64, bf16>(p, grid, stall, st);
    if (D == 64 && fp32) return launch_chunk_t<64, float>(p, grid, stall, st);
    return hipErrorInvalidValue;
}

}  // namespace kda
