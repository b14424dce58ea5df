// Host side of the KDA prefill C ABI (include/kda.h): descriptor validation,
// the launch plan, workspace sizing/caching and kernel enqueueing.
//
// Plan (host-known values only, never a device read): chains = N * H.  When
// chains fill the GPU's compute units one chunk-kernel workgroup runs each
// chain start to end (one launch, no workspace).  When they do not, each chain
// is cut into nseg segments and the path is segment build (M, C) -> COMBINE ->
// segment outputs (each chunk-kernel pass runs the in-chunk gate scan of PREP
// on its own chunks; the standalone PREP kernel is an option), following the
// PREP / SEG / COMB pipeline of the
// cudnn-frontend Hopper KDA prefill PR (#1056), whose launch selection picks
// the segment count from the SM count and N*H; here the CU count of the device
// plays that role.  The workspace is sized exactly for the plan and is empty
// when nseg == 1 (that PR's review found segment buffers sized by N*H but never
// used on the single-segment path).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

thread_local std::string g_last_error;

kda_status_t fail(kda_status_t st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status_t hip_fail(hipError_t e, const char *what)
{
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi) in bytes; empty when lo == hi
};

size_t elem_size(int32_t dt) { return dt == KDA_BF16 ? 2 : 4; }

Span span_of(const kda_tensor_t *t)
{
    Span s;
    if (!t || !t->data) return s;
    int64_t last = 0;
    for (int d = 0; d < t->ndim; ++d) {
        if (t->shape[d] == 0) return s;
        last += (t->shape[d] - 1) * t->stride[d];
    }
    s.lo = (uintptr_t)t->data;
    s.hi = s.lo + (uintptr_t)((last + 1) * (int64_t)elem_size(t->dtype));
    return s;
}

bool overlaps(const Span &a, const Span &b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool same_view(const kda_tensor_t *a, const kda_tensor_t *b)
{
    if (a->data != b->data || a->ndim != b->ndim || a->dtype != b->dtype) return false;
    for (int d = 0; d < a->ndim; ++d)
        if (a->shape[d] != b->shape[d] || (a->shape[d] > 1 && a->stride[d] != b->stride[d])) return false;
    return true;
}

int64_t numel(const kda_tensor_t *t)
{
    int64_t n = 1;
    for (int d = 0; d < t->ndim; ++d) n *= t->shape[d];
    return n;
}

// Strides of a token-major view as (batch, token, head) in elements.
struct Tok {
    int64_t sb = 0, st = 0, sh = 0;
};

struct Problem {
    bool dense = true;
    int64_t B = 0, T = 0, Ttot = 0, N = 0, H = 0, D = 0;
    bool fp32 = false;
    Tok q, k, v, g, beta, out;
    int64_t s0_sn = 0, s0_sh = 0, s0_sr = 0, sT_sn = 0, sT_sh = 0, sT_sr = 0;
    const kda_tensor_t *tq, *tk, *tv, *tg, *tb, *ts0, *tcu, *tout, *tsT;
};

kda_status_t check_basic(const kda_tensor_t *t, const char *name, bool allow_null)
{
    if (!t) return allow_null ? KDA_OK : fail(KDA_ERR_NULL, "%s descriptor is NULL", name);
    if (t->ndim < 1 || t->ndim > 4) return fail(KDA_ERR_SHAPE, "%s: ndim %d not in 1..4", name, t->ndim);
    for (int d = 0; d < t->ndim; ++d) {
        if (t->shape[d] < 0) return fail(KDA_ERR_SHAPE, "%s: negative extent", name);
        if (t->stride[d] < 0) return fail(KDA_ERR_LAYOUT, "%s: negative stride", name);
    }
    if (t->shape[t->ndim - 1] > 1 && t->stride[t->ndim - 1] != 1)
        return fail(KDA_ERR_LAYOUT, "%s: last-dimension stride must be 1", name);
    if (t->dtype != KDA_BF16 && t->dtype != KDA_F32 && t->dtype != KDA_I32)
        return fail(KDA_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
    if (!t->data && numel(t) > 0) return fail(KDA_ERR_NULL, "%s: data pointer is NULL", name);
    return KDA_OK;
}

// token-major tensor: dense [B, T, H, X] or packed [Ttot, H, X] / [1, Ttot, H, X];
// beta drops the last dimension.
kda_status_t tok_view(const kda_tensor_t *t, const char *name, const Problem &P, int64_t X, bool has_x, Tok &o)
{
    const int want = (P.dense ? 4 : 3) - (has_x ? 0 : 1);
    int64_t sh[4], sd[4];
    int nd = t->ndim;
    for (int d = 0; d < nd; ++d) { sh[d] = t->shape[d]; sd[d] = t->stride[d]; }
    if (!P.dense && nd == want + 1 && sh[0] == 1) {   // [1, Ttot, ...]
        for (int d = 0; d + 1 < nd; ++d) { sh[d] = sh[d + 1]; sd[d] = sd[d + 1]; }
        --nd;
    }
    if (nd != want) return fail(KDA_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, want, t->ndim);
    int i = 0;
    if (P.dense) {
        if (sh[0] != P.B) return fail(KDA_ERR_SHAPE, "%s: batch %lld != %lld", name, (long long)sh[0], (long long)P.B);
        o.sb = sd[0];
        i = 1;
    }
    if (sh[i] != (P.dense ? P.T : P.Ttot)) return fail(KDA_ERR_SHAPE, "%s: token extent mismatch", name);
    o.st = sd[i];
    if (sh[i + 1] != P.H) return fail(KDA_ERR_SHAPE, "%s: head extent mismatch", name);
    o.sh = sd[i + 1];
    if (has_x && sh[i + 2] != X) return fail(KDA_ERR_SHAPE, "%s: last extent %lld != %lld", name, (long long)sh[i + 2], (long long)X);
    return KDA_OK;
}

kda_status_t state_view(const kda_tensor_t *t, const char *name, const Problem &P, int64_t &sn, int64_t &sh, int64_t &sr)
{
    if (t->dtype != KDA_F32 && t->dtype != KDA_BF16) return fail(KDA_ERR_DTYPE, "%s must be fp32 or bf16", name);
    if (t->ndim != 4) return fail(KDA_ERR_SHAPE, "%s must be [N, H, K, V]", name);
    if (t->shape[0] != P.N || t->shape[1] != P.H || t->shape[2] != P.D || t->shape[3] != P.D)
        return fail(KDA_ERR_SHAPE, "%s: shape must be [%lld, %lld, %lld, %lld]", name, (long long)P.N,
                    (long long)P.H, (long long)P.D, (long long)P.D);
    sn = t->stride[0];
    sh = t->stride[1];
    sr = t->stride[2];
    return KDA_OK;
}

kda_status_t validate(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v, const kda_tensor_t *g,
                      const kda_tensor_t *beta, const kda_tensor_t *s0, const kda_tensor_t *cu,
                      const kda_tensor_t *out, const kda_tensor_t *sT, Problem &P)
{
    kda_status_t st;
    if ((st = check_basic(q, "q", false)) || (st = check_basic(k, "k", false)) || (st = check_basic(v, "v", false)) ||
        (st = check_basic(g, "g", false)) || (st = check_basic(beta, "beta", false)) ||
        (st = check_basic(out, "out", false)) || (st = check_basic(s0, "initial_state", true)) ||
        (st = check_basic(cu, "cu_seqlens", true)) || (st = check_basic(sT, "final_state", true)))
        return st;
    P.tq = q; P.tk = k; P.tv = v; P.tg = g; P.tb = beta; P.ts0 = s0; P.tcu = cu; P.tout = out; P.tsT = sT;
    if (q->dtype != KDA_BF16 && q->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "q must be bf16 or fp32");
    if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype)
        return fail(KDA_ERR_DTYPE, "q, k, v and out must share one dtype");
    if (g->dtype != KDA_F32 || beta->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "g and beta must be fp32");
    P.fp32 = q->dtype == KDA_F32;
    P.dense = (cu == nullptr);
    if (P.dense) {
        if (q->ndim != 4) return fail(KDA_ERR_SHAPE, "dense q must be [B, T, H, K]");
        P.B = q->shape[0];
        P.T = q->shape[1];
        P.N = P.B;
        P.Ttot = P.B * P.T;
        P.H = q->shape[2];
        P.D = q->shape[3];
    } else {
        if (cu->dtype != KDA_I32) return fail(KDA_ERR_DTYPE, "cu_seqlens must be int32");
        if (cu->ndim != 1 || cu->shape[0] < 1) return fail(KDA_ERR_SHAPE, "cu_seqlens must be [N + 1]");
        P.N = cu->shape[0] - 1;
        if (q->ndim == 4) {
            if (q->shape[0] != 1) return fail(KDA_ERR_SHAPE, "packed 4-D q needs batch 1");
            P.Ttot = q->shape[1]; P.H = q->shape[2]; P.D = q->shape[3];
        } else if (q->ndim == 3) {
            P.Ttot = q->shape[0]; P.H = q->shape[1]; P.D = q->shape[2];
        } else {
            return fail(KDA_ERR_SHAPE, "packed q must be [T, H, K] or [1, T, H, K]");
        }
        P.B = 1;
        P.T = 0;
    }
    if (P.H < 1) return fail(KDA_ERR_SHAPE, "H must be >= 1");
    if (P.D != 64 && P.D != 128) return fail(KDA_ERR_UNSUPPORTED, "head size %lld not in {64, 128}", (long long)P.D);
    if (P.fp32 && P.D != 64) return fail(KDA_ERR_UNSUPPORTED, "the fp32 debug mode supports head size 64 only");
    if (P.Ttot >= (int64_t)1 << 31 || P.N >= (int64_t)1 << 31 || P.N * P.H >= (int64_t)1 << 31)
        return fail(KDA_ERR_SHAPE, "problem too large for 32-bit token indexing");
    if ((st = tok_view(q, "q", P, P.D, true, P.q)) || (st = tok_view(k, "k", P, P.D, true, P.k)) ||
        (st = tok_view(v, "v", P, P.D, true, P.v)) || (st = tok_view(g, "g", P, P.D, true, P.g)) ||
        (st = tok_view(beta, "beta", P, 0, false, P.beta)) || (st = tok_view(out, "out", P, P.D, true, P.out)))
        return st;
    if (s0 && (st = state_view(s0, "initial_state", P, P.s0_sn, P.s0_sh, P.s0_sr))) return st;
    if (sT && (st = state_view(sT, "final_state", P, P.sT_sn, P.sT_sh, P.sT_sr))) return st;
    // vector widths: 4 consecutive channels per access, rows aligned to them
    auto aligned = [&](const kda_tensor_t *t) {
        if (!t || !t->data) return true;
        const size_t es = elem_size(t->dtype), vec = 4 * es;
        if ((uintptr_t)t->data % vec) return false;
        for (int d = 0; d + 1 < t->ndim; ++d)
            if (t->shape[d] > 1 && (t->stride[d] * es) % vec) return false;
        return true;
    };
    if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(g) || !aligned(out))
        return fail(KDA_ERR_LAYOUT, "q, k, v, g, out need 4-element-aligned base addresses and strides");
    // aliasing
    const Span so = span_of(out);
    const kda_tensor_t *ins[] = {q, k, v, g, beta, s0, cu};
    const char *names[] = {"q", "k", "v", "g", "beta", "initial_state", "cu_seqlens"};
    for (int i = 0; i < 7; ++i)
        if (ins[i] && overlaps(so, span_of(ins[i]))) return fail(KDA_ERR_ALIAS, "out overlaps %s", names[i]);
    if (sT) {
        const Span ss = span_of(sT);
        if (overlaps(ss, so)) return fail(KDA_ERR_ALIAS, "final_state overlaps out");
        for (int i = 0; i < 7; ++i) {
            if (!ins[i]) continue;
            if (i == 5 && same_view(sT, s0)) continue;   // exact in-place state update
            if (overlaps(ss, span_of(ins[i]))) return fail(KDA_ERR_ALIAS, "final_state overlaps %s", names[i]);
        }
    }
    return KDA_OK;
}

// Output-norm options: out_gate like out (same shape, dtype; rows 4-element aligned), weight
// fp32 [D] contiguous, eps > 0; neither may overlap out or the state the call writes
// (prefill's final state, decode's pool): other workgroups read them while it is written.
kda_status_t check_out_norm(const kda_options_t *o, const kda_tensor_t *out, int64_t D, const kda_tensor_t *state,
                            const char *state_name)
{
    if (!o || (!o->out_gate && !o->norm_weight)) return KDA_OK;
    kda_status_t st;
    if ((st = check_basic(o->out_gate, "out_gate", false)) || (st = check_basic(o->norm_weight, "norm_weight", false)))
        return st;
    if (!out) return fail(KDA_ERR_NULL, "the output norm needs out");
    const kda_tensor_t *z = o->out_gate, *w = o->norm_weight;
    if (z->dtype != out->dtype) return fail(KDA_ERR_DTYPE, "out_gate must have out's dtype");
    if (z->ndim != out->ndim) return fail(KDA_ERR_SHAPE, "out_gate must have out's shape");
    for (int d = 0; d < z->ndim; ++d)
        if (z->shape[d] != out->shape[d]) return fail(KDA_ERR_SHAPE, "out_gate must have out's shape");
    const int64_t es = (int64_t)elem_size(z->dtype);
    if ((uintptr_t)z->data % (4 * es)) return fail(KDA_ERR_LAYOUT, "out_gate needs a 4-element-aligned base");
    for (int d = 0; d + 1 < z->ndim; ++d)
        if (z->shape[d] > 1 && (z->stride[d] * es) % (4 * es))
            return fail(KDA_ERR_LAYOUT, "out_gate needs 4-element-aligned strides");
    if (w->dtype != KDA_F32 || w->ndim != 1 || w->shape[0] != D)
        return fail(KDA_ERR_SHAPE, "norm_weight must be fp32 [%lld]", (long long)D);
    if ((uintptr_t)w->data % 16) return fail(KDA_ERR_LAYOUT, "norm_weight needs a 16-byte-aligned base");
    if (!(o->norm_eps > 0.f) || !(o->norm_eps < 1e30f)) return fail(KDA_ERR_UNSUPPORTED, "norm_eps must be positive");
    const Span so = span_of(out);
    if (overlaps(so, span_of(z)) || overlaps(so, span_of(w))) return fail(KDA_ERR_ALIAS, "out overlaps out_gate or norm_weight");
    const Span ss = span_of(state);
    if (overlaps(ss, span_of(z)) || overlaps(ss, span_of(w)))
        return fail(KDA_ERR_ALIAS, "%s overlaps out_gate or norm_weight", state_name);
    return KDA_OK;
}

// ------------------------------------------------------------------ environment
// KDA_LOG=1: every plan to stderr.  KDA_CHECK=1: cu_seqlens checked on the device before
// anything else is launched (one small kernel, a stream sync and a 4-byte read back).
bool env_on(const char *name)
{
    const char *v = getenv(name);
    return v && *v && strcmp(v, "0") != 0;
}

std::mutex g_check_mu;                 // held for a whole check: one flag buffer per device
std::vector<int32_t *> g_check_flag;   // per device, allocated on first use

// The KDA_CHECK=1 device checks, before anything else of the call is enqueued: cu_seqlens
// (when given: cu[0] == 0, non-decreasing, cu[N] == T_tot), the values of g (when given:
// within [g.lo, g.hi], NaN refused) and decode's slot indices (when given: no two requests
// name the same slot in [0, P)).  Zeroes three flags, runs the checks, reads the flags back
// and synchronises the stream; returns KDA_ERR_SHAPE, KDA_ERR_RANGE or KDA_ERR_ALIAS.
struct DeviceChecks {
    const int32_t *cu = nullptr;
    int64_t N = 0, Ttot = 0;
    bool check_g = false;
    kda::CheckG g{};
    const int32_t *slots = nullptr;
    int64_t R = 0, P = 0;
};

// flags: device memory for the three flags, or NULL for the library's own buffer (allocated on
// a device's first check).
kda_status_t run_device_checks(const DeviceChecks &c, hipStream_t st, int32_t *flags)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    // the lock covers the launches and the read-back, so that checks on other streams of the
    // device never write the flags in between
    std::lock_guard<std::mutex> lk(g_check_mu);
    int32_t *flag = flags;
    if (!flag) {
        if ((int)g_check_flag.size() <= dev) g_check_flag.resize(dev + 1, nullptr);
        if (!g_check_flag[dev] && (e = hipMalloc(&g_check_flag[dev], 256)) != hipSuccess) {
            g_check_flag[dev] = nullptr;
            return hip_fail(e, "device check buffer");
        }
        flag = g_check_flag[dev];
    }
    int32_t h[3] = {0, 0, 0};
    if ((e = hipMemsetAsync(flag, 0, sizeof(h), st)) != hipSuccess) return hip_fail(e, "device check reset");
    if (c.cu && (e = kda::launch_check_cu(c.cu, (int32_t)c.N, c.Ttot, flag, st)) != hipSuccess)
        return hip_fail(e, "cu_seqlens check");
    if (c.check_g && (e = kda::launch_check_g(c.g, flag + 1, st)) != hipSuccess) return hip_fail(e, "g range check");
    if (c.slots && (e = kda::launch_check_slots(c.slots, (int32_t)c.R, (int32_t)c.P, flag + 2, st)) != hipSuccess)
        return hip_fail(e, "slot check");
    if ((e = hipMemcpyAsync(h, flag, sizeof(h), hipMemcpyDeviceToHost, st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess)
        return hip_fail(e, "device check read-back");
    if (h[0]) return fail(KDA_ERR_SHAPE, "cu_seqlens is not an offset array (cu[0] == 0, non-decreasing, cu[N] == %lld)",
                          (long long)c.Ttot);
    if (h[1]) {
        if (c.g.lo == -INFINITY) return fail(KDA_ERR_RANGE, "g (logits) holds NaN");
        return fail(KDA_ERR_RANGE, "g holds values outside [%g, %g] (or NaN)", (double)c.g.lo, (double)c.g.hi);
    }
    if (h[2]) return fail(KDA_ERR_ALIAS, "two requests name the same state slot with the state update on");
    return KDA_OK;
}

// The g view of a token-major problem for the range check: raw log decays must lie in the
// range the kernels are guaranteed on, [-5, 0]; logits (gate_act) may be anything but NaN.
kda::CheckG g_view(const kda_tensor_t *g, int64_t rows, int64_t rows_per_b, int64_t sb, int64_t st, int64_t sh,
                   int64_t H, int64_t D, bool logits)
{
    kda::CheckG c{};
    c.g = (const float *)g->data;
    c.rows = rows; c.rows_per_b = rows_per_b; c.sb = sb; c.st = st; c.sh = sh; c.H = H; c.D = D;
    c.lo = logits ? -INFINITY : -5.f;
    c.hi = logits ? INFINITY : 0.f;
    return c;
}

// ------------------------------------------------------------------ plan
struct Plan {
    int nseg = 1;
    int64_t seg_chains = 0;     // chains cut into nseg segments: the last seg_chains of the N*H
    bool pipe = false;          // pipelined 32-token kernel (d = 128, bf16)
    int chunk = 64;
    bool standalone_prep = false;
    bool lpt = false;           // chains started longest sequence first
    int cap_slots = 0;          // capped concurrency: groups of H workgroups (0 = off)
    size_t off_gamma = 0, off_maps = 0, off_start = 0, bytes = 0;
    size_t off_flags = 0;       // the capped schedule's flags, last in the workspace: a smaller
                                // workspace that holds everything before them runs uncapped
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Capped concurrency: on MI355X the chunk kernel's step time stays within 6% of its low-load
// value up to about 160 concurrent chains (dense 4,096-token chains: 128 -> 2.00 us, 160 ->
// 2.04, 192 -> 2.26, 256 -> 2.67 us per step).
constexpr int64_t kCapChains = 160;
std::atomic<uint32_t> g_cap_epoch{0};

int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

// Segment count from a cost model in units of one chunk step of a launch that leaves most CUs
// idle (~2.07 us on MI355X).  One segment: C + 3 steps (the longest chain's chunks and the pass's
// fixed cost below).  nseg segments
// of ceil(C / nseg) chunks: the map pass builds segments 0 .. nseg - 2, one workgroup per
// segment on the pipelined kernel (both maps; measured as fast per step as an output step) or
// two on the single-role kernel, in ceil(workgroups / CUs) rounds; the output pass runs
// ceil(chains nseg / CUs) rounds.  A pass that fills the CUs runs its steps ~1.2x slower (the
// clock drops under full load) and pays ~3 steps of its own (the first state, the pipeline's
// fill, the final stores); COMBINE costs ~4.4 + 0.45 per map segment.  Measured on MI355X over
// 17 dense shapes (8 to 192 chains, 32 to 2048 chunks), this picks the fastest forced count at
// every one of them.  The cheapest count wins, ties to fewer segments, keeping >= 8
// chunks per segment.  (With every CU already holding a chain, segmenting cannot pay and one
// segment is kept.)
int choose_nseg(int64_t chains, int64_t C, int cus, bool merged_maps)
{
    if (chains <= 0 || chains >= cus || C < 16) return 1;
    double best = (double)C + 3.0;
    int pick = 1;
    for (int nseg = 2; nseg <= 64 && C / nseg >= 8; ++nseg) {
        const double steps = (double)((C + nseg - 1) / nseg) + 3.0;
        const int64_t wg1 = chains * (nseg - 1) * (merged_maps ? 1 : 2), wg2 = chains * nseg;
        const double r1 = (double)((wg1 + cus - 1) / cus), r2 = (double)((wg2 + cus - 1) / cus);
        const double cost = 1.2 * steps * (r1 + r2) + 4.4 + 0.45 * (nseg - 1);
        if (cost < best) { best = cost; pick = nseg; }
    }
    return pick;
}

// Split plans: chains = k CUs + r with k >= 1 leave a last round of r chains on r CUs.  Cutting
// only those r chains into s segments -- their maps, COMBINE, then one launch holding their
// segment outputs and the k CUs whole chains -- ends at about k rounds plus two short
// segment passes.  Same cost units as choose_nseg; returns r (and s) when that beats k + 1 whole
// rounds (the last one at the low-load clock), else 0.
int64_t choose_split(int64_t chains, int64_t C, int cus, int &s_out)
{
    if (chains <= cus || C < 16) return 0;
    const int64_t k = chains / cus, r = chains % cus;
    if (r == 0) return 0;
    const double whole = 1.2 * k * (C + 3) + 1.0 * (C + 3);
    double best = whole;
    int pick = 0;
    for (int s = 2; s <= 16 && C / s >= 8; ++s) {
        const double steps = (double)((C + s - 1) / s) + 3.0;
        const double maps = (double)((r * (s - 1) + cus - 1) / cus) * steps;
        const double outs = k * (double)(C + 3) + (double)((r * s + cus - 1) / cus) * steps;
        const double cost = 1.2 * (maps + outs) + 4.4 + 0.45 * (s - 1);
        if (cost < best) { best = cost; pick = s; }
    }
    if (!pick) return 0;
    s_out = pick;
    return r;
}

// max_bytes > 0 caps the workspace (the no-alloc entry point's fixed scratch): an automatic
// segment count is lowered until the plan fits (one segment needs none); a forced segment
// count or standalone PREP that does not fit is refused.
kda_status_t make_plan(const Problem &P, const kda_options_t *o, Plan &pl, size_t max_bytes = 0)
{
    const int64_t chains = P.N * P.H;
    const int variant = o ? o->variant : 0;
    if (variant < 0 || variant > 2) return fail(KDA_ERR_UNSUPPORTED, "kernel variant %d", variant);
    // the pipelined kernel addresses a 32-token chunk of every token-major tensor with 32-bit
    // byte offsets from the chunk's first row
    auto rows32 = [](const Tok &t, int64_t es) { return 32 * t.st * es + 1024 <= (int64_t)INT32_MAX; };
    const bool pipe_ok = P.D == 128 && !P.fp32 && rows32(P.q, 2) && rows32(P.k, 2) && rows32(P.v, 2) &&
                         rows32(P.out, 2) && rows32(P.g, 4) && rows32(P.beta, 4);
    if (variant == 2 && !pipe_ok)
        return fail(KDA_ERR_UNSUPPORTED, "the pipelined kernel needs head size 128, bf16 and token strides below 2^31 / 32 bytes");
    pl.pipe = pipe_ok && variant != 1;
    pl.chunk = pl.pipe ? 32 : 64;
    const int64_t max_chunks = P.dense ? (P.T + pl.chunk - 1) / pl.chunk : (P.Ttot + pl.chunk - 1) / pl.chunk;
    const int cus = device_cus();
    if (o && o->nseg > 0) {
        if (o->nseg > 64) return fail(KDA_ERR_UNSUPPORTED, "nseg %d > 64", o->nseg);
        pl.nseg = o->nseg;
    } else {
        pl.nseg = choose_nseg(chains, max_chunks, cus, pl.pipe);
    }
    pl.seg_chains = pl.nseg > 1 ? chains : 0;
    const int split = o ? o->split_chains : 0;
    if (split < 0) return fail(KDA_ERR_UNSUPPORTED, "split_chains %d", split);
    if (split > 0) {
        if (!(o->nseg > 1) || !pl.pipe || split > chains)
            return fail(KDA_ERR_UNSUPPORTED, "split_chains needs a forced nseg > 1, the pipelined kernel and at most "
                                             "N*H chains");
        pl.seg_chains = split;
    } else if (!(o && o->nseg > 0) && pl.pipe && P.dense) {
        int s = 1;
        const int64_t r = choose_split(chains, max_chunks, cus, s);
        if (r > 0) { pl.nseg = s; pl.seg_chains = r; }
    }
    // the segment-build launch has up to chains * (nseg - 1) * 2 workgroups (a 32-bit grid)
    if (chains * pl.nseg * 2 > (int64_t)INT32_MAX)
        return fail(KDA_ERR_UNSUPPORTED, "%lld chains x %d segments exceed one launch", (long long)chains, pl.nseg);
    const int prep = o ? o->prep : 0;
    if (prep < 0 || prep > 2) return fail(KDA_ERR_UNSUPPORTED, "prep mode %d", prep);
    if (o && (o->gate_act < 0 || o->gate_act > 1 || o->beta_act < 0 || o->beta_act > 1))
        return fail(KDA_ERR_UNSUPPORTED, "gate_act %d / beta_act %d (0 or 1)", o->gate_act, o->beta_act);
    if (o && o->gate_act && !(o->gate_lower_bound >= -5.f && o->gate_lower_bound <= 0.f))
        return fail(KDA_ERR_UNSUPPORTED, "gate_lower_bound %g outside [-5, 0]", (double)o->gate_lower_bound);
    kda_status_t st;
    if ((st = check_out_norm(o, P.tout, P.D, P.tsT, "final_state"))) return st;
    if (o && o->out_gate && !pl.pipe)
        return fail(KDA_ERR_UNSUPPORTED, "the output norm runs on the pipelined kernel (head size 128, bf16)");
    if (o && o->out_gate && 32 * o->out_gate->stride[o->out_gate->ndim - 3] * 2 + 1024 > (int64_t)INT32_MAX)
        return fail(KDA_ERR_UNSUPPORTED, "out_gate token stride too large for the pipelined kernel");
    pl.standalone_prep = prep == 1;   // otherwise every chunk-kernel pass scans its own chunks
    // Capped concurrency (the kernel's cap_wait): a packed batch on one segment with every chain
    // resident at once, and more chains than the cap.  The kernel decides from the lengths
    // whether the packing leaves the longest sequence as the bound, else it runs uncapped.
    // KDA_CAP sets the cap in chains (0 turns it off).
    {
        const char *ce = getenv("KDA_CAP");
        const int64_t cap = ce ? atoll(ce) : kCapChains;
        const int64_t S = (cap > 0 && P.H > 0) ? cap / P.H : 0;
        const int cus = device_cus();
        if (pl.pipe && !P.dense && P.N > 1 && P.N <= kda::CAP_MAX_N && chains <= cus && S >= 1 &&
            S * P.H < chains && S <= kda::CAP_MAX_SLOTS && P.N * S <= kda::CAP_MAX_WORK)
            pl.cap_slots = (int)S;
    }
    auto layout = [&](int nseg) {
        size_t off = 0;
        if (pl.standalone_prep) {
            pl.off_gamma = off;
            off += align256((size_t)P.Ttot * P.H * P.D * 4);
        }
        if (nseg > 1) {
            const size_t dd = (size_t)P.D * P.D * 4;
            const size_t sc = (size_t)pl.seg_chains;           // the segmented chains' slots
            pl.off_maps = off;                                   // segments 0 .. nseg - 2
            off += align256(sc * (nseg - 1) * 2 * dd);
            pl.off_start = off;
            off += align256(sc * nseg * dd);
        }
        if (nseg == 1 && pl.cap_slots > 0) {
            pl.off_flags = off;
            off += align256((size_t)chains * 8);
        }
        return off;
    };
    pl.bytes = layout(pl.nseg);
    if (max_bytes && pl.bytes > max_bytes) {
        const bool forced = (o && o->nseg > 0) || pl.standalone_prep;
        if (forced)
            return fail(KDA_ERR_WORKSPACE, "the plan needs %zu bytes of scratch, more than the %zu the no-alloc entry point has",
                        pl.bytes, max_bytes);
        while (pl.nseg > 1 && layout(pl.nseg) > max_bytes) --pl.nseg;
        if (pl.nseg == 1) pl.seg_chains = 0;
        pl.bytes = layout(pl.nseg);
        if (pl.bytes > max_bytes) {      // only the capped schedule's flags can be left
            pl.cap_slots = 0;
            pl.bytes = layout(pl.nseg);
        }
    }
    // Chain order.  With more chains than CUs, workgroups start in launch order as CUs free up,
    // so a packed batch of mixed lengths finishes sooner when its longest sequences start first
    // (longest-processing-time order); with every chain resident at once the order is moot.
    // The lengths are on the device: the kernel ranks them (pipelined kernel, one segment,
    // at most LPT_MAX_SEQ sequences).  KDA_ORDER=natural or =longest overrides the choice.
    const char *ord = getenv("KDA_ORDER");
    const bool lpt_ok = pl.pipe && pl.nseg == 1 && !P.dense && P.N > 1 && P.N <= kda::LPT_MAX_SEQ;
    if (pl.nseg > 1) pl.cap_slots = 0;
    if (ord && strcmp(ord, "natural") == 0) pl.lpt = false;
    else if (ord && strcmp(ord, "longest") == 0) pl.lpt = lpt_ok;
    else pl.lpt = lpt_ok && chains > device_cus();
    if (env_on("KDA_LOG"))
        fprintf(stderr, "kda: plan N=%lld H=%lld D=%lld %s chains=%lld nseg=%d segmented=%lld kernel=%s chunk=%d prep=%s order=%s cap=%d workspace=%zu B\n",
                (long long)P.N, (long long)P.H, (long long)P.D, P.dense ? "dense" : "packed", (long long)chains,
                pl.nseg, (long long)pl.seg_chains, pl.pipe ? "pipelined" : "single-role", pl.chunk,
                pl.standalone_prep ? "standalone" : "in-chunk", pl.lpt ? "longest-first" : "natural",
                pl.cap_slots * (int)P.H, pl.bytes);
    return KDA_OK;
}

// ------------------------------------------------------------- profiling
struct ProfRec {
    const char *name;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;                         // launches recorded since the last read
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_pool;   // idle event pairs
bool g_prof_on = false;

// Event pairs come from a pool that profiling's enable call fills, so that a timed launch
// costs two event records and no event creation.
hipError_t prof_pair(hipEvent_t &a, hipEvent_t &b)
{
    if (!g_prof_pool.empty()) {
        a = g_prof_pool.back().first;
        b = g_prof_pool.back().second;
        g_prof_pool.pop_back();
        return hipSuccess;
    }
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    return e;
}

template <typename F>
hipError_t timed(const char *name, hipStream_t st, F &&launch)
{
    if (!g_prof_on) return launch();
    ProfRec r{name, nullptr, nullptr};
    hipError_t e;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if ((e = prof_pair(r.a, r.b)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(r.a, st)) != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(r.b, st)) != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back(r);
    return hipSuccess;
}

// --------------------------------------------------------------- enqueue
// check_flags: where the KDA_CHECK=1 device checks keep their flags (NULL: the library's own
// buffer, allocated on a device's first check).
kda_status_t run(const Problem &P, const Plan &pl, const kda_options_t *o, void *ws, size_t ws_bytes, hipStream_t st,
                 int32_t *check_flags = nullptr)
{
    // the capped schedule's flags come last: a workspace without them runs uncapped
    const size_t need = pl.cap_slots > 0 ? pl.off_flags : pl.bytes;
    if (ws_bytes < need || (need && !ws))
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, pl.bytes);
    if (ws && need && ((uintptr_t)ws % 256)) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const bool cap_on = pl.cap_slots > 0 && ws && ws_bytes >= pl.bytes && (uintptr_t)ws % 256 == 0;
    const int64_t chains = P.N * P.H;
    if (chains == 0) return KDA_OK;
    char *wsb = (char *)ws;
    if (env_on("KDA_CHECK")) {
        DeviceChecks dc;
        if (P.tcu) { dc.cu = (const int32_t *)P.tcu->data; dc.N = P.N; dc.Ttot = P.Ttot; }
        dc.check_g = true;
        dc.g = g_view(P.tg, P.Ttot, P.dense ? P.T : P.Ttot, P.g.sb, P.g.st, P.g.sh, P.H, P.D, o && o->gate_act);
        kda_status_t s = run_device_checks(dc, st, check_flags);
        if (s) return s;
    }

    kda::ChunkParams cp{};
    cp.q = P.tq->data; cp.k = P.tk->data; cp.v = P.tv->data;
    cp.g = (const float *)P.tg->data; cp.beta = (const float *)P.tb->data;
    cp.s0 = (P.ts0 && P.ts0->dtype == KDA_F32) ? (const float *)P.ts0->data : nullptr;
    cp.s0h = (P.ts0 && P.ts0->dtype == KDA_BF16) ? (const kda::bf16 *)P.ts0->data : nullptr;
    cp.o = P.tout->data;
    cp.sT = (P.tsT && P.tsT->dtype == KDA_F32) ? (float *)P.tsT->data : nullptr;
    cp.sTh = (P.tsT && P.tsT->dtype == KDA_BF16) ? (kda::bf16 *)P.tsT->data : nullptr;
    cp.cu = P.tcu ? (const int32_t *)P.tcu->data : nullptr;
    cp.q_sb = P.q.sb; cp.q_st = P.q.st; cp.q_sh = P.q.sh;
    cp.k_sb = P.k.sb; cp.k_st = P.k.st; cp.k_sh = P.k.sh;
    cp.v_sb = P.v.sb; cp.v_st = P.v.st; cp.v_sh = P.v.sh;
    cp.g_sb = P.g.sb; cp.g_st = P.g.st; cp.g_sh = P.g.sh;
    cp.b_sb = P.beta.sb; cp.b_st = P.beta.st; cp.b_sh = P.beta.sh;
    cp.o_sb = P.out.sb; cp.o_st = P.out.st; cp.o_sh = P.out.sh;
    cp.s0_sn = P.s0_sn; cp.s0_sh = P.s0_sh; cp.s0_sr = P.s0_sr;
    cp.sT_sn = P.sT_sn; cp.sT_sh = P.sT_sh; cp.sT_sr = P.sT_sr;
    cp.N = (int32_t)P.N; cp.H = (int32_t)P.H; cp.T = (int32_t)P.T;
    cp.nseg = pl.nseg;
    cp.g_is_gamma = 0;
    cp.stall_wave = (o && o->stall_wave > 0) ? o->stall_wave - 1 : -1;
    cp.stall_iters = (o && o->stall_cycles > 0) ? std::max(1, o->stall_cycles / 127) : 0;
    cp.gate_act = (o && o->gate_act) ? 1 : 0;
    cp.gate_lb = o ? o->gate_lower_bound : 0.f;
    cp.beta_act = (o && o->beta_act) ? 1 : 0;
    cp.lpt = pl.lpt ? 1 : 0;
    if (cap_on) {
        cp.cap_slots = pl.cap_slots;
        cp.cap_flags = (uint64_t *)(wsb + pl.off_flags);
        // a fresh value per call, never 0: flags left by earlier calls (or the workspace's first
        // contents, unless they happen to match) do not release a waiting workgroup early
        uint32_t e = g_cap_epoch.fetch_add(1) + 1;
        if (e == 0) e = g_cap_epoch.fetch_add(1) + 1;
        cp.cap_epoch = e;
        const char *we = getenv("KDA_CAP_WAIT_US");
        cp.cap_wait_us = we ? std::max(1, atoi(we)) : 0;
    }
    if (o && o->out_gate) {
        cp.z = o->out_gate->data;
        cp.nw = (const float *)o->norm_weight->data;
        cp.eps = o->norm_eps;
        const int nd = o->out_gate->ndim;
        const int64_t *zs = o->out_gate->stride;
        // out_gate shares out's layout: dense [B, T, H, V] or packed [T, H, V] / [1, T, H, V]
        cp.z_sb = P.dense ? zs[0] : 0;
        cp.z_st = zs[nd - 3];
        cp.z_sh = zs[nd - 2];
    }
    const bool stall = cp.stall_wave >= 0 && cp.stall_iters > 0;
    const int D = (int)P.D;
    hipError_t e;
    auto chunk = [&](int grid) {
        return pl.pipe ? kda::launch_chunk_pipe(cp, grid, stall, st) : kda::launch_chunk(cp, D, P.fp32, grid, stall, st);
    };

    if (pl.standalone_prep) {
        kda::PrepParams pp{};
        float *gam = (float *)(wsb + pl.off_gamma);
        pp.g = cp.g; pp.gamma = gam; pp.cu = cp.cu;
        pp.g_sb = P.g.sb; pp.g_st = P.g.st; pp.g_sh = P.g.sh;
        // workspace Gamma: contiguous [B*T or Ttot, H, D]
        pp.y_st = P.H * P.D; pp.y_sh = P.D; pp.y_sb = P.dense ? P.T * P.H * P.D : 0;
        pp.N = (int32_t)P.N; pp.H = (int32_t)P.H; pp.T = (int32_t)P.T; pp.D = D;
        pp.chunk = pl.chunk;
        pp.chunks_per_seq = P.dense ? (int32_t)((P.T + pl.chunk - 1) / pl.chunk) : 0;
        pp.gate_act = cp.gate_act;
        pp.gate_lb = cp.gate_lb;
        const int64_t nvc = P.dense ? P.B * pp.chunks_per_seq : (P.Ttot + pl.chunk - 1) / pl.chunk + P.N;
        if ((e = timed("kda_prep", st, [&] { return kda::launch_prep(pp, (int)nvc, st); })) != hipSuccess)
            return hip_fail(e, "PREP launch");
        cp.g = gam;
        cp.g_sb = pp.y_sb; cp.g_st = pp.y_st; cp.g_sh = pp.y_sh;
        cp.g_is_gamma = 1;
    }
    cp.seg_chain0 = 0;
    cp.n_segwg = 0;
    if (pl.nseg == 1) {
        cp.role = kda::ROLE_OUT;
        if ((e = timed("kda_chunk", st, [&] { return chunk((int)chains); })) != hipSuccess)
            return hip_fail(e, "chunk launch");
        return KDA_OK;
    }
    // chains seg_chain0 .. chains - 1 are segmented (all of them unless the plan splits)
    const int64_t segc = pl.seg_chains, whole = chains - segc;
    cp.seg_chain0 = (int32_t)whole;
    cp.n_segwg = (int32_t)(segc * pl.nseg);
    cp.ws_maps = (float *)(wsb + pl.off_maps);
    cp.ws_start = (const float *)(wsb + pl.off_start);
    // The maps of segments 0 .. nseg - 2 (COMBINE never reads the last segment's): the pipelined
    // kernel builds M and C of a segment in one workgroup, the single-role kernel in two.
    cp.role = pl.pipe ? kda::ROLE_SEG_MC : kda::ROLE_SEG_M;
    if ((e = timed("kda_chunk_segbuild", st, [&] {
             return chunk((int)(segc * (pl.nseg - 1) * (pl.pipe ? 1 : 2)));
         })) != hipSuccess)
        return hip_fail(e, "segment-build launch");
    kda::CombineParams mp{};
    mp.maps = cp.ws_maps; mp.start = (float *)(wsb + pl.off_start);
    mp.s0 = cp.s0; mp.s0h = cp.s0h; mp.s0_sn = P.s0_sn; mp.s0_sh = P.s0_sh; mp.s0_sr = P.s0_sr;
    mp.N = (int32_t)P.N; mp.H = (int32_t)P.H; mp.nseg = pl.nseg; mp.seg_chain0 = cp.seg_chain0;
    if ((e = timed("kda_combine", st, [&] { return kda::launch_combine(mp, D, !P.fp32, (int)segc, st); })) != hipSuccess)
        return hip_fail(e, "combine launch");
    // the segment outputs, then (a split plan) the whole chains 0 .. seg_chain0 - 1
    cp.role = kda::ROLE_SEG_OUT;
    if ((e = timed("kda_chunk_segout", st, [&] {
             return chunk((int)(segc * pl.nseg + whole));
         })) != hipSuccess)
        return hip_fail(e, "segment-output launch");
    return KDA_OK;
}

// kda_prefill's workspace cache: one buffer per (device, stream), so calls on different
// streams never share memory, and a buffer is only replaced after its own stream has
// finished with it.  The lock is held until the call has enqueued its kernels: a call
// from another thread on the same stream that grows the buffer then waits for them.
std::mutex g_ws_mu;
struct CachedWs {
    int dev = 0;
    void *stream = nullptr;
    void *p = nullptr;
    size_t bytes = 0;
};
std::vector<CachedWs> g_ws;

// ------------------------------------------------------ the no-alloc entry point's scratch
// kda_prefill_noalloc keeps its workspace in this fixed array: KDA_NOALLOC_SCRATCH_BYTES for the
// plan, then 256 bytes for the KDA_CHECK=1 flags.  Every GPU the library runs on holds its own
// copy, at its own address, from the code object's load until the process ends.  In host code
// the name `scratch` is a host-side stand-in, not a device address, so it is never passed to a
// kernel or a copy: the address is asked of the runtime once per device and kept.
constexpr size_t NOALLOC_FLAGS = 256;
static __device__ __align__(256) char scratch[(size_t)KDA_NOALLOC_SCRATCH_BYTES + NOALLOC_FLAGS];

std::mutex g_scratch_mu;
std::vector<char *> g_scratch_ptr;     // per device: scratch's device address

kda_status_t scratch_address(char *&ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_fail(e, "scratch address");
        if (!p) return fail(KDA_ERR_HIP, "scratch address: the runtime returned NULL");
        g_scratch_ptr[dev] = (char *)p;
    }
    ptr = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_prefill_noalloc(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                                 const kda_tensor_t *g, const kda_tensor_t *beta, const kda_tensor_t *initial_state,
                                 const kda_tensor_t *cu_seqlens, kda_tensor_t *out, kda_tensor_t *final_state,
                                 const kda_options_t *opts, void *stream)
{
    Problem P;
    kda_status_t st = validate(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, P);
    if (st) return st;
    Plan pl;
    if ((st = make_plan(P, opts, pl, (size_t)KDA_NOALLOC_SCRATCH_BYTES))) return st;
    char *ws = nullptr;
    if ((st = scratch_address(ws))) return st;
    return run(P, pl, opts, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream,
               (int32_t *)(ws + (size_t)KDA_NOALLOC_SCRATCH_BYTES));
}

kda_status_t kda_prefill_workspace_size(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                                        const kda_tensor_t *g, const kda_tensor_t *beta,
                                        const kda_tensor_t *initial_state, const kda_tensor_t *cu_seqlens,
                                        const kda_tensor_t *out, const kda_tensor_t *final_state,
                                        const kda_options_t *opts, size_t *bytes)
{
    if (!bytes) return fail(KDA_ERR_NULL, "bytes is NULL");
    Problem P;
    kda_status_t st = validate(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, P);
    if (st) return st;
    Plan pl;
    if ((st = make_plan(P, opts, pl))) return st;
    *bytes = pl.bytes;
    return KDA_OK;
}

kda_status_t kda_prefill_ws(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                            const kda_tensor_t *g, const kda_tensor_t *beta, const kda_tensor_t *initial_state,
                            const kda_tensor_t *cu_seqlens, kda_tensor_t *out, kda_tensor_t *final_state,
                            const kda_options_t *opts, void *workspace, size_t workspace_bytes, void *stream)
{
    Problem P;
    kda_status_t st = validate(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, P);
    if (st) return st;
    Plan pl;
    if ((st = make_plan(P, opts, pl))) return st;
    return run(P, pl, opts, workspace, workspace_bytes, (hipStream_t)stream);
}

kda_status_t kda_prefill(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v, const kda_tensor_t *g,
                         const kda_tensor_t *beta, const kda_tensor_t *initial_state,
                         const kda_tensor_t *cu_seqlens, kda_tensor_t *out, kda_tensor_t *final_state, void *stream)
{
    Problem P;
    kda_status_t st = validate(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, P);
    if (st) return st;
    Plan pl;
    if ((st = make_plan(P, nullptr, pl))) return st;
    if (pl.bytes == 0) return run(P, pl, nullptr, nullptr, 0, (hipStream_t)stream);
    {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        std::lock_guard<std::mutex> lk(g_ws_mu);
        CachedWs *cp = nullptr;
        for (CachedWs &x : g_ws)
            if (x.dev == dev && x.stream == stream) cp = &x;
        if (!cp) {
            g_ws.push_back(CachedWs{dev, stream, nullptr, 0});
            cp = &g_ws.back();
        }
        CachedWs &c = *cp;
        if (c.bytes < pl.bytes) {
            if (c.p) {
                if ((e = hipStreamSynchronize((hipStream_t)stream)) != hipSuccess) return hip_fail(e, "workspace sync");
                e = hipFree(c.p);
                c.p = nullptr;
                c.bytes = 0;
                if (e != hipSuccess) return hip_fail(e, "workspace free");
            }
            if ((e = hipMalloc(&c.p, pl.bytes)) != hipSuccess) {
                c.p = nullptr;
                return fail(KDA_ERR_WORKSPACE, "hipMalloc(%zu): %s", pl.bytes, hipGetErrorString(e));
            }
            c.bytes = pl.bytes;
        }
        return run(P, pl, nullptr, c.p, pl.bytes, (hipStream_t)stream);
    }
}

kda_status_t kda_decode(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v, const kda_tensor_t *g,
                        const kda_tensor_t *beta, kda_tensor_t *state_pool, const kda_tensor_t *state_indices,
                        const kda_tensor_t *num_tokens, kda_tensor_t *out, int32_t update_state,
                        const kda_options_t *opts, void *stream)
{
    kda_status_t st;
    if ((st = check_basic(q, "q", false)) || (st = check_basic(k, "k", false)) || (st = check_basic(v, "v", false)) ||
        (st = check_basic(g, "g", false)) || (st = check_basic(beta, "beta", false)) ||
        (st = check_basic(state_pool, "state_pool", false)) || (st = check_basic(state_indices, "state_indices", false)) ||
        (st = check_basic(num_tokens, "num_tokens", true)) || (st = check_basic(out, "out", true)))
        return st;
    if (q->dtype != KDA_BF16 && q->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "q must be bf16 or fp32");
    if (k->dtype != q->dtype || v->dtype != q->dtype || (out && out->dtype != q->dtype))
        return fail(KDA_ERR_DTYPE, "q, k, v and out must share one dtype");
    if (g->dtype != KDA_F32 || beta->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "g and beta must be fp32");
    if (state_pool->dtype != KDA_F32 && state_pool->dtype != KDA_BF16)
        return fail(KDA_ERR_DTYPE, "state_pool must be fp32 or bf16");
    if (state_indices->dtype != KDA_I32 || (num_tokens && num_tokens->dtype != KDA_I32))
        return fail(KDA_ERR_DTYPE, "state_indices and num_tokens must be int32");
    if (q->ndim != 4) return fail(KDA_ERR_SHAPE, "q must be [R, T, H, K]");
    const int64_t R = q->shape[0], T = q->shape[1], H = q->shape[2], D = q->shape[3];
    if (D != 64 && D != 128) return fail(KDA_ERR_UNSUPPORTED, "head size %lld not in {64, 128}", (long long)D);
    if (T < 1 || T > kda::DECODE_MAX_TOKENS)
        return fail(KDA_ERR_UNSUPPORTED, "%lld tokens per request: decode takes 1..%d", (long long)T, kda::DECODE_MAX_TOKENS);
    if (H < 1) return fail(KDA_ERR_SHAPE, "H must be >= 1");
    auto same4 = [&](const kda_tensor_t *t, const char *name) -> kda_status_t {
        if (t->ndim != 4 || t->shape[0] != R || t->shape[1] != T || t->shape[2] != H || t->shape[3] != D)
            return fail(KDA_ERR_SHAPE, "%s must be [%lld, %lld, %lld, %lld]", name, (long long)R, (long long)T,
                        (long long)H, (long long)D);
        return KDA_OK;
    };
    if ((st = same4(k, "k")) || (st = same4(v, "v")) || (st = same4(g, "g")) || (out && (st = same4(out, "out"))))
        return st;
    if (beta->ndim != 3 || beta->shape[0] != R || beta->shape[1] != T || beta->shape[2] != H)
        return fail(KDA_ERR_SHAPE, "beta must be [R, T, H]");
    if (state_pool->ndim != 4 || state_pool->shape[1] != H || state_pool->shape[2] != D || state_pool->shape[3] != D)
        return fail(KDA_ERR_SHAPE, "state_pool must be [P, %lld, %lld, %lld]", (long long)H, (long long)D, (long long)D);
    const int64_t P = state_pool->shape[0];
    if (state_indices->ndim != 1 || state_indices->shape[0] != R) return fail(KDA_ERR_SHAPE, "state_indices must be [R]");
    if (num_tokens && (num_tokens->ndim != 1 || num_tokens->shape[0] != R))
        return fail(KDA_ERR_SHAPE, "num_tokens must be [R]");
    if (R * H * (D / 32) >= (int64_t)1 << 31 || P >= (int64_t)1 << 31)
        return fail(KDA_ERR_SHAPE, "too many requests or pool slots");
    const Span sp = span_of(state_pool), so = span_of(out);
    const kda_tensor_t *ins[] = {q, k, v, g, beta, state_indices, num_tokens};
    const char *names[] = {"q", "k", "v", "g", "beta", "state_indices", "num_tokens"};
    for (int i = 0; i < 7; ++i) {
        if (!ins[i]) continue;
        if (overlaps(sp, span_of(ins[i]))) return fail(KDA_ERR_ALIAS, "state_pool overlaps %s", names[i]);
        if (overlaps(so, span_of(ins[i]))) return fail(KDA_ERR_ALIAS, "out overlaps %s", names[i]);
    }
    if (overlaps(so, sp)) return fail(KDA_ERR_ALIAS, "out overlaps state_pool");
    // state rows and output rows move as 4-element vectors
    auto aligned4 = [&](const kda_tensor_t *t) {
        if (!t || !t->data) return true;
        const size_t es = elem_size(t->dtype), vec = 4 * es;
        if ((uintptr_t)t->data % vec) return false;
        for (int d = 0; d + 1 < t->ndim; ++d)
            if (t->shape[d] > 1 && (t->stride[d] * es) % vec) return false;
        return true;
    };
    if (!aligned4(state_pool) || !aligned4(out))
        return fail(KDA_ERR_LAYOUT, "state_pool and out need 4-element-aligned base addresses and strides");
    if (opts && (opts->gate_act < 0 || opts->gate_act > 1 || opts->beta_act < 0 || opts->beta_act > 1))
        return fail(KDA_ERR_UNSUPPORTED, "gate_act %d / beta_act %d (0 or 1)", opts->gate_act, opts->beta_act);
    if (opts && opts->gate_act && !(opts->gate_lower_bound >= -5.f && opts->gate_lower_bound <= 0.f))
        return fail(KDA_ERR_UNSUPPORTED, "gate_lower_bound %g outside [-5, 0]", (double)opts->gate_lower_bound);
    if ((st = check_out_norm(opts, out, D, state_pool, "state_pool"))) return st;
    if (R == 0 || (!out && !update_state)) return KDA_OK;

    kda::DecodeParams dp{};
    dp.q = q->data; dp.k = k->data; dp.v = v->data;
    dp.g = (const float *)g->data; dp.beta = (const float *)beta->data;
    dp.pool = state_pool->data;
    dp.idx = (const int32_t *)state_indices->data;
    dp.ntok = num_tokens ? (const int32_t *)num_tokens->data : nullptr;
    dp.o = out ? out->data : nullptr;
    dp.q_sr = q->stride[0]; dp.q_st = q->stride[1]; dp.q_sh = q->stride[2];
    dp.k_sr = k->stride[0]; dp.k_st = k->stride[1]; dp.k_sh = k->stride[2];
    dp.v_sr = v->stride[0]; dp.v_st = v->stride[1]; dp.v_sh = v->stride[2];
    dp.g_sr = g->stride[0]; dp.g_st = g->stride[1]; dp.g_sh = g->stride[2];
    dp.b_sr = beta->stride[0]; dp.b_st = beta->stride[1]; dp.b_sh = beta->stride[2];
    if (out) { dp.o_sr = out->stride[0]; dp.o_st = out->stride[1]; dp.o_sh = out->stride[2]; }
    dp.p_sn = state_pool->stride[0]; dp.p_sh = state_pool->stride[1]; dp.p_sr = state_pool->stride[2];
    dp.R = (int32_t)R; dp.T = (int32_t)T; dp.H = (int32_t)H; dp.P = (int32_t)P;
    dp.update = update_state ? 1 : 0;
    dp.gate_act = (opts && opts->gate_act) ? 1 : 0;
    dp.gate_lb = opts ? opts->gate_lower_bound : 0.f;
    dp.beta_act = (opts && opts->beta_act) ? 1 : 0;
    dp.stall_wave = (opts && opts->stall_wave > 0) ? opts->stall_wave - 1 : -1;
    dp.stall_iters = (opts && opts->stall_cycles > 0) ? std::max(1, opts->stall_cycles / 127) : 0;
    if (opts && opts->out_gate) {
        dp.z = opts->out_gate->data;
        dp.z_sr = opts->out_gate->stride[0]; dp.z_st = opts->out_gate->stride[1]; dp.z_sh = opts->out_gate->stride[2];
        dp.nw = (const float *)opts->norm_weight->data;
        dp.eps = opts->norm_eps;
    }
    const hipStream_t s = (hipStream_t)stream;
    if (env_on("KDA_CHECK")) {
        DeviceChecks dc;
        dc.check_g = true;
        dc.g = g_view(g, R * T, T, g->stride[0], g->stride[1], g->stride[2], H, D, opts && opts->gate_act);
        if (update_state) { dc.slots = dp.idx; dc.R = R; dc.P = P; }
        kda_status_t cs = run_device_checks(dc, s, nullptr);
        if (cs) return cs;
    }
    hipError_t e = timed("kda_decode", s, [&] {
        return kda::launch_decode(dp, (int)D, q->dtype == KDA_F32, state_pool->dtype == KDA_BF16, s);
    });
    return e == hipSuccess ? KDA_OK : hip_fail(e, "DECODE launch");
}

kda_status_t kda_prep(const kda_tensor_t *g, const kda_tensor_t *cu_seqlens, int32_t chunk, kda_tensor_t *gamma,
                      void *stream)
{
    kda_status_t st;
    if (chunk != 32 && chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk length %d not in {32, 64}", chunk);
    if ((st = check_basic(g, "g", false)) || (st = check_basic(gamma, "gamma", false)) ||
        (st = check_basic(cu_seqlens, "cu_seqlens", true)))
        return st;
    if (g->dtype != KDA_F32 || gamma->dtype != KDA_F32) return fail(KDA_ERR_DTYPE, "g and gamma must be fp32");
    if (g->ndim != gamma->ndim) return fail(KDA_ERR_SHAPE, "gamma must have g's shape");
    for (int d = 0; d < g->ndim; ++d)
        if (g->shape[d] != gamma->shape[d]) return fail(KDA_ERR_SHAPE, "gamma must have g's shape");
    if (overlaps(span_of(g), span_of(gamma))) return fail(KDA_ERR_ALIAS, "gamma overlaps g");
    Problem P;
    P.dense = cu_seqlens == nullptr;
    if (P.dense) {
        if (g->ndim != 4) return fail(KDA_ERR_SHAPE, "dense g must be [B, T, H, K]");
        P.B = g->shape[0]; P.T = g->shape[1]; P.N = P.B; P.H = g->shape[2]; P.D = g->shape[3];
        P.Ttot = P.B * P.T;
    } else {
        if (cu_seqlens->dtype != KDA_I32 || cu_seqlens->ndim != 1 || cu_seqlens->shape[0] < 1)
            return fail(KDA_ERR_SHAPE, "cu_seqlens must be int32 [N + 1]");
        P.N = cu_seqlens->shape[0] - 1;
        if (g->ndim == 4 && g->shape[0] == 1) { P.Ttot = g->shape[1]; P.H = g->shape[2]; P.D = g->shape[3]; }
        else if (g->ndim == 3) { P.Ttot = g->shape[0]; P.H = g->shape[1]; P.D = g->shape[2]; }
        else return fail(KDA_ERR_SHAPE, "packed g must be [T, H, K]");
    }
    if (P.D < 1 || P.D > 128) return fail(KDA_ERR_UNSUPPORTED, "PREP supports 1..128 channels");
    Tok tg, ty;
    if ((st = tok_view(g, "g", P, P.D, true, tg)) || (st = tok_view(gamma, "gamma", P, P.D, true, ty))) return st;
    kda::PrepParams pp{};
    pp.g = (const float *)g->data; pp.gamma = (float *)gamma->data;
    pp.cu = cu_seqlens ? (const int32_t *)cu_seqlens->data : nullptr;
    pp.g_sb = tg.sb; pp.g_st = tg.st; pp.g_sh = tg.sh;
    pp.y_sb = ty.sb; pp.y_st = ty.st; pp.y_sh = ty.sh;
    pp.N = (int32_t)P.N; pp.H = (int32_t)P.H; pp.T = (int32_t)P.T; pp.D = (int32_t)P.D;
    pp.chunk = chunk;
    pp.chunks_per_seq = P.dense ? (int32_t)((P.T + chunk - 1) / chunk) : 0;
    if (P.N == 0 || (P.dense && P.T == 0)) return KDA_OK;
    if (cu_seqlens && env_on("KDA_CHECK")) {
        DeviceChecks dc;
        dc.cu = pp.cu; dc.N = P.N; dc.Ttot = P.Ttot;
        kda_status_t s = run_device_checks(dc, (hipStream_t)stream, nullptr);
        if (s) return s;
    }
    const int64_t nvc = P.dense ? P.B * pp.chunks_per_seq : (P.Ttot + chunk - 1) / chunk + P.N;
    hipError_t e = timed("kda_prep", (hipStream_t)stream, [&] { return kda::launch_prep(pp, (int)nvc, (hipStream_t)stream); });
    return e == hipSuccess ? KDA_OK : hip_fail(e, "PREP launch");
}

void kda_release_cached_workspace(void)
{
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (CachedWs &c : g_ws) {
        if (!c.p) continue;
        (void)hipSetDevice(c.dev);
        (void)hipDeviceSynchronize();
        (void)hipFree(c.p);
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
}

void kda_profile_enable(int on)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
    // enough idle pairs for a few hundred launches between reads
    while (g_prof_on && g_prof_pool.size() + g_prof.size() < 512) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) break;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            break;
        }
        g_prof_pool.emplace_back(a, b);
    }
}

kda_status_t kda_profile_read(const char *kernel, double *total_ms, int64_t *launches)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    double tot = 0.0;
    int64_t cnt = 0;
    kda_status_t st = KDA_OK;
    for (auto &r : g_prof) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == KDA_OK) st = hip_fail(e, "profile event");
        if (!kernel || strstr(r.name, kernel)) {
            tot += ms;
            ++cnt;
        }
        g_prof_pool.emplace_back(r.a, r.b);
    }
    g_prof.clear();
    if (total_ms) *total_ms = tot;
    if (launches) *launches = cnt;
    return st;
}

kda_status_t kda_profile_read_kernels(kda_profile_entry_t *entries, int32_t max_entries, int32_t *count)
{
    if (!count || (max_entries > 0 && !entries)) return fail(KDA_ERR_NULL, "entries or count is NULL");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::vector<kda_profile_entry_t> agg;
    kda_status_t st = KDA_OK;
    for (auto &r : g_prof) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == KDA_OK) st = hip_fail(e, "profile event");
        kda_profile_entry_t *x = nullptr;
        for (auto &a : agg)
            if (strcmp(a.name, r.name) == 0) x = &a;
        if (!x) {
            agg.push_back(kda_profile_entry_t{});
            x = &agg.back();
            snprintf(x->name, sizeof(x->name), "%s", r.name);
        }
        x->launches += 1;
        x->total_ms += ms;
        g_prof_pool.emplace_back(r.a, r.b);
    }
    g_prof.clear();
    const int32_t n = (int32_t)std::min<size_t>(agg.size(), (size_t)std::max(0, max_entries));
    for (int32_t i = 0; i < n; ++i) entries[i] = agg[i];
    *count = n;
    return st;
}

const char *kda_status_string(kda_status_t s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_LAYOUT: return "KDA_ERR_LAYOUT";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_RANGE: return "KDA_ERR_RANGE";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_last_error.c_str(); }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
