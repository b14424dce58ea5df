/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention chunked prefill.
 *
 * The operation (the reading of the pages, which name the method but never
 * print its equations; see the TensorRT-LLM KDA prefill fix PR #19826 and the
 * cudnn-frontend Hopper KDA prefill PR #1056): for every sequence n and head h
 * independently, over the sequence's tokens t in order,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * S is a d_k x d_v fp32 matrix (row = key channel, column = value channel),
 * S_{-1} = initial_state (zeros when NULL) and final_state = S after the last
 * token.  g is the per-token, per-channel natural-log decay; the kernels are
 * guaranteed on g in [-5, 0] (the production gate_lower_bound of the
 * cudnn-frontend PR's correctness section).  That range is a precondition the
 * host cannot see (g is device memory): values below -5 can overflow the
 * in-chunk gate factorisation to inf/NaN without any error being returned,
 * unless KDA_CHECK=1 (below) checks them first.  beta is the value in (0, 1)
 * (no sigmoid is applied).  No scale is applied to q.  The kernels compute the
 * chunked WY/UT form of this recurrence (TensorRT-LLM PR #19960 names the
 * WY-form chunk): the production kernel (head size 128, bf16) takes 32-token
 * chunks, the others (head size 64, the fp32 debug mode, variant 1) 64-token
 * chunks (the v64 of the cudnn-frontend kernel name); results do not depend on
 * the chunk length beyond rounding.
 *
 * Tensors (all pointers are DEVICE memory owned by the caller; the library
 * never frees or retains them):
 *   dense  (cu_seqlens == NULL): q, k, g [B, T, H, K]; v, out [B, T, H, V];
 *                                beta [B, T, H]; states [B, H, K, V]
 *   packed (cu_seqlens != NULL): q, k, g [T_tot, H, K] (or 4-D with B == 1);
 *                                v, out [T_tot, H, V]; beta [T_tot, H];
 *                                cu_seqlens int32 [N + 1] with cu[0] = 0,
 *                                non-decreasing, cu[N] = T_tot (device memory,
 *                                NOT checked on the host); states [N, H, K, V]
 *   K == V, K in {64, 128}; H >= 1; T >= 0; zero-length sequences allowed
 *   (no output rows; final_state == initial_state bit for bit).
 * Dtypes: q, k, v, out all KDA_BF16, or all KDA_F32 (the fp32 debug mode,
 *   K == 64 only); g, beta KDA_F32; initial_state and final_state each KDA_F32
 *   or KDA_BF16 (a bf16 state pool: widened to fp32 on load, the arithmetic in
 *   fp32, the final state rounded to nearest even).
 * Strides are in ELEMENTS; every tensor needs a unit last-dimension stride and
 *   all other strides are honoured (row-padded views give the same bits as
 *   contiguous tensors).
 * Aliasing: out may not overlap any input; final_state may be exactly
 *   initial_state (in-place update) but may not partially overlap it.
 *
 * Errors: every check runs on the host before anything is enqueued.  On any
 * error nothing is launched, outputs are untouched and kda_last_error() holds
 * a thread-local message.  KDA_ERR_HIP reports a HIP runtime failure (the
 * message carries hipGetErrorString).
 *
 * Asynchrony: calls enqueue on `stream` (a hipStream_t; NULL is the null
 * stream) and return without synchronising or reading device data back.
 *
 * Environment (read on every call):
 *   KDA_CHECK=1  checks the device-side preconditions before anything else is enqueued
 *                (a few small kernels, a synchronisation of `stream` and a 12-byte read
 *                back; the first such call on a device allocates a 256-byte flag buffer):
 *                  - cu_seqlens: cu[0] == 0, non-decreasing, cu[N] == T_tot, else
 *                    KDA_ERR_SHAPE (without the check a last offset past the token extent
 *                    makes the kernels read past the inputs);
 *                  - every element of g in [-5, 0] (with gate_act: not NaN), else
 *                    KDA_ERR_RANGE (kda_prefill, kda_prefill_ws, kda_decode);
 *                  - kda_decode with update_state: no two requests name the same slot in
 *                    [0, P), else KDA_ERR_ALIAS (O(R^2) comparisons on the device).
 *                Nothing further is launched on a failed check.
 *   KDA_LOG=1    prints every plan (layout, chains, segments, kernel, chain order,
 *                workspace) to stderr.
 *   KDA_ORDER    chain order of a packed single-segment launch.  By default, when there
 *                are more (sequence, head) chains than compute units and at most 512
 *                sequences, the kernel starts the longest sequences' chains first (it
 *                ranks the lengths on the device); results are the same bits in any
 *                order.  KDA_ORDER=natural keeps launch order, KDA_ORDER=longest ranks
 *                whenever the plan allows it.
 *   KDA_CAP      chains allowed to run at once in a packed single-segment launch whose
 *                chains all fit the compute units (default 160; 0 turns it off).  With
 *                more chains than that (at most 128 sequences), the
 *                kernel packs the sequences longest first into groups of H workgroups (the
 *                fewest groups, from cap / H up, with which the longest sequence still
 *                bounds the packing; none: uncapped), and a workgroup whose
 *                sequence follows another in its group waits (bounded) for that
 *                sequence's chain of the same head before its main loop: mixed-length
 *                batches finish sooner, results are the same bits.  The plan then needs 8
 *                bytes of workspace per chain, last in the workspace; a workspace without
 *                them runs the launch uncapped.  The flags tell calls and replays of one
 *                captured call apart, so calls captured in HIP graphs stay capped on
 *                every replay.
 *   KDA_CAP_WAIT_US  bound of each such wait in microseconds (test knob; default: 8 us
 *                per chunk of the awaited sequence plus 2 ms).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer or descriptor is NULL            */
    KDA_ERR_SHAPE = 2,       /* rank / extent mismatch or unsupported head size     */
    KDA_ERR_DTYPE = 3,       /* dtype not allowed for that argument                 */
    KDA_ERR_LAYOUT = 4,      /* last-dimension stride != 1 or negative stride       */
    KDA_ERR_ALIAS = 5,       /* forbidden overlap between outputs and inputs        */
    KDA_ERR_UNSUPPORTED = 6, /* valid request this library does not implement       */
    KDA_ERR_WORKSPACE = 7,   /* workspace too small or allocation failed            */
    KDA_ERR_HIP = 8,         /* HIP runtime error while enqueueing                  */
    KDA_ERR_RANGE = 9        /* an input value outside its documented range         */
                             /* (found by the KDA_CHECK=1 device checks)            */
} kda_status_t;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1, KDA_I32 = 2 } kda_dtype_t;

/* A strided view of device memory.  shape/stride entries past ndim are ignored;
 * strides count elements, not bytes. */
typedef struct {
    void *data;
    int32_t dtype; /* kda_dtype_t */
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} kda_tensor_t;

/* Planner and test knobs.  A zero-filled struct (or NULL) means automatic. */
typedef struct {
    int32_t nseg;          /* segments per (sequence, head) chain; 0 = planner's choice, 1..64 forces */
    int32_t prep;          /* 0 or 2 = in-chunk (fused) gate scan; 1 = standalone PREP kernel first     */
    int32_t stall_wave;    /* test hook: -1/0 = none; w+1 stalls wave w at every LDS hand-off        */
    int32_t stall_cycles;  /* length of each injected stall, in s_sleep units of 64 cycles           */
    int32_t variant;       /* 0 = planner; 1 = single-role 64-token chunk kernel; 2 = pipelined      */
                           /* 32-token chunk kernel (head size 128, bf16 only)                       */
    /* Activations fused into the gate scan (the production gate lower bound of the
     * cudnn-frontend PR's correctness section, and the beta-sigmoid path of the
     * TensorRT-LLM KDA prefill fix PR #19826):
     *   gate_act = 1: g holds logits x and the log decay is gate_lower_bound * sigmoid(x),
     *                 gate_lower_bound in [-5, 0] (the range the kernels are guaranteed on);
     *   beta_act = 1: beta holds logits b and the delta strength is sigmoid(b).
     * 0 (the default) takes g and beta as the values of the recurrence. */
    int32_t gate_act;
    float gate_lower_bound;
    int32_t beta_act;
    /* Output epilogue: the gated RMS normalisation of every (token, head) output row
     * (the fused output norm of TensorRT-LLM PR #19960), applied before out is written:
     *     out_c = o_c / sqrt(mean_c(o_c^2) + norm_eps) * norm_weight[c] * sigmoid(out_gate_c)
     * over the value channels c.  out_gate: out's shape, layout and dtype (4-element
     * aligned rows); norm_weight: fp32 [V], contiguous; norm_eps > 0.  NULL out_gate (the
     * default) writes o itself.  Prefill supports it on the pipelined kernel (head size
     * 128, bf16); kda_decode supports every shape it takes. */
    const kda_tensor_t *out_gate;
    const kda_tensor_t *norm_weight;
    float norm_eps;
    /* split_chains = n > 0 (with a forced nseg > 1): only the last n (sequence, head) chains
     * are cut into segments and the others run whole, their segment outputs and the whole
     * chains in one launch (pipelined kernel only; a test knob -- the planner picks such split
     * plans itself for dense batches with a little more than a multiple of the CU count of
     * chains).  0 = planner's choice. */
    int32_t split_chains;
} kda_options_t;

/*
 * kda_prefill -- the KDA chunked prefill with a library-cached workspace.
 * q, k, v, g, beta: inputs as above.  initial_state: NULL for zeros.
 * cu_seqlens: NULL for the dense layout.  out: written for every valid token.
 * final_state: NULL to skip.  stream: hipStream_t.
 * Uses (and grows on demand) a workspace cached by the library per (device,
 * stream), so calls on different streams never share it; the first call for a
 * new size may call hipMalloc (after synchronising that stream when it replaces
 * a smaller buffer), so this entry point is not meant for graph capture -- use
 * kda_prefill_ws there.  Calls from several host threads are safe: the cache
 * stays locked until a call has enqueued its kernels.  The workspace is sized
 * exactly for the plan (segment maps and start states only when chains are cut
 * into segments, nothing for a single-segment plan): the workspace review of the
 * cudnn-frontend PR #1056 found that kernel's per-shape cache sized by N*H*nseg
 * and kept for the process, hundreds of MB at N = 64, H = 32 that its
 * single-segment path never touched.
 */
kda_status_t kda_prefill(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                         const kda_tensor_t *g, const kda_tensor_t *beta,
                         const kda_tensor_t *initial_state, const kda_tensor_t *cu_seqlens,
                         kda_tensor_t *out, kda_tensor_t *final_state, void *stream);

/* Bytes of device workspace kda_prefill_ws needs for these descriptors and
 * options: 0 when the plan is a single chunk-kernel launch (8 bytes per chain when it
 * caps the chains running at once, see KDA_CAP); with nseg > 1 the
 * segment maps and segment start states (K x V each, 4 bytes an element: the
 * start states and the C maps fp32, the M maps fp32 or, on bf16 I/O, split into
 * two bf16 parts, in an internal order); with the standalone
 * PREP kernel the in-chunk gate sums (fp32, g's size).  Sized exactly for the
 * plan, never by N*H alone (the workspace review of the cudnn-frontend PR
 * #1056).  Validates everything kda_prefill_ws validates and launches nothing. */
kda_status_t kda_prefill_workspace_size(const kda_tensor_t *q, const kda_tensor_t *k,
                                        const kda_tensor_t *v, const kda_tensor_t *g,
                                        const kda_tensor_t *beta,
                                        const kda_tensor_t *initial_state,
                                        const kda_tensor_t *cu_seqlens, const kda_tensor_t *out,
                                        const kda_tensor_t *final_state,
                                        const kda_options_t *opts, size_t *bytes);

/* kda_prefill with options and a caller-owned device workspace of at least
 * kda_prefill_workspace_size() bytes (256-byte aligned; NULL with size 0 when
 * the plan needs none).  The workspace is scratch: its contents on entry do not
 * matter and are undefined on return; it may not overlap any tensor argument.
 * Allocates nothing and never synchronises (unless KDA_CHECK=1), so it can be
 * captured into a HIP graph.  A workspace smaller than needed, or misaligned,
 * returns KDA_ERR_WORKSPACE with nothing launched.  (The caller-owned buffer
 * answers the workspace review of the cudnn-frontend PR #1056: the library
 * keeps no per-shape buffers alive behind the caller's back.) */
kda_status_t kda_prefill_ws(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                            const kda_tensor_t *g, const kda_tensor_t *beta,
                            const kda_tensor_t *initial_state, const kda_tensor_t *cu_seqlens,
                            kda_tensor_t *out, kda_tensor_t *final_state,
                            const kda_options_t *opts, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * kda_prefill_noalloc -- kda_prefill_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and options without a workspace, and no allocation of any kind.  Its
 * scratch (segment maps, segment start states, standalone-PREP gate sums, the KDA_CHECK=1
 * flags) is a fixed device array of the library's, KDA_NOALLOC_SCRATCH_BYTES (64 MiB) plus
 * 256 bytes, of which every GPU the library runs on holds one copy until the process ends.
 * With an automatic segment count the planner lowers the count until the plan fits (a single
 * segment needs no scratch), so results may then differ from kda_prefill_ws's within the
 * segmented path's tolerance; a forced segment count or standalone PREP whose scratch does
 * not fit returns KDA_ERR_WORKSPACE with nothing launched.  Nothing in the scratch needs to
 * start at zero.  Every call on a GPU shares that GPU's array: two calls whose kernels may
 * overlap on one GPU (different streams, no ordering between them) race on it and must be
 * serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status_t kda_prefill_noalloc(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                                 const kda_tensor_t *g, const kda_tensor_t *beta,
                                 const kda_tensor_t *initial_state, const kda_tensor_t *cu_seqlens,
                                 kda_tensor_t *out, kda_tensor_t *final_state,
                                 const kda_options_t *opts, void *stream);

/*
 * kda_prep -- the standalone PREP kernel: the in-chunk inclusive cumulative sum
 * of g over `chunk`-token chunks (32 or 64) that restart at every sequence
 * start (the virtual chunk map, safe across sequence gaps, of the cudnn-frontend PR's
 * walkthrough: a chunk never straddles two sequences).  gamma has g's shape
 * and dtype (fp32), must not overlap g, and receives for token t of chunk
 * [t0, t0 + L):
 *     gamma[t] = (((g[t0] + g[t0+1]) + ...) + g[t])   (fp32 adds in token order),
 * the same bits the chunk kernels' fused scan produces.
 */
kda_status_t kda_prep(const kda_tensor_t *g, const kda_tensor_t *cu_seqlens, int32_t chunk,
                      kda_tensor_t *gamma, void *stream);

/*
 * kda_decode -- the recurrence token by token against a pool of states: decode
 * and multi-token (MTP) draft verification, and the replay-only commit of
 * accepted drafts (the KDA decode / verify path, state pools and replay of
 * TensorRT-LLM PR #19960).  For every request r and head h, with the slot
 * S = state_pool[state_indices[r], h] and n_r = num_tokens ? num_tokens[r] : T
 * (clamped to [0, T]), the same recurrence as kda_prefill runs over tokens
 * t = 0 .. n_r - 1 of the request:
 *     out[r, t, h] = S_t^T q_t              (when out != NULL; rows t >= n_r untouched)
 *     state_pool[state_indices[r], h] = S   (after the last token, when update_state != 0;
 *                                            otherwise the pool is only read: the verify pass)
 * q, k, g: [R, T, H, K]; v, out: [R, T, H, V]; beta: [R, T, H]; 1 <= T <= 8;
 * K == V in {64, 128}.  q, k, v, out: all bf16 or all fp32; g, beta: fp32.
 * state_pool: [P, H, K, V], fp32 or bf16 (a bf16 pool is widened to fp32 for
 * the arithmetic and rounded to nearest even when written back).
 * state_indices: int32 [R], device memory: a value outside [0, P) skips the
 * request (no output rows, no state write).  num_tokens: int32 [R], device
 * memory, or NULL.  Both are read on the device only.
 * opts: NULL, or a kda_options_t whose gate_act / gate_lower_bound / beta_act
 * take g and beta as logits exactly as in kda_prefill_ws, and whose stall_wave /
 * stall_cycles test hook stalls one of the kernel's 4 waves after every barrier
 * (the results must not change); nseg, prep and variant are ignored here.
 * Strides in elements with unit last stride, as for kda_prefill; state_pool and
 * out also need base addresses and strides aligned to 4 elements (their rows
 * move as 4-element vectors).  out may not overlap any input or the pool; the pool may not overlap any input.  Two
 * requests that name the same slot with update_state set race (the result is
 * one of the two); with update_state == 0 any indices may repeat.
 * Enqueues one kernel on `stream`; allocates nothing; never synchronises.
 */
kda_status_t kda_decode(const kda_tensor_t *q, const kda_tensor_t *k, const kda_tensor_t *v,
                        const kda_tensor_t *g, const kda_tensor_t *beta, kda_tensor_t *state_pool,
                        const kda_tensor_t *state_indices, const kda_tensor_t *num_tokens,
                        kda_tensor_t *out, int32_t update_state, const kda_options_t *opts,
                        void *stream);

/* Frees the workspaces cached by kda_prefill on every device and stream (synchronising
 * each device first), so that no scratch outlives the calls that need it (the workspace
 * review of the cudnn-frontend PR #1056 found a process-lifetime cache there).  Later
 * kda_prefill calls allocate again on demand. */
void kda_release_cached_workspace(void);

/* Kernel timing for measurement: when enabled, every kernel the library
 * enqueues is bracketed by hipEvents on its stream.  kda_profile_read()
 * synchronises those events and returns the summed milliseconds and launch
 * count of the kernels whose name contains `kernel` (e.g. "chunk"; NULL: all).
 * Every read clears all recorded launches, the ones it did not count included.
 * Enabling creates a pool of events on the current device (reused across
 * reads), so timed launches create none; call it with that device current. */
void kda_profile_enable(int on);
kda_status_t kda_profile_read(const char *kernel, double *total_ms, int64_t *launches);

/* The same records grouped by kernel name (one entry per name, in first-launch order):
 * synchronises the events, writes at most max_entries entries and their number to *count,
 * and clears every recorded launch.  Names: "kda_chunk" (single-segment pass),
 * "kda_chunk_segbuild" (segment maps), "kda_combine", "kda_chunk_segout" (segment outputs),
 * "kda_prep", "kda_decode". */
typedef struct {
    char name[32];
    int64_t launches;
    double total_ms;
} kda_profile_entry_t;
kda_status_t kda_profile_read_kernels(kda_profile_entry_t *entries, int32_t max_entries, int32_t *count);

const char *kda_status_string(kda_status_t status);
const char *kda_last_error(void);
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
