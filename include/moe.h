/*
 * moe.h — C ABI of a single-GPU Mixture-of-Experts layer for AMD Instinct
 * MI355X (gfx950): top-k routing, the dispatch schedule, dispatch, the
 * expert-grouped SwiGLU FFN, the router-weighted combine, and the backward.
 *
 * Sources (the pages that describe the method; cited by title and section):
 *   [AREX]  arex-research.com, "Cursor 放出 MoK：NVL72 训练提速 2.37 倍",
 *           section "pull 代替 push，ring buffer 踢掉 CPU：三个决定性的设计选择"
 *           (first decision: one schedule table serves dispatch, combine,
 *           reverse-combine and reverse-dispatch; second: a fixed-size ring
 *           buffer of tokens, the macrobatch, recycled per minibatch, so no
 *           token is dropped and no count goes back to the CPU; third: the
 *           minibatch size is a tunable; closing paragraph: BF16 and MXFP8
 *           modes, and the router-weight gradient fused into the SwiGLU
 *           backward).
 *   [AIGWX] aigwx.org, "Cursor 开源 MoK：面向 GB300 NVL72 的确定性 MoE 训练内核",
 *           section "详细发生了什么".
 *   [ALPHA] alphalab.site, "Mixture-of-Kittens" review: section 一 (what the
 *           layer fuses), section 二 (router projection outside the layer;
 *           the final router-weighted reduction; run-to-run bitwise
 *           determinism from a fixed accumulation order), section 三 (what
 *           the benchmark times; MXFP8 weights quantised outside timing),
 *           section 四 (synthetic Gaussian logits with top-k; tunables).
 *
 * Conventions
 *   - Token t has k slots s = t*k + j, j = 0..k-1, in the order the router
 *     picked them (descending logit, ties to the lower expert index).
 *   - Tokens are processed in macrobatches of `macrobatch` tokens.  The rows
 *     of macrobatch m are the global rows [m*M*k, (m+1)*M*k); inside a
 *     macrobatch they are grouped by expert (expert 0 first) and, within an
 *     expert, ordered by ascending slot id.
 *   - bf16 tensors are passed as pointers to 16-bit bf16 bit patterns.
 *     Weights use the [out, in] row-major convention: W_gate, W_up [E, I, H],
 *     W_down [E, H, I]; activations are row-major [tokens, H].
 *   - Every device pointer must be 16-byte aligned.  The caller owns every
 *     buffer; the library never allocates, frees, copies to the host or
 *     synchronises, and keeps no state between calls (reentrant).
 *   - Every call validates its arguments on the host first and returns a
 *     nonzero moe_status before anything is enqueued if they are wrong.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously.
 *   - Results are bit-identical across runs for the same inputs and config:
 *     no floating-point atomics; every sum has a fixed order.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,        /* bad shape, null or misaligned pointer, bad enum */
    MOE_ERR_UNSUPPORTED_DEVICE = 2, /* current device is not gfx950 (or no device)     */
    MOE_ERR_CAPACITY = 3,           /* ring capacity below one macrobatch's rows        */
    MOE_ERR_WORKSPACE = 4,          /* workspace null or smaller than required          */
    MOE_ERR_HIP = 5,                /* a HIP launch or query failed                     */
    MOE_ERR_UNSUPPORTED = 6         /* a valid request this build does not implement    */
} moe_status;

typedef enum moe_precision {
    MOE_PREC_BF16 = 0,   /* bf16 operands, fp32 accumulation                             */
    MOE_PREC_MXFP8 = 1,  /* E4M3 operands with E8M0 scales per 32 elements along K       */
    MOE_PREC_MXFP4 = 2   /* forward only: weights E2M1 with E8M0 scales per 32 along K,  */
                         /* activations (x, h) MXFP8; moe_backward returns               */
                         /* MOE_ERR_UNSUPPORTED                                          */
} moe_precision;

/* Layer shape and the tunables of [AREX] (third decision) / [ALPHA] 四, minus
 * the communication ones (there is no cross-GPU traffic on one GPU). */
typedef struct moe_config {
    int32_t T;             /* tokens, >= 1 (an empty batch is rejected: no call needed) */
    int32_t H;             /* hidden size, multiple of 128                            */
    int32_t I;             /* expert intermediate size, multiple of 128               */
    int32_t E;             /* routed experts, 1..1024                                 */
    int32_t k;             /* experts per token, 1..min(E, 32)                        */
    int32_t n_shared;      /* always-on shared experts: 0 or 1                        */
    int32_t macrobatch;    /* tokens per macrobatch (ring refill unit); 0 = T         */
    int32_t minibatch;     /* tokens per minibatch (fill granularity); 0 = macrobatch */
    int64_t capacity_rows; /* ring-buffer rows; 0 = the minimum (see moe_ring_rows)   */
    int32_t precision;     /* moe_precision                                           */
    int32_t flags;         /* MOE_FLAG_* bits; 0 = none                               */
    int32_t acc_experts;   /* several macrobatches: routed experts whose weight       */
                           /* gradients may take rows from more than one macrobatch  */
                           /* (the workspace keeps fp32 running sums for that many); */
                           /* 0 = E.  Exceeding it sets MOE_DEVERR_ACC_CAPACITY.     */
} moe_config;

/* moe_config.flags.
 * MOE_FLAG_RECOMPUTE: nothing but the schedule is saved for the backward
 *   (moe_saved is neither read nor written and may be NULL).  The backward
 *   walks macrobatches in reverse ([AREX] second decision: the reverse walk
 *   keeps the recomputation of forward activations small): the last
 *   macrobatch's gate and up projections are still in the workspace, where
 *   the forward left them, and every earlier macrobatch's are recomputed from
 *   x before its SwiGLU backward.  So moe_backward must be given the
 *   workspace of the moe_forward of the same batch, unchanged in between.
 *   Costs one gate/up GEMM per macrobatch but the last; saves the 4*S*I bytes
 *   (bf16) or 8*S*I bytes (MXFP8) of moe_saved, S = T*k (plus T*I*4 or T*I*8
 *   for a shared expert), for 4*M*k*I (or 8*M*k*I) bytes of workspace. */
#define MOE_FLAG_RECOMPUTE 1

/* The schedule table ([AREX] first decision): written by moe_schedule, read by
 * moe_forward and moe_backward.  n_macro = T / macrobatch,
 * n_mini = macrobatch / minibatch, S = T * k. */
typedef struct moe_sched {
    int32_t* topk_idx;     /* [T, k]  chosen experts                                  */
    float*   topk_w;       /* [T, k]  softmax of the chosen logits (fp32)             */
    int32_t* counts;       /* [n_macro, E]  rows per expert                           */
    int32_t* offsets;      /* [n_macro, E+1] exclusive scan of counts (local rows)    */
    int32_t* mini_counts;  /* [n_macro, E, n_mini] rows per expert per minibatch      */
    int32_t* row_of_slot;  /* [S]  global row of slot s                               */
    int32_t* slot_of_row;  /* [S]  inverse permutation                                */
} moe_sched;

/* MXFP8 weights (written by moe_quantize_weights_mxfp8): E4M3 codes (one
 * byte each) and E8M0 scales (one byte per 32 codes along the listed axis).
 * The forward reads the first three pairs; the backward's input gradients
 * read the transposed copies ([ALPHA] 三: weights are quantised outside the
 * timed region, so both orientations are prepared ahead of time).
 * Codes are row-major [rows, K].  Scales are K-step-major per matrix: for a
 * matrix of R rows and K columns they form [K/128, R, 4] bytes, the scale of
 * row r, block b (codes 32b..32b+31 of that row) at byte
 * ((b / 4) * R + r) * 4 + b % 4, so the scales of one 128-code step of
 * consecutive rows are contiguous.  Sizes below are in bytes per matrix. */
typedef struct moe_weights_mx {
    const void* w_gate_q;  const void* w_gate_s;   /* [E, I, H], [E, H/128, I, 4]  blocks along H */
    const void* w_up_q;    const void* w_up_s;     /* [E, I, H], [E, H/128, I, 4]                 */
    const void* w_down_q;  const void* w_down_s;   /* [E, H, I], [E, I/128, H, 4]  blocks along I */
    const void* w_gate_tq; const void* w_gate_ts;  /* [E, H, I], [E, I/128, H, 4]  W_gate^T, along I */
    const void* w_up_tq;   const void* w_up_ts;    /* [E, H, I], [E, I/128, H, 4]  W_up^T           */
    const void* w_down_tq; const void* w_down_ts;  /* [E, I, H], [E, H/128, I, 4]  W_down^T, along H */
    /* the shared expert (if n_shared): the same twelve arrays without the E axis */
    const void* s_gate_q;  const void* s_gate_s;
    const void* s_up_q;    const void* s_up_s;
    const void* s_down_q;  const void* s_down_s;
    const void* s_gate_tq; const void* s_gate_ts;
    const void* s_up_tq;   const void* s_up_ts;
    const void* s_down_tq; const void* s_down_ts;
} moe_weights_mx;

/* MXFP4 forward weights (written by moe_quantize_weights_mxfp4): E2M1 codes,
 * two per byte (element 2q in the low nibble of byte q), row-major
 * [rows, K/2] bytes, and E8M0 scales per 32 codes along K in the K-step-major
 * layout of moe_weights_mx ([K/128, rows, 4] bytes per matrix). */
typedef struct moe_weights_mx4 {
    const void* w_gate_q;  const void* w_gate_s;   /* [E, I, H/2], [E, H/128, I, 4] */
    const void* w_up_q;    const void* w_up_s;     /* [E, I, H/2], [E, H/128, I, 4] */
    const void* w_down_q;  const void* w_down_s;   /* [E, H, I/2], [E, I/128, H, 4] */
    const void* s_gate_q;  const void* s_gate_s;   /* the shared expert (if n_shared)  */
    const void* s_up_q;    const void* s_up_s;
    const void* s_down_q;  const void* s_down_s;
} moe_weights_mx4;

/* Weights.  bf16 arrays are always given (the MXFP8 backward writes bf16
 * gradients of them and the quantiser reads them); `mx` is required when
 * cfg->precision is MOE_PREC_MXFP8 and ignored otherwise.  The shared
 * expert's pointers are read only if n_shared. */
typedef struct moe_weights {
    const void* w_gate;    /* [E, I, H] */
    const void* w_up;      /* [E, I, H] */
    const void* w_down;    /* [E, H, I] */
    const void* s_gate;    /* [I, H]    */
    const void* s_up;      /* [I, H]    */
    const void* s_down;    /* [H, I]    */
    const moe_weights_mx* mx;
    const moe_weights_mx4* mx4;  /* required when cfg->precision is MOE_PREC_MXFP4 */
} moe_weights;

/* What the forward keeps for the backward, rows in schedule row order:
 * bf16 in BF16 mode; fp32 in MXFP8 mode, so that the backward quantises h,
 * dg and du from the same unrounded values the forward had. */
typedef struct moe_saved {
    void* g;               /* [S, I]  gate pre-activations                            */
    void* u;               /* [S, I]  up projections                                  */
    void* sg;              /* [T, I]  shared expert gate (if n_shared)                */
    void* su;              /* [T, I]  shared expert up   (if n_shared)                */
} moe_saved;

/* Parameter gradients (bf16, same layouts as the weights; overwritten). */
typedef struct moe_grads {
    void* d_w_gate;        /* [E, I, H] */
    void* d_w_up;          /* [E, I, H] */
    void* d_w_down;        /* [E, H, I] */
    void* d_s_gate;        /* [I, H]    (if n_shared) */
    void* d_s_up;          /* [I, H]    (if n_shared) */
    void* d_s_down;        /* [H, I]    (if n_shared) */
} moe_grads;

/* Human-readable name of a status code (static string, never NULL). */
MOE_API const char* moe_status_string(moe_status s);

/* Host-only: checks a config ([ALPHA] 四 tunables; T divisible by macrobatch,
 * macrobatch by minibatch; capacity).  Touches no device. */
MOE_API moe_status moe_validate_config(const moe_config* cfg);

/* Host-only: rows of the ring buffer that carries dispatched rows of one
 * macrobatch while the next is being filled ([AREX] second decision):
 * capacity_rows if set, else macrobatch*k when there is one macrobatch and
 * 2*macrobatch*k otherwise. */
MOE_API moe_status moe_ring_rows(const moe_config* cfg, int64_t* rows);

/* Host-only: bytes of device workspace that moe_schedule, moe_forward and
 * moe_backward need (one workspace serves all three; it holds the ring
 * buffer and per-call scratch, nothing that must survive between calls
 * except, under MOE_FLAG_RECOMPUTE, the forward's last macrobatch of gate
 * and up projections that the backward reads). */
MOE_API moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Host-only diagnostics: byte offset and size, inside the workspace of `cfg`,
 * of a named array the MXFP8 path keeps there (tests read them to compare
 * the activation quantisation bit for bit):
 *   "x_codes"  [T, H] E4M3 codes of x along H, written by moe_forward (the
 *              dispatch gathers routed rows from them, [ALPHA] 一: MXFP8
 *              activation quantisation inside the forward);
 *   "x_scales" [T, H/32] their E8M0 scales, row-major;
 *   "dy_codes", "dy_scales": the same of dy, written by moe_backward (the
 *              reverse-combine gathers them);
 *   "wgrad_x_codes", "wgrad_x_scales": the dW_gate / dW_up operand x of the
 *              last macrobatch moe_backward processed, quantised along the
 *              rows of each expert's group in 32-row blocks (the last one
 *              zero-padded to np_e = 32 * ceil(n_e / 32) rows) and stored
 *              group after group, transposed: group e's codes are [H, np_e]
 *              from byte 32 * B_e * H, its scales [H, np_e / 32] from byte
 *              B_e * H, where B_e = "wgrad_block_offsets"[e];
 *   "wgrad_block_offsets" int32 [E + 1]: B_e = sum over e' < e of np_e' / 32.
 * MOE_ERR_INVALID_ARG for other names or a BF16 config. */
MOE_API moe_status moe_workspace_region(const moe_config* cfg, const char* name, size_t* offset,
                                        size_t* bytes);

/* Host-only: 1 if the current HIP device is gfx950, else 0 (also 0 when no
 * device is visible).  The library refuses other devices, as the reference
 * layer refuses GPUs other than the one it was written for ([ALPHA] 四). */
MOE_API int moe_device_supported(void);

/* Routing and schedule ([ALPHA] 一 and 四: top-k over the router logits;
 * [AREX] first decision: one schedule table for all four data movements).
 *   logits [T, E] fp32 (finite), device.  Writes every array of *sched.
 * The router projection that produces the logits is outside the layer, as in
 * [ALPHA] 二. */
MOE_API moe_status moe_schedule(const moe_config* cfg, const float* logits, const moe_sched* sched,
                        void* workspace, size_t workspace_bytes, void* stream);

/* moe_schedule without a workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as moe_schedule minus the
 * workspace: its scratch (error word, per-block histograms and bases) lives in
 * a fixed 16 MiB device array inside the library, one per GPU, held until the
 * process ends.  Allocates nothing and makes no allocating call.
 *   Limit: 256 + 2 * align256(4 * E * nb) <= 16 MiB, nb = the schedule's
 *   512-slot blocks (ceil(minibatch * k / 512) per minibatch, summed over
 *   all minibatches); the 65,536-token, 512-expert, top-10 stream needs
 *   5.0 MiB.  Larger configs return MOE_ERR_WORKSPACE before anything is
 *   enqueued.
 *   Every call on a GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from different threads) race; serialise
 *   them.  The array keeps the last call's contents; what must start at zero
 *   is cleared by the call itself.  Its device error word is not reported
 *   (moe_check_device_error reads a workspace); routing of finite logits
 *   cannot produce an out-of-range entry. */
MOE_API moe_status moe_schedule_noalloc(const moe_config* cfg, const float* logits,
                                        const moe_sched* sched, void* stream);

/* The router projection upstream of the layer ([ALPHA] 二: it sits outside
 * the layer, which starts from the logits; provided so that the logit
 * gradient reaches the router weights and the tokens).
 *   x [T, H] bf16, w_router [E, H] bf16 (row e = expert e), logits [T, E]
 *   fp32 written: logits = x w_router^T, fp32 accumulation.  Needs no
 *   workspace. */
MOE_API moe_status moe_router_forward(const moe_config* cfg, const void* x, const void* w_router,
                                      float* logits, void* stream);

/* Backward of the router projection, after moe_backward produced d_logits:
 *   d_logits [T, E] fp32 (read; rounded once to bf16 as the GEMM operand);
 *   dx [T, H] bf16 read and written: dx += d_logits w_router (the stored dx
 *   and the fp32 product summed in fp32, rounded once), so that dx becomes
 *   the full input gradient of router + layer;
 *   dw_router [E, H] bf16 written: d_logits^T x, summed over the tokens in
 *   ascending order.
 * Uses the layer's workspace (a bf16 copy of d_logits); in recompute mode
 * it leaves the part that carries g, u from moe_forward to moe_backward
 * alone. */
MOE_API moe_status moe_router_backward(const moe_config* cfg, const void* x, const void* w_router,
                                       const float* d_logits, void* dx, void* dw_router,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Forward ([ALPHA] 一: dispatch, expert SwiGLU FFN, combine; 二: the
 * router-weighted reduction in a fixed order).
 *   x [T, H] bf16; y [T, H] bf16 (written);
 *   y_t = FFN_shared(x_t) + sum_{j=0..k-1} w[t,j] * o_(t,j), accumulated in
 *   fp32 in that order and rounded to bf16 once.
 *   saved: g, u written for the backward.
 * Macrobatches are processed in order through the ring buffer; every
 * dynamic size stays on the device ([AREX] second decision). */
MOE_API moe_status moe_forward(const moe_config* cfg, const moe_sched* sched, const void* x,
                       const moe_weights* w, void* y, const moe_saved* saved,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Backward ([AREX] first decision: reverse-combine and reverse-dispatch reuse
 * the schedule; closing paragraph: the router-weight gradient is fused into
 * the SwiGLU backward; [ALPHA] 一: expert gradients).  Macrobatches are walked
 * in reverse order ([AREX] second decision).
 *   dy [T, H] bf16; dx [T, H] bf16 (written);
 *   grads: every weight gradient (overwritten, not accumulated);
 *   dw [T, k] fp32: gradient of the combine weights (written);
 *   d_logits [T, E] fp32: gradient of the logits through the top-k softmax,
 *   zero for experts a token did not choose (written; may be NULL). */
MOE_API moe_status moe_backward(const moe_config* cfg, const moe_sched* sched, const moe_saved* saved,
                        const void* x, const moe_weights* w, const void* dy, void* dx,
                        const moe_grads* grads, float* dw, float* d_logits,
                        void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 weight quantisation ([AREX] closing paragraph: weights are quantised
 * ahead of time; [ALPHA] 三: outside the timed region).  Reads w's bf16 arrays
 * and writes every array of *out (caller-allocated, sizes as listed in
 * moe_weights_mx), along the OCP MX v1.0 rule: per 32-element block, scale
 * 2^(floor(log2 max|v|) - 8) clamped to [2^-127, 2^127], elements rounded to
 * nearest-even E4M3 and saturated to +-448.  Enqueued on `stream`; needs no
 * workspace. */
MOE_API moe_status moe_quantize_weights_mxfp8(const moe_config* cfg, const moe_weights* w,
                                              const moe_weights_mx* out, void* stream);

/* MXFP4 weight quantisation for the MXFP4-weight forward ([AREX], section
 * "一个代码编辑器，怎么会去写 GPU 内核？", names the authors' earlier MXFP8 and
 * NVFP4 training kernels; MXFP4 is the OCP block format of the same E2M1
 * element, with E8M0 scales per 32): reads w's bf16 arrays and
 * writes every array of *out (caller-allocated, layouts as in
 * moe_weights_mx4), per 32-element block along K: scale 2^(floor(log2
 * max|v|) - 2) clamped to [2^-127, 2^127], elements rounded to nearest-even
 * E2M1 and saturated to +-6.  Enqueued on `stream`; needs no workspace. */
MOE_API moe_status moe_quantize_weights_mxfp4(const moe_config* cfg, const moe_weights* w,
                                              const moe_weights_mx4* out, void* stream);

/* Reads and clears the sticky device error word that kernels set when a
 * caller-built schedule holds an out-of-range expert, slot or row (those
 * entries are skipped, never dereferenced), or when more routed experts take
 * rows from several macrobatches than moe_config.acc_experts allows (the
 * weight gradients of the experts past it are left unwritten).  Synchronises
 * `stream`; meant for tests.  *flags = 0 when nothing was found, else an OR
 * of the bits below. */
#define MOE_DEVERR_BAD_EXPERT 1
#define MOE_DEVERR_BAD_SLOT 2
#define MOE_DEVERR_BAD_ROW 4
#define MOE_DEVERR_BAD_OFFSETS 8
#define MOE_DEVERR_ACC_CAPACITY 16
MOE_API moe_status moe_check_device_error(void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t* flags);

/* ------------------------------------------------------------------------
 * Kernel timing (diagnostics; not part of the layer).  While enabled, every
 * kernel launch made by the calls above is bracketed by two HIP events
 * recorded on the launch stream.  moe_profile_collect waits for the pending
 * events and adds each kernel's elapsed time to a per-name total;
 * moe_profile_query reads it.  Process-wide state guarded by a mutex; off by
 * default, and free of cost while off.  Names are the kernels' short names
 * (e.g. "gemm_gate_up").
 * ------------------------------------------------------------------------ */
MOE_API moe_status moe_profile_enable(int on);
MOE_API moe_status moe_profile_collect(void);
MOE_API moe_status moe_profile_query(const char* name, int64_t* launches, double* total_ms);
/* Writes up to `cap` bytes of a newline-separated list of the kernel names
 * seen so far into buf (NUL-terminated). */
MOE_API moe_status moe_profile_names(char* buf, size_t cap);
MOE_API moe_status moe_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
