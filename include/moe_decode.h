/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) decode-time MoE layer.
 *
 * One call of moe_decode_forward computes one Mixture-of-Experts layer for a
 * decode step of `batch` tokens on one GPU:
 *
 *   z      = x Wr^T (+ b)                                   router logits
 *   S, w   = top-k of z, softmax or sigmoid weights,         selection
 *            renormalised over the selected experts
 *   out    = [x] + S2 (silu(S1 x) * (S3 x))                  shared expert
 *              + sum_{j in S} w_j W2_j (silu(W1_j x) * (W3_j x))
 *
 * The pages this follows (the Kimi K3 decode article, spke.com/es and /ko
 * ai/article/3589, Part 1 sections 1 "shapes per workload", 3 "MoE
 * scheduling and overlap" and 4 "weight prefetch"; the Hungarian summary "A
 * vLLM ugynoki kodolassal gyorsitotta a Kimi K3-at", section "Kevesebb
 * kernel") name the parts of this layer -- router scores, routed experts
 * behind tensor parallelism, a shared expert on its own stream, small-matrix
 * kernels at batch 1-2 and split-K kernels above, and a weight stream that
 * bounds small-batch decode -- but give no formulas; the formulas above are
 * the plain gated-SwiGLU reading.
 *
 * Conventions for every function:
 *  - All tensor pointers are DEVICE pointers, 16-byte aligned, row-major,
 *    owned by the caller; the library never frees them.
 *  - Every function returns a moe_status; no C++ exception crosses the ABI.
 *    On failure moe_decode_last_error() returns a message for the calling
 *    thread (valid until that thread's next call into the library).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *  - A plan is not thread-safe; distinct plans are independent.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,      /* bad argument: NULL, out of range, misaligned, aliasing   */
    MOE_ERR_UNSUPPORTED = 2,  /* valid layer the kernels do not cover; use another path
                                 (the isolation rule of the Kimi K3 decode article,
                                 Part 2 section 1: the caller falls back to its own path) */
    MOE_ERR_HIP = 3,          /* a HIP runtime call failed; message holds hipGetErrorString */
    MOE_ERR_NOMEM = 4,        /* host or device allocation failed                          */
    MOE_ERR_STATE = 5         /* call not valid in the plan's current state                */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Kernel family for the gate/up projection (the Kimi K3 decode article, Part 1
 * section 1: small-matrix kernels at batch 1-2, split-K kernels at larger
 * batches, which spread one matrix product over more GPU workers).
 *  SMALL_M: every expert is a full-K GEMV tile (lanes stream weight rows,
 *           fp32 dot products); the form for batch 1-2.
 *  SPLIT_K: experts with at least `mfma_min_tokens` tokens use split-K MFMA
 *           tiles (fp32 partials, last-arriving tile applies SiLU*up), the
 *           others GEMV tiles; the form for larger batches.
 *  AUTO:    SMALL_M for batch <= 2, SPLIT_K otherwise, and SPLIT_K also where
 *           a GEMV tile's staged activations (2 * batch * hidden bytes) exceed
 *           its LDS budget (60 KiB).                                        */
typedef enum { MOE_VARIANT_AUTO = 0, MOE_VARIANT_SMALL_M = 1, MOE_VARIANT_SPLIT_K = 2 } moe_variant;

typedef struct moe_decode_config {
    int32_t hidden;          /* H: multiple of 64, 64..16384                          */
    int32_t n_experts;       /* E: routed experts, 1..1024                            */
    int32_t top_k;           /* k: 1..min(E, 16)                                      */
    int32_t inter;           /* I: routed-expert intermediate size, multiple of 64    */
    int32_t shared_inter;    /* Is: 0 (no shared expert) or a multiple of I           */
    int32_t batch;           /* B: tokens per forward, 1..64 (one plan per batch)     */
    int32_t score_fn;        /* moe_score_fn                                          */
    int32_t renormalize;     /* 1: selected weights divided by their sum              */
    float routed_scale;      /* multiplies every routed weight (1.0 = none)           */
    int32_t add_residual;    /* 1: out = x + ...; 0: out = layer output only          */
    const float* router_bias;/* device fp32 [E] added to the logits, or NULL          */
    int32_t force_variant;   /* moe_variant                                           */
    int32_t mfma_min_tokens; /* SPLIT_K: token count from which an expert uses MFMA
                                tiles; 0 = library default (3 at batch 5-16, else
                                5, or less where the GEMV tiles' activation
                                staging does not fit)                                */
    int32_t shared_stream;   /* (the Kimi K3 decode article, Part 1 section 3: the
                                shared expert on a stream of its own, overlapped
                                with routing)
                                0: the shared expert's gate/up runs in trailing
                                workgroups of the router launch (overlap without a
                                second queue); 1: on the plan's second stream,
                                forked before the router and joined before the down
                                projection                                           */
    int32_t topk_launch;     /* batch <= 4 only.  0: default (at batch 1-2 the
                                fused experts launch where it applies, see
                                single_launch; otherwise 3 where it applies, else
                                1); 1: top-k and bucketing in the router
                                launch's last workgroup to arrive; 2: in a launch of
                                their own after the router; 3: in every routed
                                gate/up workgroup, each deriving the same work lists
                                from the logits (no hand-off between workgroups),
                                with the shared expert's gate/up in the same launch.
                                3 runs every gate/up tile as a GEMV tile: with the
                                default mfma_min_tokens that is what it does; a
                                mfma_min_tokens <= batch keeps 0 at 1, and asking
                                for 3 with it fails with MOE_ERR_UNSUPPORTED        */
    int32_t single_launch;   /* 0 (default): the library's choice.  At batch 1-2,
                                where the shape has a fused experts kernel (H <=
                                8192, I a power of two from 128, batch * k * I <=
                                4096, Is a multiple of 128 up to 512) and the device
                                holds its grid (512 workgroups at the TP8 shard, two
                                per CU) resident at once, two launches: the router
                                (+ the shared expert's gate/up), then the routed
                                experts, shared down and combine in ONE launch
                                whose workgroups hand h over through per-(token,
                                expert) counters (the Kimi K3 decode article, Part
                                1 section 2: producer and consumer fused at small
                                batch); otherwise the staged launches.  1: the staged launches always.  2: the
                                whole layer as ONE persistent launch -- possible when
                                batch <= 4, shared_stream = 0, topk_launch != 2 and
                                the shape fits it (x and h staged in LDS), else
                                MOE_ERR_UNSUPPORTED at plan time.  On MI355X it
                                measured slower than the staged launches, so the
                                default does not pick it.
                                The single launch runs every stage -- router,
                                selection, bucketing, shared and routed experts,
                                combine -- as tasks that workgroups claim in
                                dependency order, handing results over through
                                device-scope counters; it assumes its workgroups
                                (at most what fits on the GPU at once) are all
                                resident, and each wait is bounded: a wait that
                                runs out sets an error flag instead of hanging.   */
} moe_decode_config;

typedef struct moe_decode_plan_s* moe_decode_plan_t;

typedef struct moe_decode_info {
    int32_t variant;          /* resolved moe_variant (never AUTO)                       */
    int32_t n_kernels;        /* kernel launches per forward                            */
    int32_t mfma_min_tokens;  /* resolved threshold (SPLIT_K), else 0                   */
    int32_t shared_mfma;      /* 1 if the shared expert runs on MFMA tiles              */
    int32_t shared_stream;    /* resolved shared_stream                                  */
    int32_t router_mfma;      /* 1: router is a split-K MFMA launch + a top-k launch     */
    int32_t single_launch;    /* 0: staged launches; 1: the layer runs as one persistent
                                 launch (single_launch = 2 in the config); 2: batch 1-2
                                 as router launch + one experts launch (before the
                                 first forward this assumes the device holds its
                                 grid; the first forward checks, else 0)           */
    int32_t layer_grid;       /* the persistent grid's workgroup count (0 until the
                                 first forward)                                         */
    int32_t topk_launch;      /* resolved top-k placement: 1, 2 or 3 (see the config),
                                 0 with the single launch                              */
    size_t workspace_bytes;   /* device workspace owned by the plan                     */
    int32_t shared_gateup_in; /* launch holding the shared expert's gate/up: 0 none (no
                                 shared expert), 1 the router launch, 2 the routed gate/up
                                 launch, 3 its own launch on the second stream, 4 the
                                 single launch                                          */
} moe_decode_info;

/* Per-step counters the kernels write on the device (read back for tests). */
typedef struct moe_decode_stats {
    int32_t n_unique;         /* |U|: distinct routed experts selected in the step      */
    int32_t gemv_tiles;       /* routed gate/up tiles on the GEMV path                  */
    int32_t mfma_tiles;       /* routed gate/up tiles on the split-K MFMA path          */
    int32_t error_flags;      /* 0 = no device-side error was detected; else bits: 1 an
                                 invalid expert id reached the bucketing, 2 a work-list
                                 entry was inconsistent, 4 a single-launch wait ran out */
} moe_decode_stats;

/* Validates `cfg` and builds a plan on the host.  Creates no device state, so
 * it works (and its errors can be tested) without a GPU.  router_bias is only
 * stored, not dereferenced.  *out_plan is set to NULL on failure.
 * Source: the Kimi K3 decode article, Part 1 section 1 (kernel shapes chosen
 * per workload: small-matrix kernels at batch 1-2, split-K above), which is
 * the choice the plan resolves (variant, mfma_min_tokens); and Part 2 section 1
 * (isolate the changes): a shape the kernels do not cover is refused here with
 * MOE_ERR_UNSUPPORTED, so the caller keeps its own path for it, and the choice
 * made is readable through moe_decode_plan_info. */
moe_status moe_decode_plan(const moe_decode_config* cfg, moe_decode_plan_t* out_plan);

/* Runs the layer asynchronously on `stream`.
 * Source: the Kimi K3 decode article, Part 1 sections 1 (small-matrix and
 * split-K kernels by batch), 3 (router scores, tensor-parallel experts, the
 * shared expert overlapped with routing) and 4 (small-batch decode is bound by
 * loading weights); the Hungarian summary, section "Kevesebb kernel" (fewer
 * kernels per layer); the article's "What's next" (per-step host work replayed
 * as a graph).  The formulas are those at the top of this file.
 *   x        bf16 [B][H]                     layer input (and residual)
 *   router_w bf16 [E][H]                     router weight, one row per expert
 *   expert_w bf16 [E][2I][H] then [E][H][I]  per expert: W13 (rows 0..I-1 gate
 *                                            W1, rows I..2I-1 up W3), then all
 *                                            experts' down projections W2
 *   shared_w bf16 [2Is][H] then [H][Is]      shared S13 (gate rows, up rows), S2;
 *                                            ignored (may be NULL) when Is == 0
 *   out      bf16 [B][H]                     result, round-to-nearest-even;
 *                                            must not overlap x
 * The first call on a device allocates the plan's workspace (zeroed with
 * hipMemsetAsync on `stream`, so make the first call outside any graph
 * capture), a second stream and events, and builds a HIP graph of the
 * launches; later calls replay it, updating kernel arguments when the
 * pointers change.  When `stream` is being captured the kernels are launched
 * directly (and so recorded into the caller's graph, with no memset).  Work
 * is enqueued on `stream` and the plan's private stream only; the call
 * returns once it is enqueued.  Calls on one plan must not overlap (they
 * share the workspace). */
moe_status moe_decode_forward(moe_decode_plan_t plan, const void* x, const void* router_w,
                              const void* expert_w, const void* shared_w, void* out,
                              void* stream);

/* moe_decode_forward, plus a cross-layer prefetch: while the layer selects its
 * experts (a phase that leaves HBM mostly idle) it reads the NEXT layer's
 * router weight (bf16 [E][H]) and shared expert weights (the shared_w layout)
 * with ordinary cached loads and drops them, so the next layer's router and
 * shared expert find them in the 256 MB Infinity Cache.  Source: the Kimi K3
 * decode article, Part 1 section 4 (prefetching future weights into the cache
 * from a phase that cannot use the memory bandwidth).  Either next pointer may
 * be NULL (nothing of it is prefetched); they are only read.  Issued by the
 * batch 1-2 experts launch (moe_decode_plan_info: single_launch = 2); the other
 * launch forms ignore the next-layer pointers.  Errors as moe_decode_forward,
 * plus MOE_ERR_INVALID for a misaligned next pointer. */
moe_status moe_decode_forward_prefetch(moe_decode_plan_t plan, const void* x, const void* router_w,
                                       const void* expert_w, const void* shared_w, void* out,
                                       const void* next_router_w, const void* next_shared_w,
                                       void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * layer as moe_decode_forward on the same kernels, launched directly on
 * `stream` (no graph, no second stream, no events), with every scratch buffer
 * (counters, logits, routing, work lists, h, split-K and down partials) in a
 * static device array of the library, one copy per GPU, at most 48 MiB; the
 * plan's own workspace is neither allocated nor used.  Calls no hipMalloc,
 * hipFree or other allocating routine.  Arguments, layout and ownership as for
 * moe_decode_forward.  Each call first clears what must start at zero and
 * writes the shared expert's work list in the array (one small extra launch).
 * Errors: MOE_ERR_UNSUPPORTED when the plan's workspace exceeds the array
 * (moe_decode_plan_info reports workspace_bytes), or when the plan asks for
 * the single launch (single_launch = 2) or a second stream (shared_stream =
 * 1); MOE_ERR_INVALID as for moe_decode_forward.  Every call on a GPU, from
 * any plan, shares that GPU's array and it keeps the last call's contents:
 * calls that overlap on one GPU (concurrent streams, threads) race and must
 * not be issued; moe_decode_routing and moe_decode_read_stats after this call
 * read the array, so no other call may run on that GPU between them. */
moe_status moe_decode_forward_noalloc(moe_decode_plan_t plan, const void* x, const void* router_w,
                                      const void* expert_w, const void* shared_w, void* out,
                                      void* stream);

/* Source: the Kimi K3 decode article, Part 2 section 1 (a reviewer can trace
 * what the optimised path selected) and Part 2 section 4 (expert selection
 * decides which weights a step reads, so measurements report it).
 * Enqueues on `stream` device-to-device copies of the last forward's routing:
 * topk_idx int32 [B][k] (expert ids, descending logit, ties to the lower id),
 * topk_w fp32 [B][k] (routing weights in the same order), n_unique int32 [1],
 * logits fp32 [B][E] (router logits including the bias).  Any destination may
 * be NULL.  MOE_ERR_STATE before the first forward. */
moe_status moe_decode_routing(moe_decode_plan_t plan, int32_t* topk_idx, float* topk_w,
                              int32_t* n_unique, float* logits, void* stream);

/* Source: the Kimi K3 decode article, Part 2 sections 1 (traceable selection)
 * and 3 (tests must show that the changed path ran: the tile counters say
 * which gate/up form each expert took).
 * Waits for the stream of the plan's last forward (and the plan's second
 * stream) to finish, then copies the device-side counters of that forward to
 * *stats (host memory).  It synchronises nothing else.  MOE_ERR_STATE before
 * the first forward. */
moe_status moe_decode_read_stats(moe_decode_plan_t plan, moe_decode_stats* stats);

/* Resolved plan properties (host memory): which launch form, kernel count and
 * gate/up variant the plan runs.  Source: the Kimi K3 decode article, Part 2
 * section 1 (it must be traceable when the optimised path is selected and how
 * execution falls back; here the fallback is MOE_ERR_UNSUPPORTED at plan time). */
moe_status moe_decode_plan_info(moe_decode_plan_t plan, moe_decode_info* info);

/* Kernel timing.  Source: the Kimi K3 decode article, Part 2 section 4
 * (verify performance broadly, with reproducible results).
 * While enabled, forward launches eagerly (no graph) and
 * records a HIP event pair around every kernel on the stream that kernel is
 * launched on.  moe_decode_profile_read synchronises those streams and writes,
 * per kernel slot, the summed milliseconds and the launch count over all
 * forwards since profiling was enabled (arrays of `cap` entries, host memory),
 * the slot names into `names` (may be NULL), and the slot count to *n.
 * At most 1024 forwards are recorded per enable. */
moe_status moe_decode_set_profiling(moe_decode_plan_t plan, int32_t enable);
moe_status moe_decode_profile_read(moe_decode_plan_t plan, int32_t cap, double* total_ms,
                                   int32_t* launches, const char** names, int32_t* n);

/* Frees the plan and everything it owns (waits for the device).  NULL is a
 * no-op.  (Plumbing: no passage of the pages defines it.) */
moe_status moe_decode_destroy(moe_decode_plan_t plan);

/* Message for the calling thread's last failed call ("" if none).  Source: the
 * Kimi K3 decode article, Part 2 section 1 (a fallback to the standard path
 * must be traceable: the message says why a shape was refused). */
const char* moe_decode_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
