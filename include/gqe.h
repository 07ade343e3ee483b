/*
 * gqe.h -- C ABI of libgqe.so: the forward pass of the Grouped Query Experts
 * (GQE) attention layer on AMD Instinct MI355X (gfx950), plus the dense-GQA
 * layer built from the same kernels.
 *
 * Sources (cited by title and section):
 *   [GQE-x] "Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention",
 *           gist.science explainer of arXiv 2606.20945, technical summary,
 *           "Architecture and routing" (grouped expert pool, conditional
 *           activation of k experts per group, dense K/V path, output built
 *           from hard concatenation, a renormalised weighted sum and an
 *           always-on shared head) and "Experimental results" (16 query heads,
 *           8 KV groups, k=1).
 *   [GQE-n] FrontiersMind GQE news article (animattoys.com), part 4: each
 *           expert owns its query projection; a lightweight router scores all
 *           experts of every group and keeps the top k, best first; every
 *           selected expert attends over its group's shared K/V; the hard-
 *           concatenated outputs, the weighted-average slot and the shared
 *           head are merged and then projected.
 *   [GQA-w] aiboss88.com wiki "What is Grouped-Query Attention", "Mechanism":
 *           query heads in groups share one K/V head.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller allocates every buffer, device memory for all
 *     tensors and for the workspace. The library allocates, frees and keeps
 *     nothing between calls.
 *   - Execution: all work is enqueued on `stream` (a hipStream_t; NULL means
 *     the null stream) and the call returns without waiting. Outputs are
 *     valid once the stream reaches that point. Calls keep no state and may
 *     run concurrently on different streams with different workspaces.
 *   - Layout: row-major and contiguous. Weights use the [out, in] convention
 *     (y = x W^T). Token n = b*T + t. Every pointer must be 16-byte aligned.
 *   - Types: with dtype GQE_BF16, x, the weights (except br), out and
 *     slots_out are bf16; with GQE_F32 they are fp32. Router logits, router
 *     offsets br and weights w are always fp32; idx and counts are int32.
 *     Matrix products accumulate in fp32; the softmax state is fp32.
 *   - Semantics fixed by the library: attention is causal (the diagonal is
 *     included), scale 1/sqrt(d_h), no positional encoding; every batch
 *     element is an independent sequence. Expert e = g*M + m owns rows
 *     e*d_h .. e*d_h+d_h-1 of Wq. Top-k orders the experts of a group by
 *     descending logit, ties to the lower index. Routing weights are the
 *     per-group softmax probabilities of the picks, renormalised over all
 *     G*k picks of the token (they sum to 1).
 *   - Slot order of the merged output (and of Wo's input dimension):
 *     [hard slots g-major, rank-minor (G*k*d_h) | weighted slot (d_h) |
 *     shared slot (d_h)], i.e. (G*k+2)*d_h columns.
 *   - Errors: negative status codes, never an exception or a print. Every
 *     argument is checked before any HIP call, so errors are reported
 *     without touching the device. A failed kernel launch returns
 *     GQE_ERR_HIP. Inputs are never modified.
 *   - Supported shapes: d_h in {32, 64}; D a positive multiple of 64;
 *     1 <= k <= M <= 64; G*M <= 256; 0 <= shared_kv_group < G; B, T >= 1;
 *     B*T*max(G*k, 1) < 2^31.
 */
#ifndef GQE_H
#define GQE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQE_OK = 0,
    GQE_ERR_NULL = -1,         /* a required pointer is NULL */
    GQE_ERR_SHAPE = -2,        /* an inconsistent or out-of-range size */
    GQE_ERR_UNSUPPORTED = -3,  /* a valid size the library does not handle (d_h, D, M, G*M) */
    GQE_ERR_WORKSPACE = -4,    /* ws_bytes smaller than the *_workspace_bytes figure */
    GQE_ERR_ALIGN = -5,        /* a pointer not aligned to 16 bytes */
    GQE_ERR_HIP = -6,          /* the HIP runtime reported an error at launch */
    GQE_ERR_SCRATCH = -7,      /* gqe_attn_fwd_noalloc: the shape's workspace exceeds
                                  GQE_NOALLOC_SCRATCH_BYTES */
    /* Not a status: widens the enum's value range to all of int32, so that
     * gqe_status_str may be handed any int (C++ leaves reading an enum value
     * outside its range undefined). */
    GQE_STATUS_RANGE_ = 0x7fffffff
} gqe_status;

typedef enum { GQE_BF16 = 0, GQE_F32 = 1 } gqe_dtype;

/* One GQE layer. B batch, T sequence length, D model width, G KV groups,
 * M query experts per group, k experts picked per group, d_h head width,
 * shared_kv_group the KV group the always-on shared head reads,
 * dtype a gqe_dtype. */
/* How the picked experts' outputs are merged before the output projection.
 * GQE_FULL is the layer; the others are the ablations the FrontiersMind GQE
 * article compares in part 6 (and the explainer's "Experimental results"):
 *   GQE_FULL             C = [hard slots | sum_s w_s O_s | shared]   (G*k+2 slots)
 *   GQE_WEIGHTED_CONCAT  C = [p_s O_s per hard slot | shared]        (G*k+1 slots)
 *                        p_s = the pick's per-group router probability, not
 *                        renormalised (what gqe_route then returns as w)
 *   GQE_HARD_CONCAT      C = [hard slots | shared]                   (G*k+1 slots)
 *   GQE_NO_SHARED        C = [hard slots | sum_s w_s O_s]            (G*k+1 slots)
 * Wo is [D, slots*d_h] with the variant's slot count. */
typedef enum {
    GQE_FULL = 0,
    GQE_WEIGHTED_CONCAT = 1,
    GQE_HARD_CONCAT = 2,
    GQE_NO_SHARED = 3
} gqe_variant;

typedef struct {
    int64_t B, T, D;
    int32_t G, M, k, d_h, shared_kv_group;
    int32_t dtype;
    int32_t variant;   /* gqe_variant; GQE_FULL for the layer itself */
} gqe_shape;

/* Bytes of device workspace gqe_route, gqe_attn_fwd_routed and gqe_attn_fwd
 * need for this shape (one figure covers all three). Returns 0 if the shape
 * is invalid or unsupported. */
size_t gqe_workspace_bytes(const gqe_shape* s);

/* Router only. [GQE-x] "Architecture and routing" (conditional activation);
 * [GQE-n] part 4 (score every expert of every group, keep the top k).
 *   x      [B*T, D]            input activations
 *   Wr     [G*M, D]            router weight
 *   br     [G*M] fp32 or NULL  per-expert logit offset
 *   idx    [B*T, G, k] int32   out: picked expert m of group g, rank r (best first)
 *   w      [B*T, G, k] fp32    out: renormalised routing weights (the picks' own
 *                              probabilities for GQE_WEIGHTED_CONCAT)
 *   logits [B*T, G*M] fp32     out (NULL to skip): x Wr^T + br
 *   counts [G*M] int32         out (NULL to skip): tokens routed to each expert
 *   ws, ws_bytes               workspace of at least gqe_workspace_bytes(s) */
gqe_status gqe_route(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                     int32_t* idx, float* w, float* logits, int32_t* counts,
                     void* ws, size_t ws_bytes, void* stream);

/* Everything after the router, with the routing given by the caller.
 * [GQE-x] "Architecture and routing" (dense K/V path; Q only for the picked
 * experts; hard concatenation; renormalised weighted sum; shared head);
 * [GQE-n] part 4 (each picked expert attends over its group's K/V; the three
 * parts are merged and projected).
 *   x       [B*T, D]
 *   Wq      [G*M*d_h, D]          query projection of every expert
 *   Wk, Wv  [G*d_h, D]            key and value projections of every group
 *   Wq_sh   [d_h, D]              query projection of the shared head
 *   Wo      [D, slots*d_h]        output projection over the merged slots (slots:
 *                                 G*k+2 for GQE_FULL, G*k+1 for the ablations)
 *   idx     [B*T, G, k] int32     picked experts, each in [0, M), distinct
 *                                 within a group; an entry outside [0, M), or
 *                                 repeating an earlier rank's expert in its
 *                                 group, is skipped and its hard slot holds
 *                                 unspecified values (no out-of-bounds access
 *                                 results)
 *   w       [B*T, G, k] fp32      weights of the weighted slot (GQE_WEIGHTED_CONCAT:
 *                                 the factors of the hard slots; GQE_HARD_CONCAT:
 *                                 unused)
 *   out     [B*T, D]              out: layer output
 *   slots_out [B*T, slots*d_h]    out (NULL to skip): the merged slots */
gqe_status gqe_attn_fwd_routed(const gqe_shape* s, const void* x, const void* Wq, const void* Wk,
                               const void* Wv, const void* Wq_sh, const void* Wo,
                               const int32_t* idx, const float* w, void* out, void* slots_out,
                               void* ws, size_t ws_bytes, void* stream);

/* The whole GQE layer: router, sparse Q, dense K/V, causal attention of the
 * picked experts and the shared head, merged slots, output projection.
 * [GQE-x] "Architecture and routing"; [GQE-n] part 4.
 *   Arguments as in gqe_route and gqe_attn_fwd_routed.
 *   idx_out, w_out [B*T, G, k]    out (NULL to skip): the routing used */
gqe_status gqe_attn_fwd(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                        const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                        const void* Wo, void* out, int32_t* idx_out, float* w_out,
                        void* ws, size_t ws_bytes, void* stream);

/* gqe_attn_fwd without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and kernels as gqe_attn_fwd,
 * minus ws / ws_bytes: the workspace is a static device array of
 * GQE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends. The call allocates and frees nothing.
 *   - Shapes whose gqe_workspace_bytes exceeds GQE_NOALLOC_SCRATCH_BYTES
 *     return GQE_ERR_SCRATCH before any HIP call (256 MiB holds the B1 T32768
 *     D1024 G8 M2 k1 layer's 150 MB and the B2 T16384 D2048 G8 M4 k2 layer's
 *     225 MB; the 1M-token layer needs the workspace form).
 *   - Every call on a device shares that device's array, and it keeps the
 *     last call's contents (the forward needs none of them cleared). Calls
 *     that overlap on one device, on any streams or threads, race on it:
 *     the caller must order them (one stream, or events between streams).
 *   - Errors as for gqe_attn_fwd, plus GQE_ERR_SCRATCH; GQE_ERR_HIP also if
 *     the array's device address cannot be looked up. */
#define GQE_NOALLOC_SCRATCH_BYTES (256ull << 20)
gqe_status gqe_attn_fwd_noalloc(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                                const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                                const void* Wo, void* out, int32_t* idx_out, float* w_out,
                                void* stream);

/* Dense GQA baseline over the same kernels: Hq query heads, G KV groups, head
 * h reads group h / (Hq/G), every head active on every token.
 * [GQA-w] "Mechanism"; [GQE-x] "Experimental results" (the 16-query, 8-KV
 * GQA model GQE is compared with).
 *   x [B*T, D]; Wq [Hq*d_h, D]; Wk, Wv [G*d_h, D]; Wo [D, Hq*d_h]; out [B*T, D].
 * Returns 0 (workspace) or GQE_ERR_SHAPE unless Hq is a positive multiple of
 * G with Hq <= 256. */
size_t gqa_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h,
                           int32_t dtype);
gqe_status gqa_attn_fwd(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h,
                        int32_t dtype, const void* x, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wo, void* out,
                        void* ws, size_t ws_bytes, void* stream);

/* Instrumented forms of gqe_attn_fwd and gqa_attn_fwd, for measurement:
 * same arguments, same results, and `events` (may be NULL) points at
 * GQE_N_STAGES+1 (resp. GQA_N_STAGES+1) hipEvent_t handles, each NULL or an
 * event the caller created. Event i is recorded on `stream` just before
 * stage i is enqueued, the last one after the final stage, so the time
 * between events i and i+1 is stage i's device time. Stages of the GQE
 * forward: 0 projection (K, V, Q_sh, router logits), 1 route, 2 scan,
 * 3 scatter, 4 sparse Q grouped GEMM, 5 attention, 6 weighted slot,
 * 7 output projection. Stages of the GQA forward: 0 projection (Q, K, V),
 * 1 attention, 2 output projection. */
#define GQE_N_STAGES 8
#define GQA_N_STAGES 3
gqe_status gqe_attn_fwd_timed(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                              const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                              const void* Wo, void* out, int32_t* idx_out, float* w_out,
                              void* ws, size_t ws_bytes, void* stream, void* const* events);
gqe_status gqa_attn_fwd_timed(int64_t B, int64_t T, int64_t D, int32_t Hq, int32_t G, int32_t d_h,
                              int32_t dtype, const void* x, const void* Wq, const void* Wk,
                              const void* Wv, const void* Wo, void* out,
                              void* ws, size_t ws_bytes, void* stream, void* const* events);

/* ---------------------------------------------------------------------------
 * Training: a forward that keeps its state for the backward, and the backward.
 * Gradients of L = <dout, out> + L_aux through the full layer (GQE_FULL, bf16
 * inputs; other variants and fp32 layers return GQE_ERR_UNSUPPORTED).
 * [GQE-x] "Architecture and routing" (the hard concatenation carries no
 * routing gradient; the renormalised weighted slot is the router's path) and
 * "Training and loss" (a load-balancing auxiliary loss); [GQE-n] part 5 (the
 * router learns through the weighted sum; balancing keeps experts in use).
 * The picks themselves are piecewise constant: no gradient flows through idx.
 * L_aux = aux_coef * (1/G) * sum_g M * sum_m f[g,m] * P[g,m], f[g,m] the share
 * of group g's B*T*k picks that chose expert m, P[g,m] the mean over tokens of
 * the router probability (the pages name such a loss but give no formula;
 * this is the common fraction-times-probability form, per group).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace the pair gqe_attn_fwd_train / gqe_attn_bwd needs
 * (0 if the shape is invalid or unsupported for training). */
size_t gqe_train_workspace_bytes(const gqe_shape* s);

/* gqe_attn_fwd with the same arguments and results, which also leaves in ws
 * what gqe_attn_bwd reads (routing, projections, merged slots, and each
 * attention row's log-sum-exp). ws_bytes >= gqe_train_workspace_bytes(s). */
gqe_status gqe_attn_fwd_train(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                              const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                              const void* Wo, void* out, int32_t* idx_out, float* w_out,
                              void* ws, size_t ws_bytes, void* stream);

/* gqe_attn_fwd_train with the picks given by the caller instead of the
 * router's: for checking the training pair against a reference routing where
 * two experts' logits nearly tie, or for routing chosen outside the layer.
 * The router logits are still computed (the backward's router gradient
 * needs them) and the weights are the picks' group-softmax probabilities
 * from those logits, renormalised over the token's G*k picks, exactly as the
 * router forms them; the backward then differentiates this forward.
 *   idx    [B*T, G, k] int32   picks, each in [0, M) and distinct within its
 *                              group; an entry outside [0, M) or repeating an
 *                              earlier rank's expert is replaced by the
 *                              group's lowest unused expert (never an
 *                              out-of-bounds access)
 *   w_out  [B*T, G, k] fp32    out (NULL to skip): the weights used
 * Other arguments, errors and the workspace as for gqe_attn_fwd_train;
 * GQE_ERR_NULL if idx is NULL. */
gqe_status gqe_attn_fwd_train_routed(const gqe_shape* s, const void* x, const void* Wr, const float* br,
                                     const void* Wq, const void* Wk, const void* Wv, const void* Wq_sh,
                                     const void* Wo, const int32_t* idx, void* out, float* w_out,
                                     void* ws, size_t ws_bytes, void* stream);

/* Backward of the layer. ws must be the workspace of the last
 * gqe_attn_fwd_train (or gqe_attn_fwd_train_routed) with the same shape and
 * inputs on this stream, unchanged since (the call overwrites its backward
 * part).
 *   x, Wr, Wq, Wk, Wv, Wq_sh, Wo   the forward's inputs (bf16, layouts as in
 *                                  gqe_attn_fwd_routed; br is not needed)
 *   dout     [B*T, D] bf16         gradient of the loss with respect to out
 *   aux_coef                       weight of the load-balancing loss (finite)
 *   dx       [B*T, D] fp32         out: gradient of x
 *   dWr      [G*M, D] fp32         out: router weight
 *   dbr      [G*M] fp32 or NULL    out: router offsets (NULL to skip)
 *   dWq      [G*M*d_h, D] fp32     out: expert queries (zero rows for experts
 *                                  no token picked)
 *   dWk, dWv [G*d_h, D] fp32       out
 *   dWq_sh   [d_h, D] fp32         out
 *   dWo      [D, (G*k+2)*d_h] fp32 out
 *   aux_loss [1] fp32 or NULL      out: the value of L_aux
 * Gradient outputs are written, not accumulated. Deterministic: the same
 * inputs on the same device give bit-identical results (no atomics).
 * Errors as for gqe_attn_fwd; GQE_ERR_SHAPE also for a non-finite aux_coef. */
gqe_status gqe_attn_bwd(const gqe_shape* s, const void* x, const void* Wr, const void* Wq,
                        const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                        const void* dout, float aux_coef, float* dx, float* dWr, float* dbr,
                        float* dWq, float* dWk, float* dWv, float* dWq_sh, float* dWo,
                        float* aux_loss, void* ws, size_t ws_bytes, void* stream);

/* Instrumented gqe_attn_bwd (events as for gqe_attn_fwd_timed, GQE_BWD_N_STAGES+1
 * entries). Stages: 0 operand layouts (transposes), 1 slot gradients dC = dout Wo
 * and dWo, 2 attention-row preparation and router backward, 3 attention dK/dV,
 * 4 attention dQ, 5 dx, 6 weight gradients of Wq, Wk, Wv, Wq_sh, Wr. */
#define GQE_BWD_N_STAGES 7
gqe_status gqe_attn_bwd_timed(const gqe_shape* s, const void* x, const void* Wr, const void* Wq,
                              const void* Wk, const void* Wv, const void* Wq_sh, const void* Wo,
                              const void* dout, float aux_coef, float* dx, float* dWr, float* dbr,
                              float* dWq, float* dWk, float* dWv, float* dWq_sh, float* dWo,
                              float* aux_loss, void* ws, size_t ws_bytes, void* stream,
                              void* const* events);

/* ---------------------------------------------------------------------------
 * Decode: one new token per sequence over a dense KV cache. GQE keeps the K/V
 * projections, and so the KV cache, of the underlying GQA model unchanged;
 * only the query side is sparse ([GQE-x] "Architecture and routing"; [GQE-n]
 * part 4). Full layer (GQE_FULL), bf16.
 *   s          B sequences; T = cache capacity per sequence (a multiple of 32,
 *              with one group's values, d_h*B*T*2 bytes, under 4 GiB; else
 *              GQE_ERR_SHAPE); D, G, M, k, d_h, shared_kv_group as for the layer
 *   pos        [B] int32, device: sequence b has pos[b] cached positions and the
 *              new token goes at position pos[b] (0 <= pos[b] < T; an entry
 *              outside that range leaves its cache untouched and its outputs
 *              unspecified, with no out-of-bounds access)
 *   x          [B, D] bf16 new tokens; weights as in gqe_attn_fwd
 *   k_cache    [G][B][T][d_h] bf16, in/out: keys; row pos[b] is written
 *   vt_cache   [G][d_h][B*T] bf16, in/out: values transposed (element
 *              (g, c, b*T + t) is value c of position t); column b*T + pos[b]
 *              is written. Positions past pos[b] are never read as data.
 *   out        [B, D] bf16; idx_out, w_out [B, G, k] optional as in gqe_attn_fwd
 * The layouts are those the prefill uses for K and V^T, so a cache can be
 * filled by projecting a prompt with the same weights. */
size_t gqe_decode_workspace_bytes(const gqe_shape* s);
gqe_status gqe_decode_step(const gqe_shape* s, const int32_t* pos, const void* x, const void* Wr,
                           const float* br, const void* Wq, const void* Wk, const void* Wv,
                           const void* Wq_sh, const void* Wo, void* k_cache, void* vt_cache, void* out,
                           int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes, void* stream);

/* Instrumented gqe_decode_step (events as for gqe_attn_fwd_timed,
 * GQE_DECODE_N_STAGES+1 entries). Stages: 0 new-token projections, routing,
 * sparse Q and cache append; 1 attention over the cache; 2 chunk merge,
 * merged slots and output projection. */
#define GQE_DECODE_N_STAGES 3
gqe_status gqe_decode_step_timed(const gqe_shape* s, const int32_t* pos, const void* x, const void* Wr,
                                 const float* br, const void* Wq, const void* Wk, const void* Wv,
                                 const void* Wq_sh, const void* Wo, void* k_cache, void* vt_cache,
                                 void* out, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events);

/* Diagnostic, not an operation of the pages: the device's sustained bf16
 * matrix-core rate, to put the kernels' rates in context (the published
 * dense peak assumes 2.4 GHz; under a sustained matrix load the chip is
 * power-limited). Launches `workgroups` workgroups of four waves; each wave
 * issues `iters` rounds of eight independent v_mfma_f32_16x16x32_bf16 on
 * register operands (no memory traffic in the loop), i.e.
 * workgroups * 4 * iters * 8 * 16384 flops, and writes one float per
 * workgroup to out (device, [workgroups], a checksum that keeps the work
 * live). Time it with events on `stream`.
 * Errors: GQE_ERR_NULL (out), GQE_ERR_SHAPE (workgroups < 1 or > 2^20,
 * iters < 1), GQE_ERR_ALIGN (out not 16-byte aligned), GQE_ERR_HIP. */
gqe_status gqe_mfma_probe(int64_t workgroups, int32_t iters, float* out, void* stream);

/* A static, NUL-terminated description of a status code. */
const char* gqe_status_str(gqe_status st);

#ifdef __cplusplus
}
#endif

#endif /* GQE_H */
