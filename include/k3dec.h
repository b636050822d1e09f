/*
 * k3dec.h -- C ABI of libk3dec, the MoE decode-layer hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * The library computes one MoE transformer layer's token-side work at decode
 * batch sizes 1-64, as described in "Hyper Optimizing Kimi K3 in vLLM: Moving
 * Fast and Responsibly" (Part 1): router scoring with top-k expert selection,
 * the latent input projection, the routed-expert SwiGLU, the shared expert on
 * its own stream, the attention input projection, the attention output
 * projection with residual add and RMSNorm, and a side-stream weight
 * prefetch. The attention core itself is not part of the library.
 *
 * Conventions, common to every entry point:
 *  - Pointers marked "device" are device (HBM) addresses; the caller owns
 *    every buffer, including the workspace. The library never allocates,
 *    never synchronises the host and never prints.
 *  - Matrices are [out x in], row-major, with the input index contiguous
 *    (a weight row is one output's input vector). bf16 values travel as
 *    uint16_t bit patterns. Activation rows may have a leading dimension
 *    (ld*, in elements) larger than their width.
 *  - Every device pointer must be 16-byte aligned, every leading dimension
 *    and every contracted width (d, K, I) a multiple of 8 elements.
 *  - All calls are asynchronous on the given stream (a hipStream_t passed as
 *    void*; NULL means the default stream) and keep the order of their
 *    kernels on it. Inputs must stay valid and unmodified until that work
 *    completes.
 *  - Weights are read with non-temporal loads and must not change while a
 *    call that reads them is in flight; activations are read with ordinary
 *    loads after the stream ordering makes them visible.
 *  - Every fp32 -> bf16 store rounds to nearest even.
 *  - Return value: K3_OK, or a negative K3_ERR_* code. On any error other
 *    than K3_ERR_HIP nothing has been launched. Unsupported shapes fail with
 *    K3_ERR_UNSUPPORTED; there is no silent fallback to another path.
 *  - Results are deterministic: the same inputs on the same device give the
 *    same output bits, whatever the scheduling.
 */
#ifndef K3DEC_H
#define K3DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status */
#define K3_OK 0
#define K3_ERR_INVALID_ARG (-1)  /* NULL pointer, non-positive size, bad ld */
#define K3_ERR_UNSUPPORTED (-2)  /* shape outside the supported range, or misaligned */
#define K3_ERR_WORKSPACE (-3)    /* workspace NULL or smaller than the size query says */
#define K3_ERR_HIP (-4)          /* the HIP runtime reported an error at launch */
#define K3_ERR_SCRATCH (-5)      /* the shape needs more than K3_NOALLOC_SCRATCH_BYTES of scratch */

/* Limits of the library (argument checks return K3_ERR_UNSUPPORTED beyond them). */
#define K3_MAX_BATCH 64      /* tokens per call */
#define K3_MAX_EXPERTS 1024  /* routed experts E */
#define K3_MAX_TOPK 32       /* experts per token k */

/* Human-readable text for a status code (static storage, never NULL). */
const char *k3_status_string(int status);

/* Library version, as major * 10000 + minor * 100 + patch. */
int k3_version(void);

/* ------------------------------------------------------------ dispatch record
 * Each entry point records which kernel variant it launched, so tests can
 * check that a given shape really ran the path it claims (a test that runs a
 * different path proves nothing about the one it names).
 */
#define K3_OP_ROUTER_TOPK 0
#define K3_OP_PROJ_SKINNY 1
#define K3_OP_MOE_EXPERTS 2
#define K3_OP_SHARED_EXPERT 3
#define K3_OP_OPROJ_RESIDUAL 4
#define K3_OP_PREFETCH 5
#define K3_OP_ROUTER_LATENT 6
#define K3_OP_MOE_BLOCK 7
/* Not an entry point: the engine the routed experts' gate/up and down
 * products ran on in the last successful k3_moe_experts or k3_moe_block
 * call -- K3_VARIANT_DOT2 (VALU dot2 row engines: every expert holds at most
 * four tokens of the call) or K3_VARIANT_MFMA (every expert's tokens on bf16
 * MFMA 16x16x32 tiles). The automatic choice is DOT2 for b <= 4 and MFMA
 * above. k3_force_variant(K3_OP_EXPERT_ENGINE, K3_VARIANT_MFMA) runs
 * batches 2-4 on the MFMA tiles too (batch 1 and DOT2 above batch 4 are not
 * available and fail with K3_ERR_UNSUPPORTED). */
#define K3_OP_EXPERT_ENGINE 8
/* Not an entry point: the MFMA pass of the last dense projection above four
 * tokens -- K3_VARIANT_WHOLEK (5-32 tokens, K a multiple of 1024 with seven
 * or eight 1024-wide slices: whole-K workgroups, no partial sums),
 * K3_VARIANT_RESIDENT (token-resident split-K pass, up to 32 tokens) or
 * K3_VARIANT_SPLITK (per-chunk split-K pass, 33-64 tokens). Recorded by
 * k3_proj_skinny, k3_oproj_residual and the router passes of
 * k3_router_topk(_latent), k3_shared_expert and the MoE block above four
 * tokens. It cannot be forced. */
#define K3_OP_DENSE_PASS 9

#define K3_VARIANT_NONE 0
#define K3_VARIANT_DOT2 1    /* VALU dot2 GEMV: whole weight rows per wave */
#define K3_VARIANT_MFMA 2    /* bf16 MFMA 16x16x32 tiles, K split inside the workgroup */
#define K3_VARIANT_GROUPED 3 /* permutation + grouped expert tiles */
#define K3_VARIANT_STREAM 4  /* plain streaming kernel */
/* k3_router_topk at batch 1 only: the router projection's last workgroup
 * selects the experts (one kernel instead of the projection and a top-k
 * kernel). Each workgroup publishes its logits with an agent-scope release
 * fence and takes a ticket from a counter in bytes 0-3 of the workspace; the
 * holder of the last ticket acquires, resets the counter and runs the top-k.
 * Those bytes must be zero before the first call on a workspace; each call
 * leaves them zero. Measured slower on gfx950 than the two-kernel default
 * (the fences write back and invalidate the L2 of every workgroup's XCD);
 * kept so that the comparison can be repeated. */
#define K3_VARIANT_LASTWG 5
#define K3_VARIANT_WHOLEK 6   /* K3_OP_DENSE_PASS only */
#define K3_VARIANT_RESIDENT 7 /* K3_OP_DENSE_PASS only */
#define K3_VARIANT_SPLITK 8   /* K3_OP_DENSE_PASS only */

/* Variant the last successful call of `op` on this process launched. */
int k3_get_last_dispatch(int op);

/* Force a variant for `op` (K3_VARIANT_NONE restores the automatic choice).
 * A forced variant that cannot run a shape makes that call fail with
 * K3_ERR_UNSUPPORTED. For tests and measurements only. */
int k3_force_variant(int op, int variant);

/* Tracing: while set, every call of `op` records `begin` (a hipEvent_t as
 * void*) on its stream right before the op's main kernel and `end` right
 * after it -- k3_moe_experts: the grouped gate/up kernel (also when
 * k3_moe_block runs it); k3_shared_expert: its gate/up kernel;
 * k3_router_topk(_latent): the projection kernel; k3_moe_block: its first
 * kernel; the others: their only or first kernel. NULL events clear the hook. The records are plain
 * hipEventRecord calls, so they time eager calls; inside a stream capture
 * they only mark capture dependencies (ROCm rejects external event nodes).
 * Process-wide state, for measurement only; not safe against concurrent
 * calls of the same op. */
int k3_trace_events(int op, void *begin, void *end);

/* ------------------------------------------------------------ workspace sizes
 * Bytes of device workspace each entry point needs for the given shape
 * (16-byte aligned, caller-owned; 0 for a non-positive size argument).
 * Workspaces need no initialisation and keep no state between calls. A
 * workspace serves one call at a time: calls that may overlap need
 * workspaces of their own. The router queries, which are not given the
 * reduction width, return the bound over every width.
 */
size_t k3_router_topk_workspace_size(int b, int E);
size_t k3_router_topk_latent_workspace_size(int b, int E, int d_lat);
size_t k3_proj_skinny_workspace_size(int b, int K, int N);
size_t k3_moe_experts_workspace_size(int b, int d_in, int E, int k, int I, int d_out);
size_t k3_shared_expert_workspace_size(int b, int d, int I);
size_t k3_oproj_residual_workspace_size(int b, int K, int d);
size_t k3_moe_block_workspace_size(int b, int d, int E, int k, int d_lat, int I, int I_s);
size_t k3_moe_block_rmsnorm_workspace_size(int b, int d, int E, int k, int d_lat, int I, int I_s);

/* ------------------------------------------------------------ entry points */

/* Router scores and top-k selection.
 * "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3 ("Improve MoE
 * scheduling and overlap"): the router scores every expert from the layer
 * input before the routed experts run.
 *
 *   logits[t][e] = sum_i x[t][i] * w_router[e][i]  (+ bias[e])      fp32
 *   topk_ids[t]  = the k experts of highest logit, in descending logit
 *                  order; equal logits rank the lower expert index first
 *   topk_w[t][j] = softmax over the k selected logits (equivalently, the
 *                  softmax over all E renormalised over the selection);
 *                  the k weights of a token sum to 1
 *
 * x        device, [b x d] bf16, row stride ldx
 * w_router device, [E x d] bf16
 * bias     device, [E] fp32, or NULL for none
 * topk_ids device, [b x k] int32 (output)
 * topk_w   device, [b x k] fp32 (output)
 * workspace device, >= k3_router_topk_workspace_size(b, E) bytes (with the forced
 *          K3_VARIANT_LASTWG its first 4 bytes zero on the first call)
 * Limits: 1 <= b <= 64, 1 <= k <= min(E, 32), E <= 1024.
 */
int k3_router_topk(const uint16_t *x, int64_t ldx, int b, int d,
                   const uint16_t *w_router, const float *bias, int E, int k,
                   int32_t *topk_ids, float *topk_w,
                   void *workspace, size_t ws_bytes, void *stream);

/* Router scores, top-k selection and the latent input projection in one
 * pass over the same input. "Hyper Optimizing Kimi K3 in vLLM", Part 1
 * section 3: the router scores and the latent input projection are combined
 * into one matrix multiplication, removing a second read of the input and
 * a kernel launch before the experts run.
 *
 * Computes what k3_router_topk(x, ...) and k3_proj_skinny(x, w_lat -> z)
 * compute, with one pass over the router and latent rows (then a small
 * top-k kernel).
 *
 * w_lat device, [d_lat x d] bf16;  z device, [b x d_lat] bf16 (output), row
 * stride ldz; workspace >= k3_router_topk_latent_workspace_size(b, E, d_lat)
 * bytes; the other arguments and the limits are those of k3_router_topk.
 */
int k3_router_topk_latent(const uint16_t *x, int64_t ldx, int b, int d,
                          const uint16_t *w_router, const float *bias, int E, int k,
                          const uint16_t *w_lat, int d_lat, int32_t *topk_ids, float *topk_w,
                          uint16_t *z, int64_t ldz, void *workspace, size_t ws_bytes,
                          void *stream);

/* Skinny projection y = x . W^T, for the latent input projection
 * (Part 1 section 3) and the attention input projection (Part 1 section 1,
 * "Tune shapes for the workload": small-matrix kernels at batch 1-2,
 * work-splitting kernels above that).
 *
 *   y[t][n] = bf16( sum_i x[t][i] * w[n][i] ),  fp32 accumulation
 *
 * x device, [b x K] bf16, row stride ldx;  w device, [N x K] bf16;
 * y device, [b x N] bf16 (output), row stride ldy; y must not overlap x.
 * Variant: K3_VARIANT_DOT2 for b <= 4 and K <= 8192, K3_VARIANT_MFMA
 * otherwise: K is split into ranges whose fp32 partial sums go through the
 * workspace (>= k3_proj_skinny_workspace_size(b, K, N) bytes; the dot2
 * variant needs none and accepts NULL) and are summed in range order.
 * Limits: 1 <= b <= 64, K % 8 == 0.
 */
int k3_proj_skinny(const uint16_t *x, int64_t ldx, int b, int K,
                   const uint16_t *w, int N, uint16_t *y, int64_t ldy,
                   void *workspace, size_t ws_bytes, void *stream);

/* Routed experts: token-to-expert permutation, grouped SwiGLU gate/up, down
 * projection and weighted combine (Part 1 section 3; the routed experts run
 * after router and latent projection).
 *
 *   for each token t and slot j < k, with e = topk_ids[t][j]:
 *     g = w13[e][0:I]  . z_t,   u = w13[e][I:2I] . z_t     (gate rows, then up rows)
 *     h = silu(g) * u,          silu(g) = g / (1 + exp(-g))
 *     o = w2[e] . h
 *   y[t] = bf16( y_add[t] + sum_j topk_w[t][j] * o_(t,j) )
 *
 * z        device, [b x d_in] bf16, row stride ldz (the latent projection)
 * topk_ids device, [b x k] int32, each in [0, E), distinct within a token
 * topk_w   device, [b x k] fp32
 * w13      device, [E x 2I x d_in] bf16;  w2 device, [E x d_out x I] bf16
 * y_add    device, [b x d_out] fp32 added before the routed sum (the shared
 *          expert's output), or NULL for none
 * y_add_ready a hipEvent_t (as void*) that the stream waits on before the
 *          kernel that reads y_add, or NULL (then y_add must already be
 *          ordered before this call on `stream`)
 * y        device, [b x d_out] bf16 (output)
 * cu_budget upper bound on the compute units the call's kernels occupy
 *          (grid size); 0 = the whole device
 * Intermediates (h in bf16, per-slot expert outputs in fp32, the
 * permutation) live in the workspace. Ids outside [0, E) contribute
 * nothing; an id repeated within a token counts once per slot.
 * The combine adds y_add first, then the slots in order j = 0..k-1.
 * Limits: 1 <= b <= 64, 1 <= k <= 32, E <= 1024, I % 128 == 0, I <= 8192,
 * d_in % 128 == 0, d_in <= 8192, d_out % 16 == 0.
 */
int k3_moe_experts(const uint16_t *z, int64_t ldz, int b, int d_in,
                   const int32_t *topk_ids, const float *topk_w, int k,
                   const uint16_t *w13, const uint16_t *w2, int E, int I, int d_out,
                   const float *y_add, void *y_add_ready, uint16_t *y, int cu_budget,
                   void *workspace, size_t ws_bytes, void *stream);

/* Shared expert (Part 1 section 3: it runs on a separate stream, beside
 * routing or the routed experts, so it reads the layer input x).
 *
 *   y_s[t] = w2 . ( silu(w13[0:I] . x_t) * (w13[I:2I] . x_t) )      fp32
 *
 * x device, [b x d] bf16, row stride ldx;  w13 device, [2I x d] bf16;
 * w2 device, [d x I] bf16;  y_s device, [b x d] fp32 (output).
 * cu_budget as for k3_moe_experts. Limits: 1 <= b <= 64, I % 128 == 0,
 * d % 128 == 0, d and I <= 8192.
 */
int k3_shared_expert(const uint16_t *x, int64_t ldx, int b, int d,
                     const uint16_t *w13, const uint16_t *w2, int I,
                     float *y_s, int cu_budget,
                     void *workspace, size_t ws_bytes, void *stream);

/* The whole MoE block on one stream: router top-k, latent projection, shared
 * expert and routed experts, y = shared(x) + sum_j w_j routed_j(latent(x)).
 * "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3: router and latent
 * projection share one matrix pass; the shared expert's work overlaps the
 * routing. Nothing waits on another stream. At b = 1:
 *   1. one pass over x for the router rows, the latent rows and the shared
 *      expert's gate/up rows (logits, z, shared h);
 *   2. every workgroup selects the experts while its first units -- the
 *      shared expert's down rows (y_s) -- stream, then the routed gate/up
 *      rows + SwiGLU follow;
 *   3. routed down projection with the weighted combine, y_s added.
 * At 2 <= b <= 4 the selection runs in one workgroup beside the shared
 * down rows and the routed experts follow the permutation. Above b = 4 the
 * same steps run on the split-K MFMA engine (router, latent and shared
 * gate/up rows in one pass), the shared down projection after the
 * selection. Results equal k3_router_topk_latent + k3_shared_expert +
 * k3_moe_experts on the same inputs, bit for bit.
 *
 * x [b x d] bf16 (ldx); w_router [E x d], bias [E] fp32 or NULL, w_lat
 * [d_lat x d], w13 [E x 2I x d_lat], w2 [E x d x I], w13_s [2I_s x d],
 * w2_s [d x I_s] bf16. Outputs: topk_ids [b x k] int32, topk_w [b x k] fp32,
 * z [b x d_lat] bf16 (ldz), y_s [b x d] fp32 (the shared expert's output),
 * y [b x d] bf16. workspace >= k3_moe_block_workspace_size(...) bytes.
 * Limits: those of k3_router_topk_latent, k3_shared_expert and
 * k3_moe_experts.
 */
int k3_moe_block(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w_router,
                 const float *bias, int E, int k, const uint16_t *w_lat, int d_lat,
                 const uint16_t *w13, const uint16_t *w2, int I, const uint16_t *w13_s,
                 const uint16_t *w2_s, int I_s, int32_t *topk_ids, float *topk_w, uint16_t *z,
                 int64_t ldz, float *y_s, uint16_t *y, void *workspace, size_t ws_bytes,
                 void *stream);

/* The MoE block on the normalised hidden state, normalising it itself (the
 * RMSNorm that k3_oproj_residual applies, moved into the block's first
 * kernel at batch 1, so the step has one kernel boundary less):
 *
 *   x[t][n] = bf16( h32[t][n] / sqrt( (1/d) sum_m h32[t][m]^2 + eps ) * gamma[n] )
 *
 * then exactly k3_moe_block on x (same outputs, bit for bit the same as
 * k3_oproj_residual's y_norm fed to k3_moe_block).
 *
 * h32      device, [b x d] fp32, row stride d (e.g. k3_oproj_residual_h32)
 * gamma    device, [d] bf16
 * x_out    device, [b x d] bf16 (output), or NULL: receives x
 * The other arguments are k3_moe_block's (x and ldx replaced by the above).
 * workspace: >= k3_moe_block_rmsnorm_workspace_size(b, d, E, k, d_lat, I, I_s)
 * bytes. Limits: k3_moe_block's, and eps >= 0.
 */
int k3_moe_block_rmsnorm(const float *h32, int b, int d, const uint16_t *gamma, float eps,
                         uint16_t *x_out, const uint16_t *w_router, const float *bias, int E,
                         int k, const uint16_t *w_lat, int d_lat, const uint16_t *w13,
                         const uint16_t *w2, int I, const uint16_t *w13_s, const uint16_t *w2_s,
                         int I_s, int32_t *topk_ids, float *topk_w, uint16_t *z, int64_t ldz,
                         float *y_s, uint16_t *y, void *workspace, size_t ws_bytes,
                         void *stream);

/* The MoE block without a workspace argument, for callers that cannot
 * allocate device memory: code under stream (graph) capture, serving loops
 * and harnesses that forbid allocation. It runs exactly k3_moe_block (same
 * kernels, same outputs bit for bit) with the scratch memory in a static
 * device array of K3_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on, until the process ends. The first call on a device
 * looks that array's address up once; no call allocates or frees anything.
 *
 * Every call on a device shares that device's array: calls that overlap on
 * one device (two streams, or two host threads) race on it and give
 * undefined results. Serialise them, or use k3_moe_block with a workspace
 * each. The array keeps the last call's contents; no call needs it cleared.
 *
 * Arguments and limits are k3_moe_block's without workspace and ws_bytes.
 * Shapes whose k3_moe_block_workspace_size exceeds K3_NOALLOC_SCRATCH_BYTES
 * fail with K3_ERR_SCRATCH before anything is launched (the full-size layer,
 * d = d_lat = 7168, E = 384, k = 8, I = I_s = 2048, needs 27.7 MiB at
 * b = 64, so every batch 1..64 fits).
 */
#define K3_NOALLOC_SCRATCH_BYTES (32u << 20)
int k3_moe_block_noalloc(const uint16_t *x, int64_t ldx, int b, int d,
                         const uint16_t *w_router, const float *bias, int E, int k,
                         const uint16_t *w_lat, int d_lat, const uint16_t *w13,
                         const uint16_t *w2, int I, const uint16_t *w13_s,
                         const uint16_t *w2_s, int I_s, int32_t *topk_ids, float *topk_w,
                         uint16_t *z, int64_t ldz, float *y_s, uint16_t *y, void *stream);

/* Attention output projection with residual add and RMSNorm (Part 1
 * section 2, "Overlap computation and communication": the output
 * projection is fused with the attention residual that follows it).
 *
 *   h[t][n] = r[t][n] + sum_i a[t][i] * w_o[n][i]
 *   y[t][n] = bf16( h[t][n] / sqrt( (1/d) sum_m h[t][m]^2 + eps ) * gamma[n] )
 *
 * a        device, [b x K] bf16, row stride lda (may be a column slice of a
 *          wider projection output)
 * w_o      device, [d x K] bf16
 * residual device, [b x d] bf16, row stride d: read as r, overwritten with
 *          bf16(h) (in place)
 * gamma    device, [d] bf16
 * y_norm   device, [b x d] bf16 (output); must not overlap residual or a;
 *          or NULL: the norm is skipped (gamma may then be NULL too) and
 *          the fp32 h stays in the workspace for k3_moe_block_rmsnorm
 * The norm is taken over fp32 h, before h is rounded for the store.
 * workspace: >= k3_oproj_residual_workspace_size(b, K, d) bytes.
 * Limits: 1 <= b <= 64, d % 8 == 0, eps >= 0.
 */
int k3_oproj_residual(const uint16_t *a, int64_t lda, int b, int K,
                      const uint16_t *w_o, int d, uint16_t *residual,
                      const uint16_t *gamma, float eps, uint16_t *y_norm,
                      void *workspace, size_t ws_bytes, void *stream);

/* Where k3_oproj_residual leaves the fp32 h ([b x d], row stride d) in its
 * workspace: valid after the call on the same stream, until the workspace
 * is reused. Pure pointer arithmetic; NULL for a NULL workspace. */
const float *k3_oproj_residual_h32(const void *workspace);

/* Weight prefetch (Part 1 section 4, "Prefetching upcoming weights into
 * cache"): reads [p, p + bytes) once, so the next operator that reads those
 * weights finds them in the device's last-level cache (the MALL) instead of
 * HBM. Meant for a side stream while the main stream is in a phase that
 * leaves HBM bandwidth unused. Writes nothing the caller can observe.
 *
 * p device, 16-byte aligned; bytes a multiple of 16 (0 is a no-op).
 * cu_budget as for k3_moe_experts.
 */
int k3_prefetch(const void *p, size_t bytes, int cu_budget, void *stream);

/* Streaming-read reference (a measurement aid, not a step of the path):
 * reads [p, p + bytes) once with the non-temporal 128-bit loads the weight
 * streams use, one workgroup per compute unit, and discards the data. Its
 * rate over a few GB is the device's measured streaming-read ceiling, which
 * the path's kernels are compared with beside the 8 TB/s specification.
 *
 * p device, 16-byte aligned; bytes a multiple of 16 (0 is a no-op).
 * Errors as k3_prefetch. Asynchronous on `stream`.
 */
int k3_stream_read(const void *p, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* K3DEC_H */
