/*
 * moe.h - C ABI of the MI355X (gfx950) forward pass of a top-k routed
 * Mixture-of-Experts FFN layer.
 *
 * The layer, as the pages define it:
 *   z = W_r^T x                        router scores, one per expert
 *   T = TopK(z + b, k)                 b: optional selection-only bias
 *   g = softmax of z over T            (or the full softmax's value at T)
 *   y = sum_{i in T} g_i f_i(x)  (+ shared expert)
 * with each f_i a SwiGLU FFN, executed batch-wise as route -> permute ->
 * grouped expert GEMMs -> unpermute/combine.
 *
 * Sources (page title, section):
 *   [CME295]  "Week 2 Day 2: Mixture of Experts" course notes (semidirectx.com),
 *             §1.3 formalism, §3.2 balance loss, §3.3 capacity, §4.1 shared
 *             experts, §4.2 selection bias, §A.1/A.2 API and pitfalls.
 *   [FANDEX]  "Mixture-of-Experts models" (fanquanpp.github.io), step 1: route().
 *   [15-779]  CMU 15-779 "Lecture 21: Mixture-of-Experts" notes
 *             (semidirectx.com), §2.1 gating, §2.5 top-1, §3.2 the four batched
 *             steps, §3.3 permutation by prefix sum and GroupGemm, §3.5 capacity.
 *   [W11]     "W11: MoE routing and parallel cost" (botof.cn), §3 capacity, §5
 *             metrics.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them. Tensors are dense row-major, 16-byte
 *     aligned. "elt" below is float (MOE_F32) or bf16 bit patterns (MOE_BF16).
 *   - x[T, d]; w_router[E, d] (row e = expert e's score vector);
 *     w1, w3[E, d_ff, d]; w2[E, d, d_ff]; shared ws1, ws3[d_ff_shared, d],
 *     ws2[d, d_ff_shared] (n_shared == 1).
 *   - Index tensors are int32: idx[T, k] (rank order, best first),
 *     dest[T, k] (row of each assignment, -1 when dropped), src[T*k] (token of
 *     each row), offsets[E+1] (CSR indptr of the row groups).
 *   - Rows are grouped by expert and ordered by token inside a group
 *     ([15-779] §3.3). Rows [offsets[E], T*k) are unused.
 *   - Expert outputs y_perm are fp32 [T*k + n_shared*T, d]; the shared expert's
 *     output for token t is row T*k + t. The layer output y[T, d] is fp32.
 *   - `ws` is caller-provided device scratch, 256-byte aligned, of at least the
 *     size that moe_workspace_size() returns for that entry point; its contents
 *     on entry do not matter and on return are undefined. moe_combine uses no
 *     scratch and accepts ws == NULL.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; the call never synchronises the host and never reads
 *     device data back. The expert entry points (moe_expert_*, moe_forward)
 *     for decode-sized batches with a shared expert run part of their work
 *     on a side stream the library keeps per device, forked from
 *     `stream` by an event and joined back into it, so every effect of the call
 *     is still ordered on `stream`.
 *   - Arguments are validated before anything is enqueued. On any error the
 *     call returns a non-zero moe_status, enqueues nothing and leaves all
 *     outputs untouched. A failed kernel launch returns MOE_ERR_HIP (work
 *     enqueued before the failure may have run). moe_last_error() gives a
 *     message for the calling thread's most recent error.
 *   - T == 0 is valid and enqueues nothing.
 *   - The library keeps no data between calls (only the side streams and their
 *     events); calls from several host threads are safe when they use distinct
 *     workspaces and outputs.
 *   - Results are deterministic: the same inputs give bitwise-equal outputs.
 *   - The calls enqueue kernels and events only (no allocation, memset, copy or
 *     synchronisation), so a call may be captured into a HIP graph on `stream`
 *     and replayed; the side stream joins the capture through its fork event.
 *     Make one call of the same shape before capturing (it sets the kernels'
 *     LDS limits, a host-side step).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* bad size, null required pointer, k > E, ...      */
  MOE_ERR_UNSUPPORTED = 2,  /* valid layer the kernels do not cover (d % 64,
                               capacity with E*k > 4096)                        */
  MOE_ERR_WORKSPACE = 3,    /* ws NULL or ws_bytes below moe_workspace_size()  */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed       */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gate of the chosen experts ([CME295] §1.3):
 *   SELECTED: softmax of the unbiased logits over the k chosen experts
 *             (Mixtral; DeepSeek-V3 renormalised over its top-8).
 *   ALL:      the full softmax probability of each chosen expert, not
 *             renormalised (Switch top-1, [15-779] §2.5).                      */
typedef enum { MOE_GATE_SOFTMAX_SELECTED = 0, MOE_GATE_SOFTMAX_ALL = 1 } moe_gate_mode;

/* Entry points, for moe_workspace_size(). */
typedef enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_PERMUTE = 1,
  MOE_STAGE_EXPERT_FFN = 2,
  MOE_STAGE_COMBINE = 3,
  MOE_STAGE_FORWARD = 4,
  MOE_STAGE_EXPERT_GATEUP = 5,
  MOE_STAGE_EXPERT_DOWN = 6,
  MOE_STAGE_BACKWARD = 7
} moe_stage;

/* Layer shape and options. Names follow the pages: E experts
 * (num_local_experts), k active per token (num_experts_per_tok), d model
 * width, d_ff expert width (moe_intermediate_size), n_shared always-on experts
 * (n_shared_experts), capacity factor cf and balance-loss weight alpha
 * (router_aux_loss_coef) ([CME295] §A.1).                                      */
typedef struct {
  int32_t T;                /* tokens in the batch, >= 0                        */
  int32_t d;                /* model width, multiple of 64                      */
  int32_t E;                /* routed experts, 1..1024                          */
  int32_t k;                /* experts per token, 1..min(E, 16)                 */
  int32_t d_ff;             /* routed expert width, multiple of 64              */
  int32_t n_shared;         /* 0 or 1 always-on shared expert ([CME295] §4.1)   */
  int32_t d_ff_shared;      /* shared expert width, multiple of 64 (ignored when
                               n_shared == 0)                                   */
  int32_t gate_mode;        /* moe_gate_mode                                    */
  int32_t dtype;            /* moe_dtype of x and all weights                   */
  int32_t ep_ranks;         /* 0 or 1: one device. n > 1: lay the rows out as n
                               simulated expert-parallel ranks ([15-779] §5.1):
                               rank r holds experts [r*E/n, (r+1)*E/n) and
                               tokens [r*T/n, (r+1)*T/n); rows are grouped by
                               (destination rank, source rank, local expert),
                               token order inside a group, so each rank's send
                               and receive buffers are contiguous. n must
                               divide E and T, n*E <= 1024, no capacity.
                               offsets then has n*E + 1 entries (group
                               g = (r*n + s)*(E/n) + local expert) and the
                               stats counts/kept n*E (one per group).         */
  double capacity_factor;   /* cf <= 0: no capacity. Otherwise each expert keeps
                               at most C = ceil(cf*T*k/E) assignments, first
                               choices before second choices, tokens in order
                               ([15-779] §3.5, [W11] §3); dropped assignments
                               contribute 0 to y ([CME295] §3.3).              */
  float aux_alpha;          /* alpha of L_aux = alpha*E*sum f_i P_i             */
  float reserved2;          /* must be 0                                        */
} moe_config;

/* Optional router/load statistics ([CME295] §3.2 and §3.4, [W11] §3 and §5);
 * every pointer is a nullable device pointer. Means are over the T tokens;
 * p_t is the full softmax of the unbiased logits z_t.
 *   counts[E]  assignments per expert before any drop (int32)
 *   kept[E]    assignments per expert after capacity (int32)
 *   n_dropped  dropped assignments, T*k - sum(kept) (int32[1])
 *   f[E]       counts / T (all k choices counted, before drops)
 *   P[E]       mean over tokens of the full softmax probability
 *   aux        alpha * E * sum_i f_i P_i (float[1])
 *   z_loss     mean_t (log sum_i e^{z_{t,i}})^2, the router z-loss (float[1])
 *   entropy    mean_t of -sum_i p_{t,i} ln p_{t,i} (float[1])
 *   max_prob   mean_t of max_i p_{t,i} (float[1])
 *   top_gap    mean_t of p_{t,(1)} - p_{t,(2)}, the two largest probabilities
 *              (p_{(2)} = 0 when E = 1) (float[1])
 *   margin[T]  per token, s_(k) - s_(k+1): the k-th largest selection score
 *              s = z + b minus the largest score left out (+inf when k = E),
 *              how far the top-k choice is from a tie ([CME295] §1.3, the
 *              top-k step; §4.2 for b) (float)
 *   touched    experts that keep at least one assignment after capacity, i.e.
 *              whose weights the expert products read ([15-779] §3.1 and
 *              §4.2: experts a batch touches) (int32[1])
 *   max_over_mean  max_e load_e / (T*k/E), load_e = assignments before drops:
 *              the busiest expert's load over the mean ([CME295] §3.3 and
 *              §4.2; [15-779] §3.4), computed in double and rounded once to
 *              float (float[1])
 * z_loss .. margin are computed by moe_route / moe_forward; all in fp32 with
 * fixed summation orders (reproducible bit for bit). counts, kept, n_dropped,
 * touched and max_over_mean are computed by moe_permute / moe_forward; with
 * ep_ranks = n > 1, touched and max_over_mean are per expert, summed over its
 * n groups.                                                                   */
typedef struct {
  int32_t* counts;
  int32_t* kept;
  int32_t* n_dropped;
  float* f;
  float* P;
  float* aux;
  float* z_loss;
  float* entropy;
  float* max_prob;
  float* top_gap;
  float* margin;
  int32_t* touched;
  float* max_over_mean;
} moe_stats;

/* Human-readable status name; never NULL. */
const char* moe_status_string(moe_status s);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* moe_last_error(void);

/* Bytes of device workspace `stage` needs for this config (>= 256, a multiple
 * of 256). Pure host computation. Errors: INVALID_ARG for a bad config or a
 * NULL `bytes`, UNSUPPORTED for a shape the kernels do not cover.            */
moe_status moe_workspace_size(const moe_config* cfg, moe_stage stage, size_t* bytes);

/* Steps 1-3: router scores, top-k, gates ([CME295] §1.3 and §4.2;
 * [FANDEX] step 1; [15-779] §2.1).
 *   z = W_r^T x in fp32 accumulation (only the router runs in fp32:
 *   [15-779] §7.1 selective precision); selection on z + sel_bias, highest
 *   first, ties to the lower expert index; gates from the unbiased z.
 *   x[T,d] elt, w_router[E,d] elt, sel_bias[E] fp32 (nullable)
 *   -> idx[T,k] int32, gates[T,k] fp32 (both required).
 *   stats (nullable): fills f, P, aux, z_loss, entropy, max_prob and top_gap
 *   when their pointers are set.                                              */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* sel_bias, int32_t* idx, float* gates,
                     const moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Step 4: per-expert histogram, capacity and the permutation by prefix sum
 * ([15-779] §3.3 and §3.5).
 *   idx[T,k] int32 (entries must be in [0, E) and distinct per token: not
 *   checked on the device) -> offsets[E+1], dest[T,k], src[T*k] int32
 *   (required). x_perm (nullable, elt [T*k, d]): when set, also gathers
 *   x_perm[r] = x[src[r]] (x then required).
 *   stats (nullable): fills counts, kept, n_dropped, touched and
 *   max_over_mean when set.                                                  */
moe_status moe_permute(const moe_config* cfg, const int32_t* idx, const void* x,
                       int32_t* offsets, int32_t* dest, int32_t* src, void* x_perm,
                       const moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Step 5: the grouped SwiGLU experts, Z = GroupGemm(data, indptr, weights)
 * ([15-779] §3.3), f(u) = W2 (silu(W1 u) * (W3 u)), silu(v) = v/(1+e^-v), no
 * biases ([CME295] §2.1), plus the always-on shared expert on every token.
 *   data row r of group e (r in [offsets[e], offsets[e+1])) is x[src[r]]
 *   when src is set (the gather is fused), else row r of `x` itself
 *   (x then holds T*k pre-permuted rows; n_shared must be 0).
 *   -> y_perm fp32 [T*k + n_shared*T, d]; rows outside the groups and the
 *   shared block are left untouched.
 *   The SwiGLU hidden activation is rounded before the W2 product: to IEEE
 *   half (11-bit significand, round to nearest even) for bf16 layers, whose W2
 *   is then widened to half inside the product (exact for |w| >= 2^-17; smaller
 *   weights move by at most 2^-25); to fp32 for fp32 layers. Half overflows
 *   above 65504, an activation magnitude the layer's inputs never approach.  */
moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* src,
                          const int32_t* offsets, const void* w1, const void* w3,
                          const void* w2, const void* ws1, const void* ws3,
                          const void* ws2, float* y_perm, void* ws, size_t ws_bytes,
                          void* stream);

/* First half of moe_expert_ffn: the SwiGLU hidden activation
 * act[r] = silu(W1_e u) * (W3_e u) for every grouped row r, data rows as in
 * moe_expert_ffn, and for the shared expert act[T*k + t] from x[t] with ws1,
 * ws3. act is [T*k + n_shared*T, moe_act_stride(cfg)] of IEEE half (bf16
 * layers) or fp32 (fp32 layers), 2 or 4 bytes per element; routed rows use the
 * first d_ff columns, shared rows the first d_ff_shared.                      */
moe_status moe_expert_gateup(const moe_config* cfg, const void* x, const int32_t* src,
                             const int32_t* offsets, const void* w1, const void* w3,
                             const void* ws1, const void* ws3, void* act,
                             void* ws, size_t ws_bytes, void* stream);

/* Second half: y_perm[r] = W2_e act[r] in fp32 for every grouped row, and
 * y_perm[T*k + t] = Ws2 act[T*k + t] for the shared expert; act as written by
 * moe_expert_gateup (half for bf16 layers).                                  */
moe_status moe_expert_down(const moe_config* cfg, const void* act, const int32_t* offsets,
                           const void* w2, const void* ws2, float* y_perm,
                           void* ws, size_t ws_bytes, void* stream);

/* Row stride in elements of the `act` buffer: max(d_ff, n_shared*d_ff_shared);
 * -1 for an invalid config.                                                  */
int32_t moe_act_stride(const moe_config* cfg);

/* Step 6: unpermute and mix ([CME295] §1.3 y = sum g_i f_i(x); [15-779] §3.2
 * step 4): y[t] = sum_{j: dest[t,j] >= 0} gates[t,j] * y_perm[dest[t,j]]
 * (+ y_perm[T*k + t] when n_shared == 1), summed in slot order j = 0..k-1.
 *   y_perm fp32, dest int32 [T,k], gates fp32 [T,k] -> y fp32 [T,d].       */
moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* dest,
                       const float* gates, float* y, void* ws, size_t ws_bytes,
                       void* stream);

/* Backward of the layer: gradients of L = sum_t <dy_t, y_t> + L_aux (L_aux only
 * when cfg->aux_alpha > 0; [CME295] §3.2) with respect to x, W_r and every
 * expert's (and the shared expert's) weights. The forward is recomputed from
 * the same inputs (router, index, the expert pre-activations), so nothing has
 * to be kept from moe_forward. The top-k selection and capacity drops pass no
 * gradient ([CME295] §1.3); SELECTED gates: dz = g (dg - sum g dg) on the
 * selected logits, ALL gates: dz = p (dp - sum p dp) ([15-779] §2.5); the
 * expert products are the transposed GEMMs ([15-779] §7: dW2 = H^T dY, ...),
 * bf16 operands with fp32 accumulation (the SwiGLU pre-activations are kept
 * in fp32, the activation and the propagated gradients rounded to bf16 before
 * each product).
 *   inputs as moe_forward (bf16 only), dy[T,d] fp32 (required);
 *   outputs fp32, every one required except the shared expert's (required
 *   when n_shared = 1): dx[T,d], dw_router[E,d], dw1/dw3[E,d_ff,d],
 *   dw2[E,d,d_ff], dws1/dws3[d_ff_shared,d], dws2[d,d_ff_shared]; experts
 *   that receive no row get zero gradients.
 *   ws: moe_workspace_size(cfg, MOE_STAGE_BACKWARD). T == 0 leaves the
 *   outputs untouched.
 * Streams: all work runs on `stream`, ordered after what precedes the call;
 * everything after it on `stream` sees the results. Two calls that share a
 * workspace must be ordered on one stream.
 * Errors: INVALID_ARG (bad config, NULL or misaligned pointer), WORKSPACE,
 * UNSUPPORTED (fp32, ep_ranks > 1, or d, d_ff, d_ff_shared not multiples of
 * 256).                                                                       */
moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const float* sel_bias, const void* w1, const void* w3, const void* w2,
                        const void* ws1, const void* ws3, const void* ws2, const float* dy,
                        float* dx, float* dw_router, float* dw1, float* dw3, float* dw2,
                        float* dws1, float* dws3, float* dws2, void* ws, size_t ws_bytes,
                        void* stream);

/* Dispatch volume of the simulated expert-parallel layout (cfg->ep_ranks = n
 * > 1; [15-779] §5.1 and §10 exercise 6): rows[s*n + r] = rows source rank s
 * sends to destination rank r in the dispatch all-to-all (s == r stays local;
 * the combine all-to-all returns the same rows), read from the offsets that
 * moe_permute / moe_forward produced. Bytes = rows * d * element size.
 *   offsets[n*E + 1] int32, rows[n*n] int32 (both required).
 * T == 0 leaves rows untouched. Errors: INVALID_ARG (bad config,
 * ep_ranks <= 1, NULL or misaligned pointer).                                */
moe_status moe_ep_traffic(const moe_config* cfg, const int32_t* offsets, int32_t* rows,
                          void* stream);

/* Auxiliary-loss-free balancing step ([CME295] §4.2; [15-779] §2.4): after a
 * step, bias[e] -= gamma if counts[e] > T*k/E, += gamma if counts[e] < T*k/E,
 * unchanged at the mean (compared exactly as counts[e]*E vs T*k). The bias is
 * the sel_bias of moe_route / moe_forward: it moves the top-k selection only,
 * never the gates.
 *   counts[E] int32 (e.g. moe_stats.counts of the step; with ep_ranks = n > 1
 *   the per-group counts[n*E], summed per expert; required),
 *   bias[E] fp32, updated in place (required); gamma finite.
 * Errors: INVALID_ARG (bad config, NULL or misaligned pointer, non-finite
 * gamma) before anything is launched.                                        */
moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma, float* bias,
                           void* stream);

/* The whole layer in one call: y_t = sum_{i in TopK} g_{t,i} f_i(x_t) (+ the
 * shared expert) ([CME295] §1.3), batched as the four steps route -> permute
 * -> grouped experts (+shared) -> combine ([15-779] §3.2), on one stream, with
 * every intermediate in `ws`.
 *   idx_out[T,k], gates_out[T,k] (nullable) receive the routing; stats as in
 *   moe_route + moe_permute.
 *   y[T,d] fp32 is written in full (dropped assignments add 0).
 * Errors: INVALID_ARG / UNSUPPORTED / WORKSPACE before anything is launched;
 * HIP when a launch fails (moe_last_error names the kernel).               */
moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* sel_bias, const void* w1, const void* w3,
                       const void* w2, const void* ws1, const void* ws3, const void* ws2,
                       float* y, int32_t* idx_out, float* gates_out,
                       const moe_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * call and results, with no workspace argument. Its scratch is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until
 * the process ends; the array's address on a device is looked up on the first
 * call there (make that call before any capture). Enough for decode-sized
 * batches and prefills of a few hundred tokens (moe_workspace_size(cfg,
 * MOE_STAGE_FORWARD) tells); a layer that needs more returns MOE_ERR_WORKSPACE
 * before anything is launched. Calls on one GPU share its array: calls that
 * overlap on one GPU (other streams, other host threads) race and must not be
 * issued; calls ordered on one stream are safe. The array keeps the last call's
 * contents; nothing in it needs to start at zero. Other errors as moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                               const float* sel_bias, const void* w1, const void* w3,
                               const void* w2, const void* ws1, const void* ws3,
                               const void* ws2, float* y, int32_t* idx_out, float* gates_out,
                               const moe_stats* stats, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
