/*
 * moe.h -- C ABI of libmoe.so: the forward pass of a DeepSeek-V3-lineage
 * mixture-of-experts feed-forward layer on one AMD MI355X (gfx950).
 *
 * The layer (sources are page title and section):
 *
 *   z   = x . W_r^T                       router logits over E routed + S shared
 *   s   = sigmoid(z)                      independent affinities, no softmax
 *   top = top-k of s[:E] + b              bias steers selection only
 *   g   = s[top U shared] / sum(...)      one joint normalisation over k + S
 *   y   = sum_i g_i * SwiGLU_i(x)         k routed + S shared contributions
 *   b  += gamma * sign(Lbar - L)          after the batch, from the loads L
 *
 * - "Inkling, Dissected", chapter 02 "Anatomy of one MoE layer" and 02b
 *   "Sigmoid, not softmax" (router equation, joint normalisation, the
 *   per-token sketch of the layer);
 * - "Inkling, Dissected", 02e "The aux-loss-free bias" (balancing rule);
 * - "Under The Hood: Inkling from Thinking Machines", "MoE: the expert
 *   configuration" (SwiGLU experts, shared experts of the same width) and
 *   "The routing strategy: sigmoid + shared expert sink" (top-k over the
 *   routed experts only, shared scores inside the normalisation).
 *
 * Conventions for every call:
 * - Every tensor pointer is a DEVICE pointer owned by the caller; tensors
 *   are dense row-major, 16-byte aligned (256 recommended).  The library
 *   never allocates, frees or synchronises; it keeps no mutable global
 *   state apart from the scratch array of moe_dispatch_noalloc (one per
 *   GPU, described there).  Workspace is caller-provided device memory of
 *   at least moe_workspace_size() bytes for that call.
 * - Calls are asynchronous on `stream`.  The returned status covers host-side
 *   validation (nothing is launched when it is not MOE_OK) plus launch errors
 *   (MOE_ERR_HIP).  Device faults surface at the caller's next sync.
 * - No C++ exception crosses this boundary.
 * - Floating-point inputs holding NaN or Inf give undefined results.
 *   A pair whose expert id handed to moe_dispatch lies outside [0, E) is
 *   counted in no load, enters no expert's rows and gets pair_pos = -1, so
 *   moe_combine leaves it out as it does a pair dropped at capacity (and
 *   the bias update sees only the valid pairs).
 * - Supported shapes: E in {64, 128, 256}, S in {0, 1, 2}, k = 6;
 *   act == weight, either MOE_F32 or MOE_BF16, or act MOE_BF16 with weight
 *   MOE_MXFP4 for decode batches (T * k < 48 * E, the batches whose experts
 *   hold a few rows); d % 32 == 0, and for the calls that run the expert
 *   GEMMs (gate/up, down, expert_ffn, forward and their workspace sizes)
 *   also d % 256 == 0 and F % 128 == 0; 0 <= T and
 *   T * (k + S) * max(d, F) < 2^40, T * k < 2^31.  Anything else is
 *   MOE_ERR_UNSUPPORTED (or MOE_ERR_SHAPE for negative sizes, MOE_ERR_DTYPE
 *   for other dtype pairs).  With S = 0 the shared-expert pointers
 *   (ws_gate, ws_up, ws_down, y_shared) may be NULL.
 *
 * Intermediate layouts shared between calls:
 * - pair p = t * k + j is token t's slot-j routed choice (rank order).
 * - topk_idx  int32 [T, k]   routed expert ids in rank order (descending
 *                            s + b, exact ties to the lower id).
 * - gates     fp32  [T, k+S] slots 0..k-1 the routed experts in rank order,
 *                            slots k..k+S-1 the shared experts.
 * - counts    int32 [E]      L_e, routed selections per expert (the demand,
 *                            before any capacity limit).
 * - offsets   int32 [E+1]    exclusive prefix sum of the kept rows per
 *                            expert, min(L_e, C) (C below; L_e when there is
 *                            no capacity limit).
 * - sorted_pair int32 [T*k]  the kept pair numbers grouped by expert,
 *                            ascending p inside each expert; entries from
 *                            offsets[E] on are unspecified.
 * - pair_pos  int32 [T*k]    pair p sits at row pair_pos[p] of the
 *                            expert-sorted buffers, or -1 if it was dropped.
 * - h         act   [(k+S)*T, F]  SwiGLU activations: rows 0..T*k-1 routed
 *                            in sorted order, row k*T + s*T + t shared s.
 * - y_routed  act   [T*k, d] expert outputs in sorted order;
 *   y_shared  act   [S, T, d] shared-expert outputs.
 * These tables live in device memory and no call checks their contents:
 * the expert calls and combine take them as moe_dispatch wrote them
 * (offsets non-decreasing from 0 to at most T*k; sorted_pair entries below
 * offsets[E] in [0, T*k); pair_pos entries -1 or below offsets[E]).  Other
 * contents give undefined results and may make the kernels read or write
 * outside the buffers.
 *
 * Capacity ("Inkling, Dissected" 02d: each expert takes a bounded number
 * of tokens per batch; pairs beyond it are dropped and the output is built
 * from the pairs that were kept).  With capacity_factor
 * cf > 0 each routed expert keeps C = ceil(cf * k * T / E) pairs (the
 * product and quotient taken in double precision), the first C in
 * ascending pair number, i.e. ascending token; a dropped pair contributes
 * nothing to y (the other gates are not renormalised).  Shared experts have
 * no limit.  cf = 0 means no limit (dropless).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 4: MXFP4 codes and scales stored by 128-value K tile (see
 * moe_quantize_mxfp4) */
#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                 */
  MOE_ERR_SHAPE = 2,       /* negative size, non-finite gamma, or a bad
                              gate_norm, gate_scale or capacity_factor */
  MOE_ERR_DTYPE = 3,       /* unknown dtype or dtype pair                */
  MOE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required    */
  MOE_ERR_UNSUPPORTED = 5, /* valid but outside the supported shapes     */
  MOE_ERR_HIP = 6          /* a kernel launch failed                     */
} moe_status;

/* MOE_MXFP4 is a weight format only (moe_desc.weight): the routed experts'
 * matrices in FP4 with block scales (see moe_quantize_mxfp4); the shared
 * experts stay in the act dtype. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype;

/* Which call a workspace size is asked for. */
typedef enum {
  MOE_CALL_ROUTER = 0,
  MOE_CALL_DISPATCH = 1,
  MOE_CALL_GATE_UP = 2,
  MOE_CALL_DOWN = 3,
  MOE_CALL_EXPERT_FFN = 4,
  MOE_CALL_COMBINE = 5,
  MOE_CALL_BIAS_UPDATE = 6,
  MOE_CALL_FORWARD = 7
} moe_call;

/* How the gates of the k kept routed experts and the S shared experts are
 * normalised (the top-k selection is the same for both):
 *   MOE_GATE_RATIO      g_j = s_j / sum_i s_i over the k + S contributors,
 *                       s = sigmoid(z) ("Inkling, Dissected", 02b);
 *   MOE_GATE_LOGSUMEXP  g_j = exp(logsigmoid(z_j) - logsumexp_i logsigmoid(z_i))
 *                       over the same set ("Under The Hood: Inkling", the
 *                       routing strategy: log-sigmoid, then logsumexp over
 *                       the joint set of 8).
 * Both equal each other in exact arithmetic; they differ in rounding only.
 * Either is then multiplied by gate_scale (1 for the first page's layer;
 * route_scale * global_scale, e.g. 8.0 times the learned scalar, for the
 * second page's configuration). */
typedef enum { MOE_GATE_RATIO = 0, MOE_GATE_LOGSUMEXP = 1 } moe_gate_norm;

/* Layer shape.  T tokens, hidden d, expert ffn width F, E routed experts,
 * S shared experts, k routed experts per token; act is the dtype of x, h,
 * y and the expert weights, weight must equal act.  The router weights and
 * the bias are always fp32.  gate_norm and gate_scale (finite, > 0) set the
 * gate normalisation above; capacity_factor the per-expert capacity. */
typedef struct {
  int32_t T, d, F, E, S, k;
  moe_dtype act, weight;
  int32_t gate_norm;  /* moe_gate_norm */
  float gate_scale;
  float capacity_factor;  /* 0: no limit; else > 0 and finite (see above) */
} moe_desc;

/* Weights of one layer.  Expert matrices are [out, in] row-major:
 *   w_router [E+S, d] fp32  (rows E.. are the shared experts' vectors)
 *   w_gate, w_up [E, F, d]   w_down [E, d, F]        (act dtype)
 *   ws_gate, ws_up [S, F, d] ws_down [S, d, F]       (act dtype)
 * With weight == MOE_MXFP4 the routed matrices are the outputs of
 * moe_quantize_mxfp4: w_gate, w_up [E, d/128, F, 64] and w_down
 * [E, F/128, d, 64] bytes of packed FP4 codes, and sc_gate, sc_up
 * [E, d/128, F, 4], sc_down [E, F/128, d, 4] their scale bytes (NULL
 * otherwise).
 * w_router_planes (optional, may be NULL): the output of moe_router_prepare
 * for this w_router; moe_forward then routes with it instead of splitting
 * w_router again on every call.  It must be refreshed whenever w_router
 * changes. */
typedef struct {
  const float* w_router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* ws_gate;
  const void* ws_up;
  const void* ws_down;
  const uint8_t* sc_gate;
  const uint8_t* sc_up;
  const uint8_t* sc_down;
  const uint16_t* w_router_planes;
} moe_weights;

/* Optional routing outputs of moe_forward: each pointer may be NULL, in
 * which case that tensor lives in the workspace. */
typedef struct {
  int32_t* topk_idx;     /* [T, k]   */
  float* gates;          /* [T, k+S] */
  float* margin;         /* [T] s+b of the k-th minus the (k+1)-th choice */
  int32_t* counts;       /* [E]      */
  int32_t* offsets;      /* [E+1]    */
  int32_t* sorted_pair;  /* [T*k]    */
  int32_t* pair_pos;     /* [T*k]    */
} moe_routing;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static description of a status code; never NULL. */
const char* moe_status_string(moe_status status);

/* Device workspace bytes needed by `call` for this shape (0 when none).
 * Returns the same validation errors as the call itself. */
moe_status moe_workspace_size(const moe_desc* desc, moe_call call, size_t* bytes);

/* Router ("Inkling, Dissected" 02b; "Under The Hood", routing strategy).
 *   x [T, d] act, w_router [E+S, d] fp32, bias [E] fp32.
 *   z = x . w_router^T: w_router is split exactly into three bf16 planes,
 *   the products run on the bf16 matrix cores (exact in fp32), each
 *   32-element K step starts a fresh fp32 accumulator that is then added to
 *   an fp64 running sum.  s = sigmoid(z), the selection keys s + b, the
 *   top-k (rank order, exact ties to the lower id) and the gates are taken
 *   in fp64.  Writes topk_idx [T, k], gates [T, k+S] and, when non-NULL,
 *   margin [T] (key of the k-th minus the (k+1)-th choice). */
moe_status moe_router(const moe_desc* desc, const void* x, const float* w_router,
                      const float* bias, int32_t* topk_idx, float* gates,
                      float* margin_or_null, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* The router's split of w_router into bf16 planes, once per weights
 * ("Inkling, Dissected" 02b: the router scores every token against each
 * expert's vector; the vectors change only when the weights do).
 *   planes [3, P, d] bf16 bits, P = E+S rounded up to a multiple of 64:
 *   plane 0 = bf16(w), plane 1 = bf16(w - plane 0), plane 2 = bf16(w -
 *   plane 0 - plane 1), rounding to nearest even: the exact split that
 *   moe_router makes on every call; rows E+S.. are zero.
 * moe_router_planes_size gives the bytes of planes for a shape (the same
 * validation errors as moe_router; T may be 0).  moe_router_prepare writes
 * them on `stream` from w_router [E+S, d] fp32; the caller owns planes and
 * passes it as moe_weights.w_router_planes.  It needs no workspace. */
moe_status moe_router_planes_size(const moe_desc* desc, size_t* bytes);
moe_status moe_router_prepare(const moe_desc* desc, const float* w_router, uint16_t* planes,
                              hipStream_t stream);

/* Dispatch: group the T*k (token, slot) pairs by expert ("Inkling,
 * Dissected" 02: each token visits its 6 chosen experts; 02e: L_e is the
 * number of tokens that selected e), keeping at most C pairs per expert
 * when the descriptor sets a capacity.  Histogram -> exclusive scan ->
 * stable scatter; deterministic.  Writes counts, offsets, sorted_pair and
 * pair_pos (layouts above). */
moe_status moe_dispatch(const moe_desc* desc, const int32_t* topk_idx,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Dispatch without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments (minus the workspace), results and
 * errors as moe_dispatch; its scratch (the per-segment expert counts,
 * ceil(T*k / 512) * E + 1 ints) lives in a 1 MiB device array the library
 * holds on each GPU it runs on until the process ends, so T * k may be at
 * most 523776 pairs at E = 256 (1048064 at E = 128, 2096640 at E = 64);
 * larger batches return MOE_ERR_UNSUPPORTED before anything launches.  The
 * first call on a device looks the array up there (MOE_ERR_HIP if that
 * fails).  The call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different host threads without ordering) race. */
moe_status moe_dispatch_noalloc(const moe_desc* desc, const int32_t* topk_idx,
                                int32_t* counts, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos,
                                hipStream_t stream);

/* Gate/up half of every expert ("Under The Hood", expert configuration:
 * SwiGLU experts): h = silu(X W_gate^T) * (X W_up^T), X the rows of x
 * routed to the expert (rows gathered through sorted_pair) or all of x for
 * a shared expert.  Matrix cores, fp32 accumulation, h rounded to act.
 * Writes h [(k+S)*T, F]. */
moe_status moe_expert_gate_up(const moe_desc* desc, const void* x,
                              const moe_weights* w, const int32_t* offsets,
                              const int32_t* sorted_pair, void* h, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Down half of every expert ("Under The Hood", expert configuration: the
 * SwiGLU FFN's output projection; "Inkling, Dissected", 02: an expert's
 * second matrix product after the nonlinearity): y = h W_down^T per expert,
 * matrix cores, fp32 accumulation, rounded to act.  Reads h [(k+S)*T, F]
 * (routed rows in expert-sorted order, then each shared expert's T rows);
 * writes y_routed [T*k, d] (sorted order) and y_shared [S, T, d]. */
moe_status moe_expert_down(const moe_desc* desc, const moe_weights* w,
                           const int32_t* offsets, const void* h,
                           void* y_routed, void* y_shared, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Profiling variants of the two calls above, for timing their kernels
 * with events on the caller's stream.  Same arguments, results and
 * workspace; in addition marks[0] is recorded after the tile-plan kernel
 * and marks[1] after the GEMM kernel.  marks[0..1] must be valid events
 * (MOE_ERR_NULL otherwise). */
moe_status moe_expert_gate_up_marked(const moe_desc* desc, const void* x,
                                     const moe_weights* w, const int32_t* offsets,
                                     const int32_t* sorted_pair, void* h, void* ws,
                                     size_t ws_bytes, hipEvent_t* marks,
                                     hipStream_t stream);
moe_status moe_expert_down_marked(const moe_desc* desc, const moe_weights* w,
                                  const int32_t* offsets, const void* h,
                                  void* y_routed, void* y_shared, void* ws,
                                  size_t ws_bytes, hipEvent_t* marks,
                                  hipStream_t stream);

/* Every expert's whole FFN ("Under The Hood", expert configuration:
 * y_e = W_down (silu(W_gate x) * W_up x) for each routed expert on the
 * tokens dispatched to it and each shared expert on every token;
 * "Inkling, Dissected", 02: each token visits its 6 routed experts and the
 * 2 shared ones): moe_expert_gate_up then moe_expert_down, h in the
 * workspace.  Same inputs and outputs as the two calls. */
moe_status moe_expert_ffn(const moe_desc* desc, const void* x,
                          const moe_weights* w, const int32_t* offsets,
                          const int32_t* sorted_pair, void* y_routed,
                          void* y_shared, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Combine ("Inkling, Dissected" 02b: the gate-weighted sum over the 8
 * contributors).  y[t] = sum_j gates[t,j] * y_routed[pair_pos[t*k+j]]
 * (j = 0..k-1 in rank order, skipping dropped pairs, pair_pos < 0) +
 * sum_s gates[t,k+s] * y_shared[s,t], in fp32 in exactly that order,
 * rounded once to act.  Writes y [T, d]. */
moe_status moe_combine(const moe_desc* desc, const void* y_routed,
                       const void* y_shared, const float* gates,
                       const int32_t* pair_pos, void* y, hipStream_t stream);

/* Balancing-bias update ("Inkling, Dissected" 02e):
 * bias[e] += gamma * sign(k*T - E*counts[e]) in fp32 (sign(0) = 0; the
 * comparison is exact integer arithmetic).  gamma must be finite. */
moe_status moe_bias_update(const moe_desc* desc, const int32_t* counts,
                           float gamma, float* bias, hipStream_t stream);

/* FP4 expert weights ("Under The Hood: Inkling", "Quantization: BF16 vs
 * NVFP4": FP4 weights with small-block scales for the routed experts only).
 * MI355X's own FP4 format is used, OCP MXFP4: E2M1 values with one
 * power-of-two scale per 32 consecutive values along K.  For each block
 * with largest magnitude a: X = floor(log2 a) - 2, clamped to [-127, 127]
 * (-127 when a = 0); each value v becomes the E2M1 magnitude nearest to
 * |v| / 2^X (ties to the even code; above 6 saturates to 6) with v's sign
 * as bit 3.  Quantizes a bf16 stack w [E, N, K] (K % 128 == 0, else
 * MOE_ERR_SHAPE) into codes [E, K/128, N, 64]: for each 128-value K tile,
 * the 64 code bytes of every row n, rows consecutive (value 2i of the tile
 * in the low nibble of byte i), and scales [E, K/128, N, 4]: for each K
 * tile, the bytes X + 127 of its 4 blocks for every row n, rows
 * consecutive.  They are E * N * K/2 and E * N * K/32 bytes.  Device pointers;
 * asynchronous. */
moe_status moe_quantize_mxfp4(int32_t E, int32_t N, int32_t K, const void* w,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* The whole layer ("Inkling, Dissected", 02b: the per-token sketch of
 * router, top-6, joint gates and the weighted sum of the 8 experts' outputs;
 * 02e: the bias moves once the batch is done): router (with the incoming
 * bias), dispatch, expert FFN, combine, and the bias update in place from
 * this batch's loads (the next batch routes with the new bias; gamma == 0
 * leaves it unchanged).  The update is applied once the router has read
 * the bias: for batches of at most 4096 (token, slot) pairs routed to
 * 32-row tiles it runs in the dispatch launch, otherwise after the combine.
 * Writes y [T, d] and, when `routing` is non-NULL, its non-NULL members
 * (the tensors a caller wants to keep; the others live in the workspace). */
moe_status moe_forward(const moe_desc* desc, const void* x,
                       const moe_weights* w, float* bias, float gamma, void* y,
                       const moe_routing* routing_or_null, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Profiling variant of moe_forward, for timing its stages and GEMM kernels
 * with events on the caller's stream inside a timed run of the layer.
 * Same arguments, results and workspace; in addition marks[0..6] are
 * recorded after the router, the dispatch, the GEMMs' tile plan, the
 * gate/up GEMM, the down GEMM, the combine and the bias update (marks[6]
 * also when gamma == 0).  Where the dispatch launch also writes the tile
 * plan and applies the bias update (small batches, see moe_forward),
 * marks[2] follows marks[1] and marks[6] follows marks[5] directly.
 * marks[0..6] must be valid events (MOE_ERR_NULL otherwise). */
moe_status moe_forward_marked(const moe_desc* desc, const void* x,
                              const moe_weights* w, float* bias, float gamma,
                              void* y, const moe_routing* routing_or_null,
                              void* ws, size_t ws_bytes, hipEvent_t* marks,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
