/*
 * edge0.h - C ABI of the MI355X (gfx950) streaming-MoE decode path.
 *
 * Sources (cited by page title and section):
 *   [Edge0]     "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
 *               with Trained Routing Prediction" (arXiv HTML).
 *   [Review]    "Waking the MoE on SSD: Serving a 35B MoE at 20 tok/s on a
 *               24 GB Desktop with Edge0" (jaehun.me review of the paper).
 *   [Cacheable] "Cacheable by Design?" (arXiv 2608.18261).
 *
 * One decode step of one streaming MoE layer: a per-layer prerouter head
 * predicts the next layer's routing one token ahead ([Edge0] §3.2 "Head",
 * "Prediction-as-routing"), a softmax-top-K commits it ([Edge0] App. A), the
 * int4 group-quantised experts named by the routing are dequantised from a
 * pool of slots in HBM and run as SwiGLU FFNs with an unmerged LoRA delta
 * ([Edge0] §3.1 "Math contract", §3.3), and the outputs are combined with
 * the routing weights.  Staging copies predicted experts into slots ahead of
 * use ([Edge0] Figure 1, §3.1 "Executor paths").
 *
 * Conventions for every call
 *   - Pointers marked "device" are device memory on the current HIP device;
 *     "host" pointers are host memory.  The library never allocates, frees
 *     or retains caller memory, except inside the opaque handles
 *     (edge0_stack, edge0_stager) which own what their create call says.
 *   - Kernels are enqueued on the given stream (NULL = the null stream); a
 *     call returns once its work is enqueued, and outputs are valid when the
 *     stream reaches that point.
 *   - bf16 and fp16 are passed as their 16-bit patterns; fp32 as float.
 *   - Return value: EDGE0_OK (0) or a negative EDGE0_E* code.  No C++
 *     exception crosses the ABI.  Arguments are checked before anything is
 *     enqueued; on an error return nothing was enqueued.
 *   - Device-side checks: an expert id outside [0, E) or a slot outside
 *     [0, n_slots) met by a kernel is not dereferenced; that expert's
 *     contribution is skipped and EDGE0_ERANGE is recorded in the workspace
 *     error word (edge0_workspace_error reads and clears it).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef EDGE0_H
#define EDGE0_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EDGE0_OK = 0,
  EDGE0_EINVAL = -1,   /* NULL required pointer, unsupported shape or argument */
  EDGE0_EHIP = -2,     /* a HIP runtime or launch error */
  EDGE0_ENOSLOT = -3,  /* every slot of the pool is pinned by pending sets */
  EDGE0_ERANGE = -4,   /* an expert id or slot index out of range */
  EDGE0_ENOMEM = -5,   /* an allocation owned by a handle failed */
  EDGE0_ESCRATCH = -6  /* the shape needs more scratch than the static workspace holds */
};

/* Returns a static string describing an EDGE0_* code. */
const char* edge0_strerror(int code);

/* -------------------------------------------------------------------------
 * Model description ([Edge0] §3 "System Design": one spec per model with
 * expert count, K, routing family, quantisation and weight layout).
 *
 * Supported values: d_model % 64 == 0 and d_model / 32 in {8, 16, 32} or a
 * multiple of 64; d_inter % 64 == 0; group_size % 32 == 0 dividing both
 * d_model and d_inter; 1 <= top_k <= min(16, n_experts); n_experts <= 1024;
 * lora_rank in {0, 8, 16, 32, 64}; head_hidden % 64 == 0 (or 0 when no head
 * is used).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t d_model;      /* d: hidden size */
  int32_t n_experts;    /* E: routed experts per layer */
  int32_t d_inter;      /* I: expert intermediate size */
  int32_t top_k;        /* K: experts per token */
  int32_t group_size;   /* g: int4 quantisation group along the input axis */
  int32_t lora_rank;    /* r: recovery-LoRA rank, 0 = no adapter */
  float lora_alpha;     /* alpha: the delta is scaled by alpha / r */
  int32_t head_hidden;  /* H: prerouter fc1 width */
  int32_t routing;      /* routing family of the commit: EDGE0_ROUTE_* */
  int32_t n_groups;     /* sigmoid-group: n groups of E / n contiguous experts */
  int32_t top_groups;   /* sigmoid-group: G groups survive */
  float route_scale;    /* sigmoid-group: s, the K weights sum to s */
} edge0_moe_shape;

/* Routing families ([Edge0] §2 "MoE routing", App. A).  A zero-filled shape
 * is softmax-top-K; the sigmoid-group fields are read only for family 1,
 * which needs E % n == 0, E / n >= 2, n <= 64, 1 <= G <= n,
 * K <= G * E / n and a finite s.  The decode stack (edge0_stack_create)
 * takes softmax-top-K only. */
#define EDGE0_ROUTE_SOFTMAX_TOPK 0
#define EDGE0_ROUTE_SIGMOID_GROUP 1

/* -------------------------------------------------------------------------
 * Expert bundle = the content of one slot ([Edge0] §3.1 "Executor paths":
 * the nine arrays gate/up/down x weights/scales/biases; §3.3: the LoRA is
 * kept as separate low-rank factors, never merged).
 *
 * Dequantised weight: W[o][i] = s[o][i/g] * q[o][i] + b[o][i/g], q in 0..15
 * ([Edge0] §2 "Quantization": int4 affine, groups along the input axis).
 *
 * Device layout inside a bundle (every array starts on a 256-byte boundary):
 *   gate_q, up_q : u32 [I][d/8], row-major; input i of row o is the nibble
 *                  at bits 4*(i%8) of word o*(d/8) + i/8.
 *   down_q       : u32 tiled [d/64][I/32][64][4]: 1 KiB tile (rb, c) holds
 *                  rows 64*rb..64*rb+63, inputs 32*c..32*c+31; row o of the
 *                  tile is its 16 bytes at offset 16*(o%64), nibble order as
 *                  above within each word.
 *   gate_s/b, up_s/b : bf16 [I][d/g] row-major.
 *   down_s/b     : bf16 [I/g][d] (group-major: all rows of group 0 first).
 *   LoRA (lora_rank > 0), bf16: a_gate [r][d], b_gate [I][r], a_up [r][d],
 *                  b_up [I][r], a_down [r][I], b_down [d][r], row-major.
 * The logical (row-major [out][in/8] words, [out][in/g] scales) form is what
 * edge0_pack_bundle accepts.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b;
  int64_t a_gate, b_gate, a_up, b_up, a_down, b_down;  /* -1 when lora_rank == 0 */
  int64_t bytes;                                       /* total, multiple of 256 */
} edge0_bundle_layout;

/* Byte offsets of the arrays inside one bundle.  EDGE0_EINVAL for an
 * unsupported shape. */
int edge0_bundle_layout_of(const edge0_moe_shape* shape, edge0_bundle_layout* out);

/* Logical (row-major) expert arrays, all device pointers, as produced by a
 * checkpoint: *_q u32 [out][in/8], *_s and *_b bf16 [out][in/g]; gate and up
 * are [I x d], down is [d x I].  LoRA pointers may be NULL iff lora_rank == 0. */
typedef struct {
  const void *gate_q, *gate_s, *gate_b, *up_q, *up_s, *up_b, *down_q, *down_s, *down_b;
  const void *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;
} edge0_expert_arrays;

/* Writes one bundle in the device layout at bundle_dst (device, layout.bytes
 * bytes, 256-byte aligned) from the logical arrays.  Pure data movement (no
 * rounding); sources and destination must not overlap. */
int edge0_pack_bundle(const edge0_moe_shape* shape, const edge0_expert_arrays* src,
                      void* bundle_dst, hipStream_t stream);

/* Pool of staged slots in HBM: slot s occupies [base + s*slot_bytes,
 * base + s*slot_bytes + layout.bytes).  slot_bytes >= layout.bytes and a
 * multiple of 256. */
typedef struct {
  void* base;           /* device */
  int64_t slot_bytes;
  int32_t n_slots;
} edge0_slot_pool;

/* -------------------------------------------------------------------------
 * Workspace: scratch device memory for the single-layer calls below
 * (partial sums, LoRA factors, the SwiGLU activations, completion counters
 * and the error word).  The caller allocates edge0_workspace_bytes(shape)
 * bytes (256-byte aligned) and zero-fills them once before first use; the
 * calls leave the counters zero again.  Calls that may run concurrently
 * need distinct workspaces.
 * ---------------------------------------------------------------------- */
size_t edge0_workspace_bytes(const edge0_moe_shape* shape);

/* Waits for `stream`, then returns the workspace error word (EDGE0_OK or
 * EDGE0_ERANGE) and clears it. */
int edge0_workspace_error(void* workspace, hipStream_t stream);

/* -------------------------------------------------------------------------
 * The commit of a routing from logits l [E] ([Edge0] §2 "MoE routing",
 * App. A), by shape->routing:
 *  softmax-top-K ("Softmax-topk"): ids = the K largest logits in order
 *    (value descending, lower index first on ties); w_k = exp(l_k - l_max) /
 *    sum_{j in ids} exp(l_j - l_max), which equals g[ids]/sum g[ids] for
 *    g = softmax(l).
 *  sigmoid-group ("Sigmoid-group"): sigma = sigmoid(l); selection score
 *    c = sigma + route_bias (the bias is 0 when route_bias is NULL);
 *    group i = experts [i E/n, (i+1) E/n), scored by the sum of its two
 *    largest c; the G best groups survive (lower group first on ties);
 *    ids = the K largest c among their experts, in rank order (lower index
 *    first on ties); w_k = s * sigma[ids_k] / (sum_j sigma[ids_j] + 1e-20).
 *    The bias steers the choice only; the weights use the raw sigmoid.
 * Decisions are taken on fp32 scores; NaN ranks lowest.
 *   route_bias : device fp32 [E] or NULL (read by sigmoid-group only)
 *   ids_out    : device int32 [K];  w_out : device fp32 [K]
 * ---------------------------------------------------------------------- */

/* The commit alone, from device fp32 logits [E] (one wave; no workspace). */
int edge0_route_commit(const edge0_moe_shape* shape, const float* logits,
                       const float* route_bias, int32_t* ids_out, float* w_out,
                       hipStream_t stream);

/* Plain router: logits = W_r x (fp32 accumulation), then the commit above.
 *   w_router : device bf16 [E][d]
 *   x        : device bf16 [d]
 *   logits_out : device fp32 [E] or NULL
 * ---------------------------------------------------------------------- */
int edge0_router(const edge0_moe_shape* shape, const void* w_router, const float* route_bias,
                 const void* x, float* logits_out, int32_t* ids_out, float* w_out,
                 void* workspace, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Prerouter head and commit ([Edge0] §3.2 "Head", "Prediction-as-routing",
 * "Feature drift"; [Review] toy example).  The head owned by layer N runs
 * at token t on layer N's normalised hidden state and predicts layer N+1's
 * routing at token t+1:
 *   f      = [x ; onehot(ids_now) ; onehot(ids_prev)]        (d + 2E)
 *   z1     = fc1 f + b1,  a = 0.5 z1 (1 + erf(z1 / sqrt 2))   (H)
 *   logits = w2 a + b2 + wl x                                 (E)
 * then the same commit as edge0_router (shape->routing; route_bias is the
 * predicted layer's selection bias for sigmoid-group, or NULL: the
 * prediction is routed through the same math, [Edge0] §2 "MoE routing",
 * §3.2 "Prediction-as-routing").  The one-hot blocks hold a 1
 * per routed expert (binary, not weighted); ids_now is the routing layer N
 * executed at token t, ids_prev the routing it executed at token t-1 (NULL
 * at the first decode token: that block is zero).
 * Head weights (fp16, device): fc1 is split into its hidden-state columns
 * w1x [H][d] and its one-hot columns stored transposed, w1oh [2E][H] (row e
 * is the column of expert e in this token's block, row E+e in the previous
 * token's block); b1 [H]; w2 [E][H]; b2 [E]; wl [E][d] (linear residual,
 * no bias).  b1, b2, wl may be NULL (zero).
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *w1x, *w1oh, *b1, *w2, *b2, *wl;
} edge0_head;

int edge0_prerouter(const edge0_moe_shape* shape, const edge0_head* head,
                    const float* route_bias, const void* x,
                    const int32_t* ids_now, const int32_t* ids_prev,
                    float* logits_out, int32_t* ids_out, float* w_out,
                    void* workspace, hipStream_t stream);

/* -------------------------------------------------------------------------
 * One MoE layer over the committed experts ([Edge0] §3.1 "Math contract",
 * §3.3; Figure 1 sum node):
 *   for each k:  e = ids[k], slot = slot_table[e]
 *     G = gate(x) + (a/r) B_gate (A_gate x),  U = up(x) + (a/r) B_up (A_up x)
 *     h = silu(G) * U,                        silu(z) = z / (1 + e^-z)
 *     D_k = down(h) + (a/r) B_down (A_down h)
 *   y = bf16( sum_k w[k] D_k )   (fp32 throughout, one rounding at the end)
 *   slot_table : device int32 [E], id -> slot ("take" through the slot
 *                table: indices stay on the device, [Edge0] §3.1)
 *   ids, w     : device int32 [K], fp32 [K]
 *   x, y       : device bf16 [d]; y must not alias x
 * ---------------------------------------------------------------------- */
int edge0_moe_layer(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                    const int32_t* slot_table, const int32_t* ids, const float* w,
                    const void* x, void* y, void* workspace, hipStream_t stream);

/* -------------------------------------------------------------------------
 * edge0_moe_layer without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * edge0_moe_layer, but the scratch (partial sums, LoRA factors, SwiGLU
 * activations, the fixed-point accumulator, the error word) is a static
 * device array of the library, EDGE0_STATIC_WORKSPACE_BYTES (1 MiB) per
 * GPU, which each GPU the library runs on holds until the process ends.
 * The call allocates and frees nothing.  Its first call on a device looks
 * up that device's copy of the array and zero-fills it with a kernel on
 * `stream`; calls leave it ready for the next.
 *   error_out : device int32 (may be NULL): receives EDGE0_OK, or
 *               EDGE0_ERANGE when an id or slot was out of range (that
 *               expert's contribution was skipped), once the stream
 *               reaches the end of the call.
 * Returns EDGE0_ESCRATCH (nothing enqueued) when the shape's workspace
 * (edge0_workspace_bytes) exceeds the static array.  Every call on one GPU
 * shares its array: calls that may overlap on one GPU (several streams or
 * threads) race and must be serialised by the caller.
 * ---------------------------------------------------------------------- */
#define EDGE0_STATIC_WORKSPACE_BYTES ((size_t)1 << 20)
int edge0_moe_layer_noalloc(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                            const int32_t* slot_table, const int32_t* ids, const float* w,
                            const void* x, void* y, int32_t* error_out, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Several tokens through one MoE layer, grouped by expert.  Defined token by
 * token exactly as edge0_moe_layer: for token j with routing ids[j][.],
 * w[j][.],  y[j] = bf16( sum_k w[j][k] D_{ids[j][k]}(x[j]) )  ([Edge0] §3.1
 * "Math contract", §3.3); the grouping only reorders the work.  The (token,
 * k) pairs are bucketed by expert on the device (counting sort, stable by
 * token; an id repeated within a token's routing is kept once with the
 * repeats' weights added).  From 3 tokens per call on, every expert's
 * products run on MFMA in tiles of up to 16 of its tokens (bf16 operands
 * holding the exact 128 + q nibble values and the activations, fp32
 * accumulation, the group affine applied per group in fp32); smaller calls
 * run multi-token GEMVs (at most 8 of an expert's tokens per workgroup).
 *   n_tokens   : 0..64 (0: nothing is enqueued)
 *   slot_table : device int32 [E], id -> slot
 *   ids, w     : device int32 / fp32 [n_tokens][K]
 *   x, y       : device bf16 [n_tokens][d]; y must not alias x
 *   workspace  : edge0_grouped_workspace_bytes(shape) bytes, zero-filled once
 *                before first use (calls leave it ready for the next call);
 *                calls that may run concurrently need distinct workspaces
 *   flags      : 0 (as above); EDGE0_GROUPED_NO_MFMA: every expert as
 *                GEMVs; EDGE0_GROUPED_MFMA_MIN(n) (1 <= n <= 255): experts
 *                chosen by >= n tokens on MFMA, the others as GEMVs.  Shapes
 *                outside the MFMA tiles' (d_model <= 2048 and a multiple of
 *                8 g, g of 32 or 64, d_inter a multiple of 128, even
 *                lora_rank <= 16) always run as GEMVs.
 * Supported shapes: those of edge0_moe_layer with d_inter <= 1024 and
 * d_model <= 4096 (edge0_grouped_workspace_bytes returns 0 otherwise). */
enum { EDGE0_GROUPED_NO_MFMA = 1 };
#define EDGE0_GROUPED_MFMA_MIN(n) (((n) & 0xFF) << 8)
size_t edge0_grouped_workspace_bytes(const edge0_moe_shape* shape);
int edge0_moe_grouped(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                      const int32_t* slot_table, int32_t n_tokens, const int32_t* ids,
                      const float* w, const void* x, void* y, void* workspace, int32_t flags,
                      hipStream_t stream);

/* -------------------------------------------------------------------------
 * The same layer with the recovery LoRA given apart from the bundles
 * ([Edge0] §3.3: the adapters ship as files beside the base weights, so a
 * new adapter generation swaps files, not bundles).  Six bf16 factors per
 * expert, row-major as in the bundle (a_gate [r][d], b_gate [I][r], a_up
 * [r][d], b_up [I][r], a_down [r][I], b_down [d][r]); each pointer is expert
 * 0's factor and expert e's is expert_stride * e elements further on.
 * expert_stride = 0: one adapter shared by every expert.  The slot pool may
 * then hold bundles in the LoRA-free layout (edge0_bundle_layout_of with
 * lora_rank 0; the int4 arrays are at the same offsets either way).
 * Results are those of edge0_moe_layer with the same adapters in the
 * bundles, bit for bit.  lora may be NULL when lora_rank == 0. */
typedef struct {
  const void *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;  /* device, bf16 */
  int64_t expert_stride;                                        /* elements */
} edge0_lora;
int edge0_moe_layer_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                         const edge0_lora* lora, const int32_t* slot_table, const int32_t* ids,
                         const float* w, const void* x, void* y, void* workspace,
                         hipStream_t stream);

/* -------------------------------------------------------------------------
 * Whole-layer prefill ([Edge0] §3.1 "Executor paths", whole-layer; §3.2
 * "Two consumption profiles": prefill takes every expert of a layer, and
 * there is nothing to predict).  The result is edge0_moe_grouped's, token by
 * token (an id repeated within a token's routing is kept once, its weights
 * summed in k order), for up to 4096 tokens per call: the (token, k) pairs
 * are bucketed by expert over many workgroups into tiles of up to 64 pairs
 * of one expert, which run through LDS-staged GEMMs on bf16 MFMA (int4
 * weights as exact 128 + q; each group's scale applied in fp32 per group,
 * the groups' (b - 128 s) terms against the per-group activation sums on
 * MFMA to fp32 precision; the LoRA terms on MFMA with t as bf16 hi + lo);
 * each pair's weighted row is stored
 * and every token's K rows are added in k order (calls are
 * bit-reproducible).
 *   slot_table, ids, w, x, y : as edge0_moe_grouped ([n_tokens][K] routing,
 *                [n_tokens][d] bf16 in and out; y must not alias x)
 *   max_tokens : the token bound the workspace was sized for
 *                (1 <= max_tokens <= 4096, n_tokens <= max_tokens)
 *   workspace  : edge0_prefill_workspace_bytes(shape, max_tokens) bytes,
 *                zero-filled once before first use (calls leave it ready)
 * Shapes: those of edge0_moe_grouped with g of 32 or 64, d_model <= 2048 and
 * a multiple of 128 and of 4 g, d_inter a multiple of 64 with at most 32
 * groups (d_inter / g <= 32), lora_rank <= 16; EDGE0_EINVAL otherwise.  An id or slot out of range is recorded in the
 * workspace error word (edge0_workspace_error) and its pair contributes
 * nothing. */
size_t edge0_prefill_workspace_bytes(const edge0_moe_shape* shape, int32_t max_tokens);
int edge0_moe_prefill(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                      const int32_t* slot_table, int32_t n_tokens, const int32_t* ids,
                      const float* w, const void* x, void* y, void* workspace,
                      int32_t max_tokens, hipStream_t stream);

/* The grouped and the prefill call with the recovery LoRA given apart from
 * the bundles ([Edge0] §3.3), as edge0_moe_layer_lora: the six bf16 factors
 * of expert 0 and the expert stride in elements (0: one adapter shared by
 * every expert); the pool may hold LoRA-free bundles.  Results are those of
 * edge0_moe_grouped / edge0_moe_prefill with the same adapters in the
 * bundles, bit for bit.  lora may be NULL only when lora_rank == 0;
 * EDGE0_EINVAL for a NULL factor or a negative stride. */
int edge0_moe_grouped_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                           const edge0_lora* lora, const int32_t* slot_table, int32_t n_tokens,
                           const int32_t* ids, const float* w, const void* x, void* y,
                           void* workspace, int32_t flags, hipStream_t stream);
int edge0_moe_prefill_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                           const edge0_lora* lora, const int32_t* slot_table, int32_t n_tokens,
                           const int32_t* ids, const float* w, const void* x, void* y,
                           void* workspace, int32_t max_tokens, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Merge-and-requantise, the measurement behind keeping the LoRA unmerged
 * ([Edge0] §3.3 "Recovery LoRA: Unmerged by Design" and its footnote 2).
 * For each projection of one expert: W' = s q + b + (alpha/r) B A, then per
 * group of g inputs s' = bf16((max - min) / 15), b' = bf16(min) (nearest,
 * ties to even), q' = round((w' - b') / s') to nearest-even, clipped to
 * 0..15 (0 where s' is 0).
 *   src_bundle : device, one expert bundle of `shape` (with its LoRA)
 *   dst_bundle : device, written in the LoRA-free layout of the same shape
 *                (edge0_bundle_layout_of with lora_rank 0): the merged expert
 *   stats_out  : device double [6]: sum(actual * delta), sum(delta^2) for
 *                gate, up, down, actual = s' q' + b' - (s q + b); the weight
 *                retention of a projection is the first over the second
 *   workspace  : edge0_merge_workspace_bytes(shape) bytes (partial sums);
 *                calls that share a workspace must not overlap
 * The sums are reduced in a fixed order (the same bits every call).  On the
 * GPU, delta is an fp32 sum of the exact bf16 products (on the matrix cores
 * for groups of up to 128 inputs), and q' is decided from (w' - b') times the
 * fp32 reciprocal of s'. */
size_t edge0_merge_workspace_bytes(const edge0_moe_shape* shape);
int edge0_merge_requant(const edge0_moe_shape* shape, const void* src_bundle, void* dst_bundle,
                        double* stats_out, void* workspace, hipStream_t stream);

/* -------------------------------------------------------------------------
 * Decode stack: n_layers pre-norm residual MoE blocks (no attention),
 *   x_L = bf16(RMSNorm(h_L)),  RMSNorm(h) = h / sqrt(mean(h^2) + eps)
 *   routing_L = committed prediction (consumer layers, step > 0) or the
 *               plain router (every other layer, and every layer at step 0)
 *   y_L = edge0_moe_layer(x_L),  h_{L+1} = bf16(h_L + y_L)
 *   heads of owner layers predict (L+1, step+1) from x_L, the ids layer L
 *   executed now and at the previous step ([Edge0] §3.2 "Head",
 *   "Motivation": double shift, one token of lead).
 * The handle owns its routing state, per-layer buffers and workspace.
 * Weights stay caller-owned and must outlive the handle.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_layers;
  int32_t owner_first, owner_last;        /* heads run at layers [first, last] */
  int32_t consumer_first, consumer_last;  /* layers routed by predictions     */
  float rms_eps;
} edge0_stack_spec;

typedef struct edge0_stack edge0_stack;

/* slot_tables : device int32 [n_layers][E]
 * routers     : host array [n_layers] of device bf16 [E][d] (entries of
 *               consumer layers are still used at step 0)
 * heads       : host array [n_layers]; entries of owner layers are used
 * Every owner L must have L+1 a consumer and vice versa; at most 48 owners,
 * and either all owner heads have the linear residual (wl) or none.  The
 * heads of a step run as one batch after its last layer: the predictions
 * are consumed at the next step ("one flush per step"). */
int edge0_stack_create(edge0_stack** out, const edge0_moe_shape* shape,
                       const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                       const int32_t* slot_tables, const void* const* routers,
                       const edge0_head* heads);
/* The same stack with each layer's recovery LoRA given apart from the
 * bundles ([Edge0] §3.3: a new adapter generation swaps files, not bundles):
 * layer_loras is a host array [n_layers] of edge0_lora (layer L's six
 * factor pointers of expert 0 and the expert stride, 0 = one adapter for
 * every expert of the layer), copied into the handle; the pointed-to
 * factors stay caller-owned.  The pool, and a stager's host bundles, may
 * hold LoRA-free bundles (edge0_bundle_layout_of with lora_rank 0), which
 * also makes every staged bundle smaller.  Results are those of
 * edge0_stack_create with the same adapters in the bundles, bit for bit.
 * Only the EDGE0_STACK_GRAPHS mode runs such a stack (edge0_stack_set_mode
 * refuses the others with EDGE0_EINVAL).  layer_loras may be NULL only when
 * lora_rank == 0; EDGE0_EINVAL for a NULL factor or a negative stride. */
int edge0_stack_create_lora(edge0_stack** out, const edge0_moe_shape* shape,
                            const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                            const int32_t* slot_tables, const void* const* routers,
                            const edge0_head* heads, const edge0_lora* layer_loras);

/* Runs decode step `step` (0, 1, 2, ... in order) on h0 (device bf16 [d]),
 * writing the final hidden state to h_out (device bf16 [d]).  Uses a HIP
 * graph of the step's launches after the first call of each step parity. */
int edge0_stack_step(edge0_stack* st, const void* h0, void* h_out, int32_t step,
                     hipStream_t stream);

/* Device pointers to the handle's per-layer results of the last step:
 *   x : bf16 [n_layers][d]   (normalised inputs)
 *   y : bf16 [n_layers][d]   (layer outputs)
 *   h : bf16 [n_layers+1][d] (h[0] = h0, h[L+1] after layer L)
 *   ids, w : int32/fp32 [n_layers][K] (routing each layer executed)
 *   pred_ids, pred_w : int32/fp32 [n_layers][K] (row L+1: the prediction
 *                head L made this step for the next step) */
typedef struct {
  const void *x, *y, *h;
  const int32_t* ids;
  const float* w;
  const int32_t* pred_ids;
  const float* pred_w;
} edge0_stack_buffers;
int edge0_stack_get_buffers(const edge0_stack* st, edge0_stack_buffers* out);
void edge0_stack_destroy(edge0_stack* st);

/* How edge0_stack_step runs the layers (the results are the same, within
 * the tolerance of fp32 summation order; the gathered routing runs as an
 * ordinary launch after the layers in every mode, and so do the heads except
 * under the folded head schedule below):
 *   EDGE0_STACK_GRAPHS (default): the step's per-layer launches, replayed as
 *     HIP graphs (two or three dependent launches per layer).
 *   EDGE0_STACK_PERSISTENT: one cooperative launch of K * d_inter / 16
 *     workgroups runs every layer.  The workgroups hand the layer input, h
 *     and the fixed-point y to each other through device-coherent memory,
 *     separated by grid-wide arrival counters, and each issues the loads of
 *     its next phase (consumer layers' experts are known from the previous
 *     step's predictions) before it waits ([Edge0] §3.2 "Prediction-as-
 *     routing": the routing is committed one token ahead).  Requires
 *     d_model 2048, n_experts <= 256, lora_rank 0, 8 or 16, top_k <= 16,
 *     d_inter % 32 == 0, d_model/64 dividing K * d_inter / 16 (and at least
 *     n_experts and 2 * top_k * lora_rank of them, and a multiple of 8),
 *     n_layers <= 48, and a device that can keep that
 *     many workgroups resident; otherwise EDGE0_EINVAL and the mode is
 *     unchanged.  Every wait is bounded (edge0_stack_set_spin_limit): a
 *     workgroup that waits longer records EDGE0_EHIP in the workspace error
 *     word and the launch ends early with incomplete results; the handle
 *     must then be destroyed.
 * EDGE0_EINVAL for another mode value. */
/*   EDGE0_STACK_XCD: one cooperative launch of 256 workgroups (32 per XCD)
 *     runs every layer with one grid-wide and one XCD-local hand-off per
 *     layer.  With K routed experts each XCD works on one expert of the
 *     routing (8/K XCDs share an expert, each a slice of its d_inter rows):
 *     its workgroups compute the gate/up rows of the slice (each with the
 *     expert's whole LoRA A x, from A rows held in registers), exchange the
 *     slice's SwiGLU activations within the XCD, and add the slice's down
 *     contribution (and its share of the LoRA-down delta) for 64 output rows
 *     each into the layer's fixed-point y.  Each register set of weights is
 *     reloaded for the next layer right after use: prediction-routed layers'
 *     experts are known when the step starts ([Edge0] §3.2
 *     "Prediction-as-routing").  Router layers share their logits within
 *     each XCD and load their experts after the top-K.  Requires d_model
 *     2048, top_k in {1, 2, 4, 8} with d_inter * top_k / 8 equal to 384 or
 *     768, n_experts <= 256, lora_rank 0, 8 or 16, n_layers <= 64 and a
 *     device that can keep 256 workgroups of 512 threads resident;
 *     otherwise EDGE0_EINVAL.  Waits are bounded as in the persistent mode.
 */
/*   EDGE0_STACK_XLAYER: the XCD split of EDGE0_STACK_XCD, one launch per
 *     layer, replayed as HIP graphs.  The kernel boundary hands y to the next
 *     layer (fixed-point atomics, exact and order-free); inside a launch the
 *     only hand-off is h within each XCD (and a router layer's logits).  A
 *     layer's experts are loaded as its launch starts: the slots of the
 *     predicted routing are resolved by a small kernel after the heads.  Same
 *     shape requirements as EDGE0_STACK_XCD; waits are bounded likewise.
 */
enum { EDGE0_STACK_GRAPHS = 0, EDGE0_STACK_PERSISTENT = 1, EDGE0_STACK_XCD = 2,
       EDGE0_STACK_XLAYER = 3 };
int edge0_stack_set_mode(edge0_stack* st, int32_t mode);
/* When the owner layers' heads run in a step of the EDGE0_STACK_GRAPHS mode
 * ([Edge0] §3.2 "Head": the heads' evaluation stays off the layers'
 * dependent chain; "Motivation": a head's prediction is consumed at the next
 * token, so nothing in the step waits for it):
 *   EDGE0_HEADS_AFTER_LAYERS (default): all heads as one batch (two
 *     launches: fc1 rows, then fc2 rows and the routing commits) after the
 *     last layer;
 *   EDGE0_HEADS_FOLDED: head L's fc1 rows run as workgroups appended to
 *     layer L's down-projection launch; the fc2 rows and commits stay one
 *     batch after the last layer.
 * The predictions are the same bit for bit either way (the same rows and
 * commit code over the same inputs).  The other modes and the staged step
 * run the heads after the layers whatever the setting.  Changing it waits
 * for the device and rebuilds the step graphs.  EDGE0_EINVAL for another
 * value. */
enum { EDGE0_HEADS_AFTER_LAYERS = 0, EDGE0_HEADS_FOLDED = 1 };
int edge0_stack_set_head_schedule(edge0_stack* st, int32_t schedule);
/* Polls per bounded wait before a workgroup gives up (0: the default, about
 * a second): the persistent mode's phase waits, and in the graphs mode the
 * gate/up workgroups' wait for their expert's LoRA A x, which workgroups of
 * the same launch compute.  A timed-out wait records EDGE0_EHIP (see
 * edge0_stack_error).  A failure-path aid; EDGE0_EINVAL for polls < 0. */
int edge0_stack_set_spin_limit(edge0_stack* st, int64_t polls);
/* Workspace error word of the handle (see edge0_workspace_error): the
 * recorded codes, cleared. */
int edge0_stack_error(edge0_stack* st);

/* Measurement aid: while kernel != 0, edge0_stack_step enqueues the step's
 * launches directly instead of replaying its graph, with a HIP event pair
 * around one launch class in every layer (kernel: 1 the gate/up GEMV, 2 the
 * down GEMV + combine, 3 the LoRA-in GEMV; 0 turns it off).  After a step,
 * edge0_stack_kernel_ms writes that launch's duration in ms for each layer
 * (up to cap values) and the count to *n.  In the persistent mode the one
 * layer launch of the step is bracketed and *n is 1. */
int edge0_stack_set_timing(edge0_stack* st, int32_t kernel);
/* Measurement aid of the EDGE0_STACK_XCD mode: while trace != NULL (device
 * uint64 [256][32]), every step's launch stores, per workgroup w, the
 * device's 100 MHz real-time clock at up to 32 points of layer `layer` to
 * trace[32 w + p] (0 layer start, 2 staged rows landed, 3 LoRA A x done,
 * 4 gate/up done, 5 h stored, 7 the XCD's h collected, 8 down done, 9 y
 * partial stored, 10 y rows stored, 11 y collected; 16-24 finer points of
 * the compute waves; 12 and 13 the shader clock counter at 0 and 11).
 * NULL turns it off. */
int edge0_stack_set_trace(edge0_stack* st, int32_t layer, uint64_t* trace);
int edge0_stack_kernel_ms(edge0_stack* st, float* ms_out, int32_t cap, int32_t* n);

/* -------------------------------------------------------------------------
 * Expert staging ([Edge0] Figure 1: bounded streaming pool with LRU
 * replacement and a staged fixed-slot double buffer; §3.1 "Executor paths":
 * experts are copied into slots and the kernels index them through the slot
 * table; §3.2 "Motivation": the next token's sets are known one token ahead,
 * so their reads overlap compute; Table 1 caption: one LRU of bundles shared
 * by all layers; [Cacheable] App. E: LRU replay).
 *
 * One pool of n_slots slots is shared by all layers.  A request names a
 * layer L, a step t and the set of expert ids layer L will use at step t.
 * Its ids are pinned from the request until edge0_*_release(L, t); then,
 * in order, a resident (L, id) is a hit, a missing one takes the lowest free
 * slot, else evicts the unpinned slot touched longest ago.  Every touched id
 * takes the next value of one global clock, so the choice is deterministic.
 * At most two sets of a layer (steps t and t+1) may be pending at once.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t requests;     /* sets requested */
  int64_t touches;      /* ids requested (hits + misses) */
  int64_t hits, misses;
  int64_t evictions;    /* misses that replaced a resident bundle */
  int64_t bytes_staged; /* host-to-device bytes enqueued (stager only) */
} edge0_stage_stats;

/* Host-only replacement policy (no device work), also used by the stager. */
typedef struct edge0_lru edge0_lru;
int edge0_lru_create(edge0_lru** out, int32_t n_slots, int32_t n_layers, int32_t n_experts);
/* ids: host int32 [n], distinct, each in [0, n_experts); n <= 16.
 * slots_out (host int32 [n]) receives each id's slot; hit_out (host int32
 * [n], may be NULL) 1 for a hit; evicted_out (host int32 [n], may be NULL)
 * the key L'*n_experts + e' whose bundle the miss replaced, or -1.
 * EDGE0_ENOSLOT (state unchanged) when the misses exceed the free and
 * unpinned slots; EDGE0_EINVAL for a bad id, a duplicate, or a set of
 * (layer, step) already pending. */
int edge0_lru_request(edge0_lru* lru, int32_t layer, int32_t step, const int32_t* ids,
                      int32_t n, int32_t* slots_out, int32_t* hit_out, int32_t* evicted_out);
/* Unpins the set of (layer, step); EDGE0_EINVAL if it is not pending. */
int edge0_lru_release(edge0_lru* lru, int32_t layer, int32_t step);
int edge0_lru_stats(const edge0_lru* lru, edge0_stage_stats* out);
void edge0_lru_destroy(edge0_lru* lru);

/* The stager: the same policy plus the data movement.
 *   pool         : the device slot pool (pool.slot_bytes >= the bundle
 *                  layout's bytes)
 *   host_bundles : host array [n_layers * n_experts]; entry L*E + e points to
 *                  the bundle of (L, e) in the device bundle layout, in pinned
 *                  host memory the device can read (hipHostMalloc), 16-byte
 *                  aligned, layout.bytes bytes; EDGE0_EINVAL otherwise.  The
 *                  memory must outlive the handle (the array is copied).
 *   slot_table   : device int32 [n_layers][n_experts]; the stager sets it to
 *                  -1 at create and keeps it equal to the pool's content
 *                  (id -> slot, -1 when not resident) as of the last wait or
 *                  flush on the compute stream.
 * The handle owns its policy state and HIP events (released by destroy). */
typedef struct edge0_stager edge0_stager;
int edge0_stager_create(edge0_stager** out, const edge0_moe_shape* shape,
                        const edge0_slot_pool* pool, int32_t n_layers,
                        const void* const* host_bundles, int32_t* slot_table);
/* Request (layer, step, ids) and enqueue on `stream` one copy kernel that
 * reads the missing bundles from host memory into their slots: on a side
 * stream this prefetches (the copies overlap whatever the compute stream
 * runs), on the compute stream it is a blocking on-demand fill.  The
 * slot-table update is queued for the compute stream (edge0_stager_wait).  A copy
 * into a slot that a layer read before first waits for that layer's
 * release point; a hit on a slot being filled on another stream waits for
 * that fill.  slots_out: host int32 [n] or NULL. */
int edge0_stage_experts(edge0_stager* sg, int32_t layer, int32_t step, const int32_t* ids,
                        int32_t n, int32_t* slots_out, hipStream_t stream);
/* Before the kernels that read the set of (layer, step): applies the
 * pending slot-table updates on compute_stream and makes it wait until the
 * set is in its slots (no event wait when it was staged on compute_stream
 * itself).  The slot table is written on the compute stream only. */
int edge0_stager_wait(edge0_stager* sg, int32_t layer, int32_t step, hipStream_t compute_stream);
/* -------------------------------------------------------------------------
 * Expert files: the SSD tier under the pinned host pool ([Edge0] §3.1
 * "Problem" and Figure 1: the weights live on the SSD, the page cache and the
 * staged slots above them; the checkpoint is stacked per layer, so a layer's
 * experts are direct reads).  One file per layer: a 4096-byte header (magic
 * "E0LAYER1", version 1, the layer, the expert count, bundle and record
 * bytes, the shape struct), then expert e's bundle in the device layout at
 * offset 4096 + e * record_bytes, zero-padded to record_bytes (a multiple of
 * 4096, so reads with O_DIRECT are aligned).
 * ---------------------------------------------------------------------- */
int64_t edge0_layer_file_record_bytes(const edge0_moe_shape* shape);
/* Writes layer `layer`'s file from E bundles (host-readable pointers, the
 * layout's bytes each).  EDGE0_EINVAL on an I/O error. */
int edge0_layer_file_write(const char* path, const edge0_moe_shape* shape, int32_t layer,
                           const void* const* bundles);

/* The open files of n_layers layers (paths[L] is layer L's file; each header
 * must name that layer and this shape), n_buffers pinned staging buffers of
 * one record each (16..4096; at least the misses of one request) and
 * n_threads I/O threads (1..64).  flags: EDGE0_FILE_DIRECT opens the files
 * with O_DIRECT (reads bypass the page cache), else reads go through it.
 * The handle must outlive every stager created on it. */
#define EDGE0_FILE_DIRECT 1
typedef struct edge0_filetier edge0_filetier;
typedef struct {
  int64_t reads;    /* records read */
  int64_t bytes;    /* bytes read */
  int64_t read_ns;  /* host time in read batches */
} edge0_file_stats;
int edge0_filetier_create(edge0_filetier** out, const edge0_moe_shape* shape, int32_t n_layers,
                          const char* const* paths, int32_t n_buffers, int32_t n_threads,
                          int32_t flags);
int edge0_filetier_stats(const edge0_filetier* ft, edge0_file_stats* out);
void edge0_filetier_destroy(edge0_filetier* ft);
/* A stager whose misses come from the layer files: a request's misses are
 * read in parallel (blocking the calling thread) into staging buffers, then
 * copied into their slots on the request's stream as edge0_stage_experts
 * copies host bundles (fill kernel or DMA); a staging buffer is reused once
 * the copy that last read it has completed.  Everything else is as
 * edge0_stager_create. */
int edge0_stager_create_files(edge0_stager** out, const edge0_moe_shape* shape,
                              const edge0_slot_pool* pool, int32_t n_layers,
                              edge0_filetier* files, int32_t* slot_table);

/* Applies the pending slot-table updates on compute_stream (the table then
 * maps every resident key once the stream reaches this point). */
int edge0_stager_flush(edge0_stager* sg, hipStream_t compute_stream);
/* Marks the point on compute_stream after the last kernel reading the set
 * of (layer, step) and unpins it: later copies into its slots wait for
 * that point. */
int edge0_stager_release(edge0_stager* sg, int32_t layer, int32_t step,
                         hipStream_t compute_stream);
/* How fills move bytes: EDGE0_COPY_KERNEL (default) - one kernel per
 * request reads the host bundles over the host link, so a fill on the
 * compute stream orders with the layer kernels without switching engines;
 * EDGE0_COPY_DMA - one hipMemcpyAsync per bundle on the DMA engines.  Same
 * results; EDGE0_EINVAL for another value. */
enum { EDGE0_COPY_KERNEL = 0, EDGE0_COPY_DMA = 1 };
int edge0_stager_set_copy_mode(edge0_stager* sg, int32_t mode);
int edge0_stager_stats(const edge0_stager* sg, edge0_stage_stats* out);
void edge0_stager_destroy(edge0_stager* sg);

/* One decode step of the stack over a staged pool.  With ahead = 0 or 1 the
 * routing ids of every layer are given (a routing trace): the weights are the softmax of the
 * layer's own logits taken at the given ids, w = g[ids] / sum g[ids]
 * ([Edge0] App. A), from the plain router of the layer or, for a
 * prediction-routed layer, from the logits its head produced at the
 * previous step.
 *   ahead = 1 (prediction arm): prediction-routed layers (step > 0) use sets
 *     staged one step ahead on copy_stream; every other layer runs its
 *     router, then fills its own set on demand on `stream`.  After the
 *     step's batched heads, the sets of the next step's prediction-routed
 *     layers (next_ids_host) are requested on copy_stream, which first
 *     waits for the heads ("one flush per step").
 *   ahead = 0 (on-demand arm): every layer runs its router and then fills
 *     its set on demand on `stream`; no heads run.
 *   ids_dev  : device int32 [n_layers][K], the routing of this step
 *   ids_host : host int32 [n_layers][K], the same ids
 *   next_ids_host : host int32 [n_layers][K], the routing of step + 1 (ahead
 *     = 1; NULL on the last step: nothing is prefetched)
 *   ahead = EDGE0_STAGE_LOOP (2, the closed loop of [Edge0] §3.2
 *     "Motivation" and "Prediction-as-routing"): no routing is given (ids_*
 *     may be NULL).  A router layer commits the softmax-top-K of its own
 *     router on the device; the host reads those K ids back (a wait on
 *     `stream`) and fills the set on demand.  A prediction-routed layer
 *     (step > 0) executes the routing its owner's head committed at the
 *     previous step, staged one step ahead.  After the batched heads the
 *     host reads every prediction back once (one wait on `stream`) and
 *     requests the next step's predicted sets on copy_stream: the staged
 *     set is the routed set.  The executed routing is in the buffers'
 *     ids/w, the predictions in pred_ids/pred_w (edge0_stack_get_buffers).
 * The stack must have been created on the stager's pool and slot table.
 * Enqueued directly (not as a graph).  The requests follow the canonical
 * order: per layer its own request (if any) before it computes and its
 * release after; the next step's predicted sets after the last layer. */
#define EDGE0_STAGE_LOOP 2
typedef struct {
  const int32_t* ids_dev;
  const int32_t* ids_host;
  const int32_t* next_ids_host;
  int32_t ahead;              /* 0 on demand, 1 prediction arm, EDGE0_STAGE_LOOP */
  hipStream_t copy_stream;
} edge0_stage_plan;
int edge0_stack_step_staged(edge0_stack* st, edge0_stager* sg, const edge0_stage_plan* plan,
                            const void* h0, void* h_out, int32_t step, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* EDGE0_H */
