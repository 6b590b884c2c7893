// Internal interface of the MoE-layer kernels, shared by the single-layer
// entry point and the stack runtime.
#pragma once

#include "common.h"

namespace e0 {

// Address of LoRA factor i of routed expert k, whose bundle is at b and has
// the factor at bundle offset off: the bundle's copy, or the separate
// adapter of expert ids[k] (clamped into range: an invalid id's expert has
// weight 0 and is reported by the slot resolution).
#define E0_LORA_E(a, b, e, i, off)                                                        \
  ((a).lora_sep ? (a).lo_base[i] + (size_t)max(0, min((e), (a).E - 1)) * (a).lo_stride \
                : (b) + (off))
#define E0_LORA(a, b, k, i, off) E0_LORA_E(a, b, (a).ids[k], i, off)

struct MoeArgs {
  const uint8_t* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  const int32_t* table;
  const int32_t* ids;
  const float* w;
  const uint16_t* x;        // normalised input (bf16 [d])
  uint16_t* y;
  const uint16_t* h_norm;   // optional: the first kernel computes x = bf16(RMSNorm(h_norm))
  uint16_t* x_out;          //   and workgroup 0 stores it here (then x == x_out)
  float eps;
  const uint16_t* h_res;  // optional residual input: h_out = bf16(h_res + y)
  uint16_t* h_out;
  int d, E, I, K, g, r;
  float scale;  // alpha / r
  edge0_bundle_layout lay;
  uint32_t* err;
  uint32_t* cnt_down;
  float* t_in;
  // [K][2][I]: gate then up rows of each routed expert without their LoRA
  // term, from the fused layer kernel (its down kernel finishes them)
  float* gu_pre;
  uint16_t* hp_hi;
  uint16_t* hp_lo;
  float* hs;
  float* tdpart;
  int32_t* slots;           // [K] slot of each routed expert (-1: invalid), set by k_layer_in
  unsigned long long* acc;  // [d] this layer's y in fixed point (down units add into it)
  const unsigned long long* acc_prev;  // [d] the previous layer's (combined by k_layer_in)
  int S;  // down slices
  // LoRA A x of the fused layer kernel, computed once per routed expert by
  // n_prod producer workgroups (prod_rows A rows each) into t_hand [K][2r];
  // the down launch after it reads them.  Waits (router logits) give up after
  // `spin` polls (error EDGE0_EHIP).
  float* t_hand;
  int n_prod, prod_rows;
  // a router layer's logits, computed by the producers (route_rows each)
  // and handed to every workgroup through lg_hand [2][E]: parity `par` is
  // written, the other parity's entries are emptied for the next router layer
  float* lg_hand;
  int route_rows, par;
  // adapters given apart from the bundles (edge0_moe_layer_lora): factor i
  // (a_gate, b_gate, a_up, b_up, a_down, b_down) of expert e at
  // lo_base[i] + e * lo_stride bytes; when lora_sep is false each expert's
  // factors are in its bundle at the layout's offsets
  bool lora_sep;
  const uint8_t* lo_base[6];
  int64_t lo_stride;
  // the E entries of lg_hand the launch before this layer's down kernel
  // read (a router layer's logits), or NULL: the down kernel empties them,
  // so every router layer finds both parities empty whatever the parities
  // of the router layers before it
  float* lg_consumed;
  // optional (single-layer calls on the static scratch): the combine kernel
  // moves the error word here (EDGE0_OK or EDGE0_ERANGE) and clears it
  int32_t* err_out;
  int64_t spin;
};
constexpr uint32_t kTHandEmpty = 0xFFFFFFFFu;  // a NaN no stored value takes
constexpr int64_t kFusedDefaultSpin = 1 << 21;

int fill_moe_args(const edge0_moe_shape* sh, const edge0_slot_pool* pool, const int32_t* table,
                  const int32_t* ids, const float* w, const void* x, void* y, void* workspace,
                  MoeArgs* a, bool lora_in_bundle = true);
// First launch of a layer (k_layer_in), by flags:
//   IN_COMBINE: y_prev = bf16(acc_prev), h = bf16(h_prev + y_prev)
//   IN_NORM:    x = bf16(RMSNorm(h)) (h = h_prev without IN_COMBINE)
//   IN_ROUTER:  router logits rows
//   IN_TOPK:    softmax-top-K of `logits` (computed by every workgroup)
//   IN_LORA:    t = A x rows of the K experts' gate/up adapters
//   IN_GATHER:  routing ids given (a.ids); w = softmax of `logits` taken at
//               those ids, stored to w_out
// k_layer_fused takes IN_COMBINE (else h = h_prev) and IN_ROUTER (the router
// rows and the top-K inside the launch: w_router, ids_out, w_out).
// Workgroup 0 stores h, y_prev, x, the committed ids/w and the slots.
enum { IN_COMBINE = 1, IN_NORM = 2, IN_ROUTER = 4, IN_TOPK = 8, IN_LORA = 16, IN_GATHER = 32 };
struct LayerIn {
  int flags;
  const uint16_t* h_prev;
  uint16_t* h_out;
  uint16_t* y_prev_out;
  uint16_t* x_out;
  float eps;
  const uint16_t* w_router;
  float* logits;
  int32_t* ids_out;
  float* w_out;
};

// Optional event pair recorded around one of the launches (measurement aid):
// which = 1 the gate/up GEMV, 2 the down GEMV, 3 the layer-input launch.
struct LaunchTiming {
  int which;
  hipEvent_t start, stop;
};
int launch_layer_in(const MoeArgs& a, const LayerIn& li, hipStream_t stream,
                    const LaunchTiming* timing = nullptr);
// `fc1` (optional): a head's fc1 rows, run by workgroups of the down launch
struct HeadPart;
int launch_expert_gemvs(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing = nullptr,
                        const HeadPart* fc1 = nullptr);
// the down GEMV alone; `defer` after k_layer_fused, whose gate/up rows (gu_pre,
// without their LoRA terms) the down units finish into h themselves
int launch_down(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing = nullptr,
                const HeadPart* fc1 = nullptr, bool defer = false);
// Layer input + gate/up in one launch for a layer whose routing (a.ids) is
// known before it starts; li carries the prologue (combine, residual, RMSNorm)
// arguments.  Wide rows (d_model 2048 or 4096), lora_rank <= 16.
bool layer_fused_ok(const MoeArgs& a);
int launch_layer_fused(const MoeArgs& a, const LayerIn& li, hipStream_t stream,
                       const LaunchTiming* timing = nullptr);
int launch_combine(const MoeArgs& a, hipStream_t stream);

// y = bf16 of the layer's fixed-point accumulator, outputs 256 u .. 256 u +
// 255; optional residual h_out = bf16(h_res + y); the error word moves to
// err_out if one is given (every kernel that may record an error ran before)
__device__ __forceinline__ void combine_unit(const MoeArgs& a, unsigned u) {
  const int o = (int)u * 256 + (int)threadIdx.x;
  if (o == 0 && a.err_out != nullptr) {
    *a.err_out = *a.err != 0u ? EDGE0_ERANGE : EDGE0_OK;
    *a.err = 0u;
  }
  if (o >= a.d) return;
  const uint32_t yb = f2bf(from_fix(a.acc[o]));
  a.y[o] = (uint16_t)yb;
  if (a.h_out != nullptr) a.h_out[o] = (uint16_t)f2bf(bf2f(a.h_res[o]) + bf2f(yb));
}

// A batch of prerouter heads (one per owner layer): head i reads x at
// x + i*x_stride and its routing at ids_now/ids_prev + i*ids_stride (ids_prev
// may be NULL), and writes its committed ids/w at ids_out/w_out +
// i*out_stride.  a, res, logits are [n][H], [n][E], [n][E]; counters [n].
constexpr int kMaxHeads = 48;
struct HeadBatch {
  int n, d, E, K, H;
  int has_res;
  const uint16_t* w1x[kMaxHeads];
  const uint16_t* w1oh[kMaxHeads];
  const uint16_t* b1[kMaxHeads];
  const uint16_t* w2[kMaxHeads];
  const uint16_t* b2[kMaxHeads];
  const uint16_t* wl[kMaxHeads];
  const uint16_t* x;
  int x_stride;
  const int32_t* ids_now;
  const int32_t* ids_prev;
  int ids_stride;
  float *a, *res, *logits;
  uint32_t* counters;
  int32_t* ids_out;
  float* w_out;
  int out_stride;
  uint32_t* err;
  RouteRule rule;                    // the commit (kind 0 in the stack)
};
// fc1 = false: the fc2 rows and commits only (the fc1 rows ran already)
int launch_heads(const HeadBatch& hb, hipStream_t stream, bool fc1 = true);

// One head's fc1 (and residual) rows run as workgroups beside another
// launch: the stack's folded head schedule runs head L's fc1 rows in layer
// L's down-projection launch instead of after the step's last layer.  The
// rows are the batched head kernel's own code, so the results are the same
// bit for bit.
struct HeadPart {
  int n_wg;             // workgroups of kHeadFc1Rows rows
  int d, E, K, H, has_res;
  const uint16_t *w1x, *w1oh, *b1, *w2, *b2, *wl;
  const uint16_t* x;
  const int32_t *ids_now, *ids_prev;  // ids_prev NULL: no previous token
  float *a, *res, *logits;
  uint32_t* counter;    // completion counter of the fc2 workgroups (reset by the last)
  int32_t* ids_out;
  float* w_out;
  uint32_t* err;
  RouteRule rule;
};
constexpr int kHeadFc1Rows = 4;    // fc1 rows per 256-thread workgroup (a row per wave)
// head i of a batch as a part (the workgroup count left to the caller)
__host__ __device__ inline HeadPart head_part(const HeadBatch& hb, int i) {
  HeadPart h{};
  h.d = hb.d;
  h.E = hb.E;
  h.K = hb.K;
  h.H = hb.H;
  h.has_res = hb.has_res;
  h.w1x = hb.w1x[i];
  h.w1oh = hb.w1oh[i];
  h.b1 = hb.b1[i];
  h.w2 = hb.w2[i];
  h.b2 = hb.b2[i];
  h.wl = hb.wl[i];
  h.x = hb.x + (size_t)i * hb.x_stride;
  h.ids_now = hb.ids_now != nullptr ? hb.ids_now + (size_t)i * hb.ids_stride : nullptr;
  h.ids_prev = hb.ids_prev != nullptr ? hb.ids_prev + (size_t)i * hb.ids_stride : nullptr;
  h.a = hb.a + (size_t)i * hb.H;
  h.res = hb.res + (size_t)i * hb.E;
  h.logits = hb.logits + (size_t)i * hb.E;
  h.counter = hb.counters + i;
  h.ids_out = hb.ids_out + (size_t)i * hb.out_stride;
  h.w_out = hb.w_out + (size_t)i * hb.out_stride;
  h.err = hb.err;
  h.rule = hb.rule;
  return h;
}

// the file tier, for the stager
int filetier_read(edge0_filetier* ft, const int32_t* keys, int n, const void** dev_out,
                  int* buf_out);
int filetier_mark(edge0_filetier* ft, const int* bufs, int n, hipStream_t stream);
bool filetier_matches(const edge0_filetier* ft, const edge0_moe_shape& s, int n_layers);

// what the stack runtime needs to know of a stager
edge0_slot_pool stager_pool(const edge0_stager* sg);
const int32_t* stager_table(const edge0_stager* sg);
int stager_layers(const edge0_stager* sg);


// The resident decode step as one persistent cooperative launch (flow.hip):
// G = K * d_inter / 16 workgroups stay resident for all layers and hand data
// to each other through device-coherent memory and arrival counters.
constexpr int kFlowMaxPhases = 192;  // up to 4 phases per layer
constexpr int kFlowCounters = 8;     // arrival counters per phase, 256 bytes apart
constexpr int64_t kFlowDefaultSpin = 1 << 21;  // polls per wait (about a second)
struct FlowArgs {
  int d, E, I, K, g, r, n_layers;
  float scale, eps;
  edge0_bundle_layout lay;
  const uint8_t* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  const int32_t* tables;             // [L][E]
  const uint16_t* const* routers;    // device array [L] of bf16 [E][d]
  const int32_t* pred_ids;           // [L][K] routing of consumer layers (step > 0)
  const float* pred_w;
  int32_t* exec_ids;                 // [L][K] routing the router layers commit
  float* exec_w;
  int consumer_first, consumer_last, step;
  uint16_t *x, *y, *h;               // [L][d], [L][d], [L+1][d]; h[0] holds h0
  unsigned long long* acc;           // [2][d] fixed-point y
  uint32_t* hp_hi;                   // [K][I/2] pair words of bf16(h)
  uint32_t* hp_lo;                   // [K][I/2] pair words of bf16(h - bf16(h))
  float* hs;                         // [K][I/16]
  unsigned long long* tdown;         // [K][r] A_down h, fixed point
  float* t_in;                       // [K][2r] LoRA A x of the routed experts
  float* logits;                     // [E]
  uint32_t* cnt;                     // [kFlowMaxPhases][8][64] arrival counters
  uint32_t* err;
  uint32_t* abort_word;
  int64_t spin;
  int S;                             // down slices: G = (d / 64) * S
  int cps;                           // input chunks per down slice
  uint32_t target[kFlowMaxPhases];   // counter value that completes phase p
};
// shapes the persistent step covers: d_model 2048, n_experts <= 256,
// lora_rank 0, 8 or 16, top_k <= 16, d_inter % 32 == 0, G a multiple of d/64,
// at most 16 down tiles per unit, 4 * n_layers <= kFlowMaxPhases
bool flow_shape_ok(const edge0_moe_shape& sh, int n_layers);
int flow_grid(const edge0_moe_shape& sh);
// EDGE0_OK when G workgroups of the step kernel can be resident at once
int flow_coresident(int G);
int launch_flow_step(const FlowArgs& a, int G, hipStream_t stream);

// The resident decode step as one persistent launch with the work split by
// XCD (xstep.hip): 256 workgroups, one grid-wide and one XCD-local hand-off
// per layer, weights loaded one layer ahead.
constexpr int kXMaxLayers = 64;
struct XArgs {
  int d, E, I, K, g, r, n_layers;
  int P, Ix, RW;                     // XCDs per expert, slice rows, rows per workgroup
  float scale, eps;
  // byte offsets of the bundle arrays (32-bit: a bundle is far below 4 GiB)
  struct {
    uint32_t gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b;
    uint32_t a_gate, b_gate, a_up, b_up, a_down, b_down;
  } lay;
  const uint8_t* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  const int32_t* tables;             // [L][E]
  const uint16_t* const* routers;    // device array [L] of bf16 [E][d]
  const int32_t* pred_ids;           // [L][K] routing of prediction-routed layers
  const float* pred_w;
  int32_t* exec_ids;                 // [L][K] routing the router layers commit
  float* exec_w;
  int consumer_first, consumer_last, step;
  uint16_t *x, *y, *h;               // [L][d], [L][d], [L+1][d]; h[0] holds h0
  // hand-off words (tag << 32 | payload), the tag = a.tag0 + layer
  unsigned long long* yp;            // [2][8][d] fp32 partials of y per XCD (layer parity)
  unsigned long long* yb;            // [8][d/2] bf16 pairs of y, one copy per XCD
  unsigned long long* xh;            // [8][768] h words of each XCD slice
  unsigned long long* xlog;          // [8][256] router logits of each XCD
  uint32_t tag0;                     // tag of layer 0 of this launch (never 0)
  uint32_t* err;
  uint32_t* abort_word;
  int64_t spin;
  // measurement aid: when set, workgroup w stores the 100 MHz real-time
  // clock at 16 points of layer trace_layer to trace[16 w ..]
  unsigned long long* trace;
  int trace_layer;
};
bool xstep_shape_ok(const edge0_moe_shape& sh, int n_layers);
int xstep_coresident();
int launch_xstep(const XArgs& a, hipStream_t stream);

// One layer of the same XCD split per launch (xlayer mode, graph-replayed):
// the kernel boundary hands y to the next layer (fixed-point atomics here,
// plain loads there), and h is handed within each XCD inside the launch.
struct XLArgs {
  XArgs base;                        // shape, layout, pool, error/abort, spin
  int layer;
  bool router;                       // routed by the plain router (else by pred_slot)
  const uint16_t* w_router;          // router layers: bf16 [E][d]
  const int32_t* table_row;          // router layers: [E] id -> slot
  const int32_t* pred_slot;          // prediction-routed layers: [K] slots of the routing
  const float* pred_w;               // ... and their weights
  int32_t* exec_ids;                 // router layers: [K] the committed routing
  float* exec_w;
  const uint16_t* h_prev;            // bf16 [d]: h_{L-1} (h0 at layer 0)
  const unsigned long long* acc_in;  // [d] fixed-point y_{L-1}, NULL at layer 0
  unsigned long long* acc_out;       // [d] this layer's y (zero on entry)
  unsigned long long* acc_zero;      // [d] cleared here for the layer after next
  uint16_t *x_out, *y_prev_out, *h_out;  // records: x_L, y_{L-1}, h_L (workgroup 0)
  unsigned long long* hx;            // [8][768] this layer's h words (tag 1 = written)
  unsigned long long* hx_clear;      // the other parity's, cleared here
  unsigned long long* lx;            // [8][256] router logits words
  unsigned long long* lx_clear;
};
int launch_xlayer(const XLArgs& a, hipStream_t stream, const LaunchTiming* timing = nullptr);
// slot of every prediction-routed layer's routing: slot[L][k] = table[L][ids[L][k]]
int launch_pred_slots(const int32_t* tables, const int32_t* ids, int32_t* slots, int n_layers,
                      int E, int K, int n_slots, uint32_t* err, hipStream_t stream);

RouteRule route_rule(const edge0_moe_shape* shape, const float* bias);
// the commit alone (one wave): ids/w of the K chosen experts from logits [E]
int launch_commit(const float* logits, int E, int K, const RouteRule& rr, int32_t* ids, float* w,
                  hipStream_t stream);
int launch_router(const edge0_moe_shape* shape, const void* w_router, const float* route_bias,
                  const void* x, const uint16_t* h_norm, uint16_t* x_out, float eps,
                  float* logits_out, int32_t* ids_out, float* w_out, void* workspace,
                  hipStream_t stream);

}  // namespace e0
