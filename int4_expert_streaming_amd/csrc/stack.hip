// Decode-stack runtime: n_layers pre-norm residual MoE blocks without
// attention, with prerouter heads predicting the next layer's routing one
// token ahead and that prediction consumed as the routing.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction": §3.2 "Motivation" (double shift: the
// head owned by layer N runs at token t and predicts layer N+1 at token
// t+1), "Head" (owner and consumer layer ranges), "Prediction-as-routing",
// "Feature drift" (the head's one-hot inputs are the routing the layer
// executed); §6 (per-step graph building is the cost to amortise - here the
// step's launches are replayed as HIP graphs).
//
// Routing buffers.  exec[s&1][L] holds the routing a plain-router layer
// computed at step s; pred[(s+1)%3][L+1] the prediction head L made at step
// s.  A consumer layer at step s>0 routes by pred[s%3][L].  Three prediction
// buffers keep the routing of step s-1 (the heads' "previous token" input)
// intact while step s writes the next predictions.
#include <cstdlib>
#include <new>
#include <vector>

#include "moe_internal.h"

namespace e0 {

// routing each layer executed at step s, gathered into one [L][K] array
struct GatherArgs {
  const int32_t* exec_ids;
  const float* exec_w;
  const int32_t* pred_ids;
  const float* pred_w;
  int n_layers, K, consumer_first, consumer_last, step;
  int32_t* ids;
  float* w;
};
__device__ __forceinline__ void gather_routing(const GatherArgs& g) {
  for (int t = threadIdx.x; t < g.n_layers * g.K; t += blockDim.x) {
    const int L = t / g.K;
    const bool by_pred = L >= g.consumer_first && L <= g.consumer_last && g.step > 0;
    g.ids[t] = by_pred ? g.pred_ids[t] : g.exec_ids[t];
    g.w[t] = by_pred ? g.pred_w[t] : g.exec_w[t];
  }
}
__global__ void k_gather_routing(GatherArgs g) { gather_routing(g); }
// the last layer's combine (workgroups 1 ..) and the gather (workgroup 0) in
// one launch: neither reads what the other writes
__global__ __launch_bounds__(256) void k_combine_gather(MoeArgs a, GatherArgs g) {
  if (blockIdx.x == 0)
    gather_routing(g);
  else
    combine_unit(a, blockIdx.x - 1);
}

}  // namespace e0

using namespace e0;

struct edge0_stack {
  edge0_moe_shape shape;
  edge0_stack_spec spec;
  edge0_slot_pool pool;
  const int32_t* tables;
  std::vector<const void*> routers;
  std::vector<edge0_head> heads;
  // device state
  uint16_t *x, *y, *h;       // [L][d], [L][d], [L+1][d]
  int32_t* exec_ids[2];
  float* exec_w[2];
  int32_t* pred_ids[3];
  float* pred_w[3];
  float* logits;             // [E] router logits of the current layer
  int32_t* run_ids[2];       // [L][K] routing executed, by step parity
  float* run_w[2];
  float *head_a, *head_res, *head_logits;
  uint32_t* head_cnt;
  void* ws;
  size_t ws_bytes;
  int32_t last_step;
  hipStream_t cap;           // capture stream
  HeadBatch heads_batch;     // head weights of the owner layers and scratch
  int timed_kernel;          // measurement aid: which launch class carries events
  std::vector<hipEvent_t> ev_start, ev_stop;  // one pair per layer
  hipGraphExec_t graphs[8];  // [0] step 0, [1] step 1, [2 + s%6] later steps
  hipEvent_t ev_heads;       // staged steps: the heads of the step have run
  int32_t* loop_host;        // staged closed loop: pinned [2][L][K] ids read back
  int head_schedule;         // EDGE0_HEADS_AFTER_LAYERS (default) or EDGE0_HEADS_FOLDED
  std::vector<edge0_lora> loras;  // adapters given apart, one table per layer (empty: in the bundles)
  // persistent mode (EDGE0_STACK_PERSISTENT)
  int mode;
  uint32_t* flow_cnt;                // [kFlowMaxPhases][kFlowCounters][64] arrival counters
  uint32_t* flow_abort;              // raised by a workgroup whose wait timed out
  const uint16_t** flow_routers;     // device copy of the router pointers
  std::vector<uint32_t> flow_uses;   // completed uses of each counter
  int64_t spin;                      // polls per bounded wait before giving up (both modes)
  // XCD-split persistent mode (EDGE0_STACK_XCD)
  unsigned long long* x_words;       // hand-off words: y partials, y copies, h slices, logits
  uint32_t* x_abort;
  uint32_t x_layers;                 // layers run so far (the next launch's first tag - 1)
  unsigned long long* x_trace;       // measurement aid (edge0_stack_set_trace), or NULL
  int x_trace_layer;
  // XCD-split layers mode (EDGE0_STACK_XLAYER): one launch per layer, graphs
  unsigned long long* xl_acc;        // [3][d] fixed-point y, by running layer number mod 3
  unsigned long long* xl_words;      // [2][8][768] h words, then [2][8][256] logits words
  int32_t* xl_slots;                 // [2][L][K] slots of the predicted routing, by step parity
};

static bool is_consumer(const edge0_stack_spec& s, int L) {
  return L >= s.consumer_first && L <= s.consumer_last;
}
static bool is_owner(const edge0_stack_spec& s, int L) {
  return L >= s.owner_first && L <= s.owner_last;
}

// fc1 false: the heads' fc1 rows ran beside the layers; only fc2 and the commits here
// comb (optional): the last layer's combine, launched with the routing gather
static int enqueue_tail(edge0_stack* st, int step, hipStream_t stream, bool fc1 = true,
                        const MoeArgs* comb = nullptr);

// Layer L's adapters given apart (edge0_stack_create_lora), if any
static void stack_lora(const edge0_stack* st, int L, MoeArgs& a) {
  if (st->loras.empty() || st->shape.lora_rank == 0) return;
  const edge0_lora& lo = st->loras[L];
  const void* f[6] = {lo.a_gate, lo.b_gate, lo.a_up, lo.b_up, lo.a_down, lo.b_down};
  a.lora_sep = true;
  for (int i = 0; i < 6; ++i) a.lo_base[i] = static_cast<const uint8_t*>(f[i]);
  a.lo_stride = lo.expert_stride * 2;  // bf16 elements
}

// The routing layer L executes at step s (its ids and weights).
static int32_t* layer_ids(const edge0_stack* st, int L, int s) {
  const bool by_pred = is_consumer(st->spec, L) && s > 0;
  return (by_pred ? st->pred_ids[s % 3] : st->exec_ids[s & 1]) + (size_t)L * st->shape.top_k;
}
static float* layer_w(const edge0_stack* st, int L, int s) {
  const bool by_pred = is_consumer(st->spec, L) && s > 0;
  return (by_pred ? st->pred_w[s % 3] : st->exec_w[s & 1]) + (size_t)L * st->shape.top_k;
}

// The folded head schedule: head L's fc1 rows run beside layer L's down
// projection (x_L and the routing layer L executed are complete by then);
// the fc2 rows and commits of all heads run batched after the last layer.
// The inputs are those of the batched heads: x_L, the routing of layer L at
// this step and at the previous one.  False: no head rows beside layer L.
static bool folded_fc1(const edge0_stack* st, int L, int step, HeadPart* out) {
  const edge0_stack_spec& sp = st->spec;
  if (st->head_schedule != EDGE0_HEADS_FOLDED || !is_owner(sp, L)) return false;
  const int d = st->shape.d_model;
  HeadBatch hb = st->heads_batch;
  hb.x = st->x + (size_t)sp.owner_first * d;
  hb.ids_now = hb.ids_prev = nullptr;
  hb.ids_out = nullptr;  // the fc1 rows commit nothing
  hb.w_out = nullptr;
  HeadPart& h = *out;
  h = head_part(hb, L - sp.owner_first);
  h.n_wg = (h.H + (h.has_res ? h.E : 0) + kHeadFc1Rows - 1) / kHeadFc1Rows;
  h.ids_now = layer_ids(st, L, step);
  h.ids_prev = step > 0 ? layer_ids(st, L, step - 1) : nullptr;
  return true;
}

// The XCD-split layers mode: per layer one launch of k_xlayer (the layer's
// input, routing, gate/up, SwiGLU, down and combine), then the last layer's
// combine, the gathered routing, the batched heads and the slots of the
// routing they predicted.  y buffer of layer L of step s: acc[(n_layers s +
// L) % 3]; hand-off words by layer parity.  Step 0 starts from cleared
// buffers (also when a handle restarts at step 0).
__global__ void k_xl_clear(unsigned long long* a, size_t na, unsigned long long* b, size_t nb) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < na + nb;
       i += (size_t)gridDim.x * blockDim.x) {
    if (i < na) a[i] = 0ull;
    else b[i - na] = 0ull;
  }
}

static int enqueue_xlayer_step(edge0_stack* st, int step, hipStream_t stream) {
  const edge0_moe_shape& sh = st->shape;
  const int Lc = st->spec.n_layers, K = sh.top_k, E = sh.n_experts;
  const size_t d = sh.d_model;
  const WsLayout wl = ws_layout(&sh);
  char* ws = static_cast<char*>(st->ws);
  const size_t n_hx = 8 * 768, n_lx = 8 * 256;
  if (step == 0) {
    k_xl_clear<<<64, 256, 0, stream>>>(st->xl_acc, 3 * d, st->xl_words, 2 * n_hx + 2 * n_lx);
    E0_CHECK_LAUNCH();
  }
  XLArgs la{};
  XArgs& a = la.base;
  a.d = sh.d_model;
  a.E = E;
  a.I = sh.d_inter;
  a.K = K;
  a.g = sh.group_size;
  a.r = sh.lora_rank;
  a.n_layers = Lc;
  a.P = 8 / K;
  a.Ix = sh.d_inter / a.P;
  a.RW = a.Ix / 32;
  a.scale = sh.lora_rank > 0 ? sh.lora_alpha / (float)sh.lora_rank : 0.f;
  a.eps = st->spec.rms_eps;
  edge0_bundle_layout lay;
  if (bundle_layout(&sh, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  auto off32 = [](int64_t v) { return v < 0 ? 0u : (uint32_t)v; };
  a.lay.gate_q = off32(lay.gate_q);
  a.lay.gate_s = off32(lay.gate_s);
  a.lay.gate_b = off32(lay.gate_b);
  a.lay.up_q = off32(lay.up_q);
  a.lay.up_s = off32(lay.up_s);
  a.lay.up_b = off32(lay.up_b);
  a.lay.down_q = off32(lay.down_q);
  a.lay.down_s = off32(lay.down_s);
  a.lay.down_b = off32(lay.down_b);
  a.lay.a_gate = off32(lay.a_gate);
  a.lay.b_gate = off32(lay.b_gate);
  a.lay.a_up = off32(lay.a_up);
  a.lay.b_up = off32(lay.b_up);
  a.lay.a_down = off32(lay.a_down);
  a.lay.b_down = off32(lay.b_down);
  a.pool = static_cast<const uint8_t*>(st->pool.base);
  a.slot_bytes = st->pool.slot_bytes;
  a.n_slots = st->pool.n_slots;
  a.err = reinterpret_cast<uint32_t*>(ws + wl.err);
  a.abort_word = st->x_abort;
  a.spin = st->spin;
  a.trace = st->x_trace;
  a.trace_layer = st->x_trace_layer;
  const unsigned base = (unsigned)Lc * (unsigned)step;  // running layer number of layer 0
  for (int L = 0; L < Lc; ++L) {
    const unsigned ell = base + (unsigned)L;
    la.layer = L;
    la.router = !(is_consumer(st->spec, L) && step > 0);
    la.w_router = static_cast<const uint16_t*>(st->routers[L]);
    la.table_row = st->tables + (size_t)L * E;
    la.pred_slot = st->xl_slots + ((size_t)(step & 1) * Lc + L) * K;
    la.pred_w = st->pred_w[step % 3] + (size_t)L * K;
    la.exec_ids = st->exec_ids[step & 1] + (size_t)L * K;
    la.exec_w = st->exec_w[step & 1] + (size_t)L * K;
    la.h_prev = st->h + (size_t)(L > 0 ? L - 1 : 0) * d;
    la.acc_in = L > 0 ? st->xl_acc + (size_t)((ell + 2) % 3) * d : nullptr;
    la.acc_out = st->xl_acc + (size_t)(ell % 3) * d;
    la.acc_zero = st->xl_acc + (size_t)((ell + 1) % 3) * d;
    la.x_out = st->x + (size_t)L * d;
    la.y_prev_out = L > 0 ? st->y + (size_t)(L - 1) * d : nullptr;
    la.h_out = st->h + (size_t)L * d;
    la.hx = st->xl_words + (size_t)(L & 1) * n_hx;
    la.hx_clear = st->xl_words + (size_t)((L + 1) & 1) * n_hx;
    la.lx = st->xl_words + 2 * n_hx + (size_t)(L & 1) * n_lx;
    la.lx_clear = st->xl_words + 2 * n_hx + (size_t)((L + 1) & 1) * n_lx;
    LaunchTiming lt{st->timed_kernel, nullptr, nullptr};
    if (st->timed_kernel > 0) {
      lt.start = st->ev_start[L];
      lt.stop = st->ev_stop[L];
    }
    const int rc = launch_xlayer(la, stream, st->timed_kernel > 0 ? &lt : nullptr);
    if (rc != EDGE0_OK) return rc;
  }
  // the last layer's combine and residual: y = bf16(acc), h_out = bf16(h + y)
  MoeArgs c{};
  c.d = sh.d_model;
  c.acc = st->xl_acc + (size_t)((base + (unsigned)Lc - 1) % 3) * d;
  c.y = st->y + (size_t)(Lc - 1) * d;
  c.h_res = st->h + (size_t)(Lc - 1) * d;
  c.h_out = st->h + (size_t)Lc * d;
  c.err_out = nullptr;
  int rc = launch_combine(c, stream);
  if (rc != EDGE0_OK) return rc;
  if ((rc = enqueue_tail(st, step, stream)) != EDGE0_OK) return rc;
  // slots of the routing the heads predicted for the next step
  return launch_pred_slots(st->tables, st->pred_ids[(step + 1) % 3],
                           st->xl_slots + (size_t)((step + 1) & 1) * Lc * K, Lc, E, K,
                           st->pool.n_slots, a.err, stream);
}

// enqueue all launches of decode step `step` (h[0] already holds h0), one
// stream: the heads come last (a forked branch for them, parallel nodes in
// the captured graph, measured slower).
static int enqueue_step(edge0_stack* st, int step, hipStream_t stream) {
  if (st->mode == EDGE0_STACK_XLAYER) return enqueue_xlayer_step(st, step, stream);
  const edge0_moe_shape& sh = st->shape;
  const int d = sh.d_model, K = sh.top_k, Lc = st->spec.n_layers, E = sh.n_experts;
  MoeArgs a{};
  for (int L = 0; L < Lc; ++L) {
    uint16_t* hL = st->h + (size_t)L * d;
    uint16_t* xL = st->x + (size_t)L * d;
    const bool by_pred = is_consumer(st->spec, L) && step > 0;
    int32_t* ids = layer_ids(st, L, step);
    float* w = layer_w(st, L, step);
    HeadPart hpart;
    const HeadPart* hp = folded_fc1(st, L, step, &hpart) ? &hpart : nullptr;
    int rc = fill_moe_args(&sh, &st->pool, st->tables + (size_t)L * E, ids, w, xL,
                           st->y + (size_t)L * d, st->ws, &a, st->loras.empty());
    if (rc != EDGE0_OK) return rc;
    stack_lora(st, L, a);
    a.spin = st->spin;
    // fixed-point y accumulators alternate between layers
    unsigned long long* acc0 = a.acc;
    a.acc = acc0 + (size_t)(L & 1) * d;
    a.acc_prev = acc0 + (size_t)((L + 1) & 1) * d;
    // layer input: the previous layer's combine + residual (L > 0), RMSNorm,
    // then the LoRA A x rows (routing known) or the router rows
    LayerIn li{};
    li.flags = IN_NORM | (L > 0 ? IN_COMBINE : 0);
    li.h_prev = L > 0 ? st->h + (size_t)(L - 1) * d : hL;
    li.h_out = hL;
    li.y_prev_out = L > 0 ? st->y + (size_t)(L - 1) * d : nullptr;
    li.x_out = xL;
    li.eps = st->spec.rms_eps;
    LaunchTiming lt{st->timed_kernel, nullptr, nullptr};
    if (st->timed_kernel > 0) {
      lt.start = st->ev_start[L];
      lt.stop = st->ev_stop[L];
    }
    if (by_pred && layer_fused_ok(a) && L > 0) {
      // routing known before the layer: input and gate/up in one launch
      li.flags |= IN_LORA;
      if ((rc = launch_layer_fused(a, li, stream, st->timed_kernel > 0 ? &lt : nullptr)) !=
              EDGE0_OK ||
          (rc = launch_down(a, stream, st->timed_kernel > 0 ? &lt : nullptr, hp, true)) != EDGE0_OK)
        return rc;
      continue;
    }
    if (by_pred) {
      li.flags |= IN_LORA;
      if ((rc = launch_layer_in(a, li, stream)) != EDGE0_OK) return rc;
    } else {
      li.flags |= IN_ROUTER;
      li.w_router = static_cast<const uint16_t*>(st->routers[L]);
      li.logits = st->logits;
      if (layer_fused_ok(a)) {
        // router rows, top-K, LoRA-in and gate/up in one launch
        LayerIn lr = li;
        lr.flags |= IN_LORA;
        lr.ids_out = ids;
        lr.w_out = w;
        a.par = L & 1;  // parity of the logits hand-off
        a.lg_consumed = a.lg_hand + (size_t)a.par * E;  // emptied again by the down kernel
        if ((rc = launch_layer_fused(a, lr, stream, st->timed_kernel > 0 ? &lt : nullptr)) !=
                EDGE0_OK ||
            (rc = launch_down(a, stream, st->timed_kernel > 0 ? &lt : nullptr, hp, true)) != EDGE0_OK)
          return rc;
        continue;
      }
      if ((rc = launch_layer_in(a, li, stream)) != EDGE0_OK) return rc;
      LayerIn l2{};
      l2.flags = IN_TOPK | IN_LORA;
      l2.logits = st->logits;
      l2.ids_out = ids;
      l2.w_out = w;
      if ((rc = launch_layer_in(a, l2, stream)) != EDGE0_OK) return rc;
    }
    if ((rc = launch_expert_gemvs(a, stream, st->timed_kernel > 0 ? &lt : nullptr, hp)) !=
        EDGE0_OK)
      return rc;
  }
  // the last layer's combine and residual
  a.h_res = st->h + (size_t)(Lc - 1) * d;
  a.h_out = st->h + (size_t)Lc * d;
  return enqueue_tail(st, step, stream, st->head_schedule != EDGE0_HEADS_FOLDED, &a);
}

// after the layers: the routing every layer executed, gathered, and every
// owner layer's head, batched
static int enqueue_tail(edge0_stack* st, int step, hipStream_t stream, bool fc1,
                        const MoeArgs* comb) {
  const edge0_moe_shape& sh = st->shape;
  const int d = sh.d_model, K = sh.top_k, Lc = st->spec.n_layers;
  int rc = EDGE0_OK;
  const GatherArgs g{st->exec_ids[step & 1], st->exec_w[step & 1], st->pred_ids[step % 3],
                     st->pred_w[step % 3],   Lc,  K,  st->spec.consumer_first,
                     st->spec.consumer_last, step, st->run_ids[step & 1], st->run_w[step & 1]};
  if (comb != nullptr)
    k_combine_gather<<<1 + (comb->d + 255) / 256, 256, 0, stream>>>(*comb, g);
  else
    k_gather_routing<<<1, 256, 0, stream>>>(g);
  E0_CHECK_LAUNCH();
  // every owner layer's head, batched: layer L's head reads x_L and the
  // routing layer L executed now and at the previous step, and commits the
  // routing of layer L+1 for the next step
  if (st->spec.owner_first <= st->spec.owner_last) {
    HeadBatch hb = st->heads_batch;
    const int L0 = st->spec.owner_first;
    hb.x = st->x + (size_t)L0 * d;
    hb.ids_now = st->run_ids[step & 1] + (size_t)L0 * K;
    hb.ids_prev = step > 0 ? st->run_ids[(step - 1) & 1] + (size_t)L0 * K : nullptr;
    hb.ids_out = st->pred_ids[(step + 1) % 3] + (size_t)(L0 + 1) * K;
    hb.w_out = st->pred_w[(step + 1) % 3] + (size_t)(L0 + 1) * K;
    rc = launch_heads(hb, stream, fc1);
    if (rc != EDGE0_OK) return rc;
  }
  return EDGE0_OK;
}

// Persistent mode: layers 0..n-1 as one cooperative launch, then the
// gathered routing and the batched heads as usual.
static int enqueue_flow_step(edge0_stack* st, int step, hipStream_t stream) {
  const edge0_moe_shape& sh = st->shape;
  const int Lc = st->spec.n_layers, K = sh.top_k;
  const WsLayout wl = ws_layout(&sh);
  char* ws = static_cast<char*>(st->ws);
  FlowArgs a{};
  a.d = sh.d_model;
  a.E = sh.n_experts;
  a.I = sh.d_inter;
  a.K = K;
  a.g = sh.group_size;
  a.r = sh.lora_rank;
  a.n_layers = Lc;
  a.scale = sh.lora_rank > 0 ? sh.lora_alpha / (float)sh.lora_rank : 0.f;
  a.eps = st->spec.rms_eps;
  if (bundle_layout(&sh, &a.lay) != EDGE0_OK) return EDGE0_EINVAL;
  a.pool = static_cast<const uint8_t*>(st->pool.base);
  a.slot_bytes = st->pool.slot_bytes;
  a.n_slots = st->pool.n_slots;
  a.tables = st->tables;
  a.routers = st->flow_routers;
  a.pred_ids = st->pred_ids[step % 3];
  a.pred_w = st->pred_w[step % 3];
  a.exec_ids = st->exec_ids[step & 1];
  a.exec_w = st->exec_w[step & 1];
  a.consumer_first = st->spec.consumer_first;
  a.consumer_last = st->spec.consumer_last;
  a.step = step;
  a.x = st->x;
  a.y = st->y;
  a.h = st->h;
  a.acc = reinterpret_cast<unsigned long long*>(ws + wl.acc);
  a.hp_hi = reinterpret_cast<uint32_t*>(ws + wl.hp_hi);
  a.hp_lo = reinterpret_cast<uint32_t*>(ws + wl.hp_lo);
  a.hs = reinterpret_cast<float*>(ws + wl.hs);
  a.tdown = reinterpret_cast<unsigned long long*>(ws + wl.tdpart);  // K * r <= its size / 8
  a.t_in = reinterpret_cast<float*>(ws + wl.t_in);
  a.logits = st->logits;
  a.cnt = st->flow_cnt;
  a.err = reinterpret_cast<uint32_t*>(ws + wl.err);
  a.abort_word = st->flow_abort;
  a.spin = st->spin;
  const int G = flow_grid(sh);
  const int rbs = sh.d_model / 64, NC = sh.d_inter / 32;
  a.S = G / rbs;
  a.cps = (NC + a.S - 1) / a.S;
  // the phases of this step in order (R for router layers, T when there is
  // LoRA, A, D); each of phase p's counters completes when it has received
  // G / kFlowCounters more arrivals than at its last use
  int p = 0;
  for (int L = 0; L < Lc; ++L) {
    const bool by_pred = is_consumer(st->spec, L) && step > 0;
    const int n = (by_pred ? 2 : 3) + (sh.lora_rank > 0 ? 1 : 0);
    for (int i = 0; i < n; ++i, ++p)
      a.target[p] = (uint32_t)(G / kFlowCounters) * (st->flow_uses[p] + 1u);
  }
  LaunchTiming lt{st->timed_kernel, nullptr, nullptr};
  if (st->timed_kernel > 0 && hipEventRecord(st->ev_start[0], stream) != hipSuccess)
    return EDGE0_EHIP;
  const int rc = launch_flow_step(a, G, stream);
  if (rc != EDGE0_OK) return rc;
  (void)lt;
  if (st->timed_kernel > 0 && hipEventRecord(st->ev_stop[0], stream) != hipSuccess)
    return EDGE0_EHIP;
  for (int i = 0; i < p; ++i) ++st->flow_uses[i];
  return enqueue_tail(st, step, stream);
}

// The XCD-split persistent mode: the step's layers in one cooperative
// launch (xstep.hip), then the gathered routing and the batched heads.
static int enqueue_xstep_step(edge0_stack* st, int step, hipStream_t stream) {
  const edge0_moe_shape& sh = st->shape;
  const int Lc = st->spec.n_layers, K = sh.top_k;
  const WsLayout wl = ws_layout(&sh);
  char* ws = static_cast<char*>(st->ws);
  XArgs a{};
  a.d = sh.d_model;
  a.E = sh.n_experts;
  a.I = sh.d_inter;
  a.K = K;
  a.g = sh.group_size;
  a.r = sh.lora_rank;
  a.n_layers = Lc;
  a.P = 8 / K;
  a.Ix = sh.d_inter / a.P;
  a.RW = a.Ix / 32;
  a.scale = sh.lora_rank > 0 ? sh.lora_alpha / (float)sh.lora_rank : 0.f;
  a.eps = st->spec.rms_eps;
  edge0_bundle_layout lay;
  if (bundle_layout(&sh, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  auto off32 = [](int64_t v) { return v < 0 ? 0u : (uint32_t)v; };  // -1: no LoRA array
  a.lay.gate_q = off32(lay.gate_q);
  a.lay.gate_s = off32(lay.gate_s);
  a.lay.gate_b = off32(lay.gate_b);
  a.lay.up_q = off32(lay.up_q);
  a.lay.up_s = off32(lay.up_s);
  a.lay.up_b = off32(lay.up_b);
  a.lay.down_q = off32(lay.down_q);
  a.lay.down_s = off32(lay.down_s);
  a.lay.down_b = off32(lay.down_b);
  a.lay.a_gate = off32(lay.a_gate);
  a.lay.b_gate = off32(lay.b_gate);
  a.lay.a_up = off32(lay.a_up);
  a.lay.b_up = off32(lay.b_up);
  a.lay.a_down = off32(lay.a_down);
  a.lay.b_down = off32(lay.b_down);
  a.pool = static_cast<const uint8_t*>(st->pool.base);
  a.slot_bytes = st->pool.slot_bytes;
  a.n_slots = st->pool.n_slots;
  a.tables = st->tables;
  a.routers = st->flow_routers;
  a.pred_ids = st->pred_ids[step % 3];
  a.pred_w = st->pred_w[step % 3];
  a.exec_ids = st->exec_ids[step & 1];
  a.exec_w = st->exec_w[step & 1];
  a.consumer_first = st->spec.consumer_first;
  a.consumer_last = st->spec.consumer_last;
  a.step = step;
  a.x = st->x;
  a.y = st->y;
  a.h = st->h;
  a.yp = st->x_words;
  a.yb = a.yp + 2 * 8 * 2048;
  a.xh = a.yb + 8 * 1024;
  a.xlog = a.xh + 8 * 768;
  a.tag0 = st->x_layers + 1u;
  a.err = reinterpret_cast<uint32_t*>(ws + wl.err);
  a.abort_word = st->x_abort;
  a.spin = st->spin;
  a.trace = st->x_trace;
  a.trace_layer = st->x_trace_layer;
  if (st->timed_kernel > 0 && hipEventRecord(st->ev_start[0], stream) != hipSuccess)
    return EDGE0_EHIP;
  const int rc = launch_xstep(a, stream);
  if (rc != EDGE0_OK) return rc;
  if (st->timed_kernel > 0 && hipEventRecord(st->ev_stop[0], stream) != hipSuccess)
    return EDGE0_EHIP;
  st->x_layers += (uint32_t)Lc;  // the tags the launch used
  return enqueue_tail(st, step, stream);
}

static int stack_create(edge0_stack** out, const edge0_moe_shape* shape,
                        const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                        const int32_t* slot_tables, const void* const* routers,
                        const edge0_head* heads, const edge0_lora* loras) {
  if (!out || !shape || !shape_ok(shape) || !spec || !pool || !pool->base || !slot_tables ||
      !routers || !heads)
    return EDGE0_EINVAL;
  if (loras != nullptr && shape->lora_rank > 0)
    for (int L = 0; L < spec->n_layers; ++L) {
      const edge0_lora& lo = loras[L];
      if (!lo.a_gate || !lo.b_gate || !lo.a_up || !lo.b_up || !lo.a_down || !lo.b_down ||
          lo.expert_stride < 0)
        return EDGE0_EINVAL;
    }
  // the step's fused routing (router layers and heads) is softmax-top-K
  if (shape->routing != EDGE0_ROUTE_SOFTMAX_TOPK) return EDGE0_EINVAL;
  const int Lc = spec->n_layers;
  if (Lc < 1 || spec->rms_eps < 0.f) return EDGE0_EINVAL;
  if (spec->owner_last - spec->owner_first + 1 > kMaxHeads) return EDGE0_EINVAL;
  // the batched heads either all carry the linear residual or none does
  for (int L = spec->owner_first; L <= spec->owner_last; ++L)
    if (L >= 0 && L < Lc && (heads[L].wl == nullptr) != (heads[spec->owner_first].wl == nullptr))
      return EDGE0_EINVAL;
  // every owner L predicts consumer L+1 and every consumer has an owner
  for (int L = 0; L < Lc; ++L) {
    if (is_owner(*spec, L) && !(L + 1 < Lc && is_consumer(*spec, L + 1))) return EDGE0_EINVAL;
    if (is_consumer(*spec, L) && !(L >= 1 && is_owner(*spec, L - 1))) return EDGE0_EINVAL;
    if (!routers[L]) return EDGE0_EINVAL;
    if (is_owner(*spec, L) && (!heads[L].w1x || !heads[L].w1oh || !heads[L].w2 ||
                               shape->head_hidden <= 0))
      return EDGE0_EINVAL;
  }
  edge0_stack* st = new (std::nothrow) edge0_stack();
  if (!st) return EDGE0_ENOMEM;
  st->shape = *shape;
  st->spec = *spec;
  st->pool = *pool;
  st->tables = slot_tables;
  st->routers.assign(routers, routers + Lc);
  st->heads.assign(heads, heads + Lc);
  if (loras != nullptr && shape->lora_rank > 0) st->loras.assign(loras, loras + Lc);
  st->last_step = -1;
  st->spin = kFlowDefaultSpin;
  st->head_schedule = EDGE0_HEADS_AFTER_LAYERS;
  const size_t d = shape->d_model, K = shape->top_k;
  st->ws_bytes = edge0_workspace_bytes(shape);
  bool ok = hipMalloc((void**)&st->x, Lc * d * 2) == hipSuccess &&
            hipMalloc((void**)&st->y, Lc * d * 2) == hipSuccess &&
            hipMalloc((void**)&st->h, (Lc + 1) * d * 2) == hipSuccess &&
            hipMalloc(&st->ws, st->ws_bytes) == hipSuccess &&
            hipMalloc((void**)&st->run_ids[0], Lc * K * 4) == hipSuccess &&
            hipMalloc((void**)&st->run_ids[1], Lc * K * 4) == hipSuccess &&
            hipMalloc((void**)&st->run_w[0], Lc * K * 4) == hipSuccess &&
            hipMalloc((void**)&st->run_w[1], Lc * K * 4) == hipSuccess &&
            hipMalloc((void**)&st->logits, (size_t)shape->n_experts * 4) == hipSuccess;
  const int n_heads = spec->owner_last >= spec->owner_first ? spec->owner_last - spec->owner_first + 1 : 0;
  const size_t E = shape->n_experts, H = shape->head_hidden;
  ok = ok && hipMalloc((void**)&st->head_a, (n_heads + 1) * H * 4) == hipSuccess &&
       hipMalloc((void**)&st->head_res, (n_heads + 1) * E * 4) == hipSuccess &&
       hipMalloc((void**)&st->head_logits, (n_heads + 1) * E * 4) == hipSuccess &&
       hipMalloc((void**)&st->head_cnt, (n_heads + 1) * 4) == hipSuccess &&
       hipMemset(st->head_cnt, 0, (n_heads + 1) * 4) == hipSuccess;
  if (ok && n_heads > 0) {
    HeadBatch& hb = st->heads_batch;
    hb.n = n_heads;
    hb.d = shape->d_model;
    hb.E = shape->n_experts;
    hb.K = shape->top_k;
    hb.H = shape->head_hidden;
    hb.has_res = heads[spec->owner_first].wl != nullptr;
    for (int i = 0; i < n_heads; ++i) {
      const edge0_head& h = heads[spec->owner_first + i];
      hb.w1x[i] = static_cast<const uint16_t*>(h.w1x);
      hb.w1oh[i] = static_cast<const uint16_t*>(h.w1oh);
      hb.b1[i] = static_cast<const uint16_t*>(h.b1);
      hb.w2[i] = static_cast<const uint16_t*>(h.w2);
      hb.b2[i] = static_cast<const uint16_t*>(h.b2);
      hb.wl[i] = static_cast<const uint16_t*>(h.wl);
    }
    hb.x_stride = shape->d_model;
    hb.ids_stride = shape->top_k;
    hb.out_stride = shape->top_k;
    hb.a = st->head_a;
    hb.res = st->head_res;
    hb.logits = st->head_logits;
    hb.counters = st->head_cnt;
    hb.err = reinterpret_cast<uint32_t*>(st->ws);  // the workspace error word (offset 0)
  }
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipMalloc((void**)&st->exec_ids[i], Lc * K * 4) == hipSuccess &&
         hipMalloc((void**)&st->exec_w[i], Lc * K * 4) == hipSuccess;
  for (int i = 0; i < 3 && ok; ++i)
    ok = hipMalloc((void**)&st->pred_ids[i], Lc * K * 4) == hipSuccess &&
         hipMalloc((void**)&st->pred_w[i], Lc * K * 4) == hipSuccess;
  ok = ok && hipMemset(st->ws, 0, st->ws_bytes) == hipSuccess &&
       hipMemset(static_cast<uint8_t*>(st->ws) + ws_layout(shape).lg_hand, 0xFF,
                 (size_t)4 * 2 * shape->n_experts) == hipSuccess &&
       hipMemset(st->x, 0, Lc * d * 2) == hipSuccess &&
       hipMemset(st->y, 0, Lc * d * 2) == hipSuccess;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipMemset(st->exec_ids[i], 0, Lc * K * 4) == hipSuccess &&
         hipMemset(st->exec_w[i], 0, Lc * K * 4) == hipSuccess;
  for (int i = 0; i < 3 && ok; ++i)
    ok = hipMemset(st->pred_ids[i], 0, Lc * K * 4) == hipSuccess &&
         hipMemset(st->pred_w[i], 0, Lc * K * 4) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&st->cap, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    edge0_stack_destroy(st);
    return EDGE0_ENOMEM;
  }
  *out = st;
  return EDGE0_OK;
}

extern "C" int edge0_stack_create(edge0_stack** out, const edge0_moe_shape* shape,
                                  const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                                  const int32_t* slot_tables, const void* const* routers,
                                  const edge0_head* heads) {
  return stack_create(out, shape, spec, pool, slot_tables, routers, heads, nullptr);
}

extern "C" int edge0_stack_create_lora(edge0_stack** out, const edge0_moe_shape* shape,
                                       const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                                       const int32_t* slot_tables, const void* const* routers,
                                       const edge0_head* heads, const edge0_lora* layer_loras) {
  if (shape && shape->lora_rank > 0 && !layer_loras) return EDGE0_EINVAL;
  return stack_create(out, shape, spec, pool, slot_tables, routers, heads, layer_loras);
}

extern "C" int edge0_stack_step(edge0_stack* st, const void* h0, void* h_out, int32_t step,
                                hipStream_t stream) {
  if (!st || !h0 || !h_out || step < 0) return EDGE0_EINVAL;
  if (step != 0 && step != st->last_step + 1) return EDGE0_EINVAL;  // steps run in order
  const size_t d = st->shape.d_model;
  if (hipMemcpyAsync(st->h, h0, d * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return EDGE0_EHIP;
  if (st->mode == EDGE0_STACK_PERSISTENT || st->mode == EDGE0_STACK_XCD) {
    const int rc = st->mode == EDGE0_STACK_XCD ? enqueue_xstep_step(st, step, stream)
                                               : enqueue_flow_step(st, step, stream);
    if (rc != EDGE0_OK) return rc;
    if (hipMemcpyAsync(h_out, st->h + (size_t)st->spec.n_layers * d, d * 2,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return EDGE0_EHIP;
    st->last_step = step;
    return EDGE0_OK;
  }
  if (st->timed_kernel > 0) {
    // measurement mode: the same launches enqueued directly (events cannot be
    // timed inside a graph), each layer's chosen launch bracketed by events
    const int rc = enqueue_step(st, step, stream);
    if (rc != EDGE0_OK) return rc;
    if (hipMemcpyAsync(h_out, st->h + (size_t)st->spec.n_layers * d, d * 2,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return EDGE0_EHIP;
    st->last_step = step;
    return EDGE0_OK;
  }
  const int gi = step <= 1 ? step : 2 + step % 6;
  if (!st->graphs[gi]) {
    hipGraph_t g = nullptr;
    if (hipStreamBeginCapture(st->cap, hipStreamCaptureModeThreadLocal) != hipSuccess)
      return EDGE0_EHIP;
    const int rc = enqueue_step(st, step, st->cap);
    const hipError_t ec = hipStreamEndCapture(st->cap, &g);
    if (rc != EDGE0_OK) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (ec != hipSuccess) return EDGE0_EHIP;
    const hipError_t ei = hipGraphInstantiate(&st->graphs[gi], g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (ei != hipSuccess) {
      st->graphs[gi] = nullptr;
      return EDGE0_EHIP;
    }
  }
  if (hipGraphLaunch(st->graphs[gi], stream) != hipSuccess) return EDGE0_EHIP;
  if (hipMemcpyAsync(h_out, st->h + (size_t)st->spec.n_layers * d, d * 2,
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return EDGE0_EHIP;
  st->last_step = step;
  return EDGE0_OK;
}

// ----------------------------------------------------------- staged step
// host ids of every layer: in range and distinct (checked before anything
// is enqueued)
static bool ids_ok(const int32_t* ids, int n_layers, int K, int E) {
  for (int L = 0; L < n_layers; ++L)
    for (int i = 0; i < K; ++i) {
      const int32_t v = ids[L * K + i];
      if (v < 0 || v >= E) return false;
      for (int j = 0; j < i; ++j)
        if (ids[L * K + j] == v) return false;
    }
  return true;
}

static int enqueue_staged_step(edge0_stack* st, edge0_stager* sg, const edge0_stage_plan& plan,
                               int step, hipStream_t stream) {
  const edge0_moe_shape& sh = st->shape;
  const int d = sh.d_model, K = sh.top_k, Lc = st->spec.n_layers, E = sh.n_experts;
  const bool ahead = plan.ahead != 0;
  const bool loop = plan.ahead == EDGE0_STAGE_LOOP;
  float* w_exec = st->exec_w[step & 1];
  MoeArgs a{};
  int rc;
  for (int L = 0; L < Lc; ++L) {
    uint16_t* hL = st->h + (size_t)L * d;
    uint16_t* xL = st->x + (size_t)L * d;
    const bool by_pred = ahead && is_consumer(st->spec, L) && step > 0;
    // closed loop: a prediction-routed layer executes its head's committed
    // routing, a router layer the top-K of its own router
    const int32_t* ids =
        loop ? (by_pred ? st->pred_ids[step % 3] : st->exec_ids[step & 1]) + (size_t)L * K
             : plan.ids_dev + (size_t)L * K;
    float* w = w_exec + (size_t)L * K;
    rc = fill_moe_args(&sh, &st->pool, st->tables + (size_t)L * E, ids, w, xL,
                       st->y + (size_t)L * d, st->ws, &a, st->loras.empty());
    if (rc != EDGE0_OK) return rc;
    stack_lora(st, L, a);
    unsigned long long* acc0 = a.acc;
    a.acc = acc0 + (size_t)(L & 1) * d;
    a.acc_prev = acc0 + (size_t)((L + 1) & 1) * d;
    LayerIn li{};
    li.flags = IN_NORM | (L > 0 ? IN_COMBINE : 0);
    li.h_prev = L > 0 ? st->h + (size_t)(L - 1) * d : hL;
    li.h_out = hL;
    li.y_prev_out = L > 0 ? st->y + (size_t)(L - 1) * d : nullptr;
    li.x_out = xL;
    li.eps = st->spec.rms_eps;
    if (by_pred) {
      // the set was staged one step ahead: wait for its copies, weights
      // from the logits the owner's head produced at the previous step
      if ((rc = edge0_stager_wait(sg, L, step, stream)) != EDGE0_OK) return rc;
      li.flags |= IN_GATHER | IN_LORA;
      li.logits = st->head_logits + (size_t)(L - 1 - st->spec.owner_first) * E;
      li.w_out = w;
      if ((rc = launch_layer_in(a, li, stream)) != EDGE0_OK) return rc;
    } else {
      // router first; the set is known once it ran: fill it on demand on the
      // compute stream, then the weights and the LoRA A x rows
      li.flags |= IN_ROUTER;
      li.w_router = static_cast<const uint16_t*>(st->routers[L]);
      li.logits = st->logits;
      if ((rc = launch_layer_in(a, li, stream)) != EDGE0_OK) return rc;
      const int32_t* want = loop ? nullptr : plan.ids_host + (size_t)L * K;
      if (loop) {
        // commit on the device; the host learns the set by reading it back
        int32_t* exec = st->exec_ids[step & 1] + (size_t)L * K;
        RouteRule rr{};
        if ((rc = launch_commit(st->logits, E, K, rr, exec, w, stream)) != EDGE0_OK) return rc;
        if (hipMemcpyAsync(st->loop_host + (size_t)L * K, exec, (size_t)K * 4,
                           hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
          return EDGE0_EHIP;
        want = st->loop_host + (size_t)L * K;
        if (!ids_ok(want, 1, K, E)) return EDGE0_ERANGE;
      }
      if ((rc = edge0_stage_experts(sg, L, step, want, K, nullptr, stream)) != EDGE0_OK ||
          (rc = edge0_stager_wait(sg, L, step, stream)) != EDGE0_OK)
        return rc;
      LayerIn l2{};
      l2.flags = IN_GATHER | IN_LORA;
      l2.logits = st->logits;
      l2.w_out = w;
      if ((rc = launch_layer_in(a, l2, stream)) != EDGE0_OK) return rc;
    }
    if ((rc = launch_expert_gemvs(a, stream)) != EDGE0_OK) return rc;
    if ((rc = edge0_stager_release(sg, L, step, stream)) != EDGE0_OK) return rc;
  }
  a.h_res = st->h + (size_t)(Lc - 1) * d;
  a.h_out = st->h + (size_t)Lc * d;
  if ((rc = launch_combine(a, stream)) != EDGE0_OK) return rc;
  if (loop) {
    // prediction-routed layers executed the heads' routing, the others their
    // router's
    k_gather_routing<<<1, 256, 0, stream>>>(GatherArgs{
        st->exec_ids[step & 1], w_exec, st->pred_ids[step % 3], w_exec, Lc, K,
        st->spec.consumer_first, st->spec.consumer_last, step, st->run_ids[step & 1],
        st->run_w[step & 1]});
  } else {
    // every layer executed the given ids
    k_gather_routing<<<1, 256, 0, stream>>>(GatherArgs{plan.ids_dev, w_exec, plan.ids_dev, w_exec,
                                                       Lc, K, 1, 0, step, st->run_ids[step & 1],
                                                       st->run_w[step & 1]});
  }
  E0_CHECK_LAUNCH();
  if (!ahead || st->spec.owner_first > st->spec.owner_last) return EDGE0_OK;
  HeadBatch hb = st->heads_batch;
  const int L0 = st->spec.owner_first;
  hb.x = st->x + (size_t)L0 * d;
  hb.ids_now = st->run_ids[step & 1] + (size_t)L0 * K;
  hb.ids_prev = step > 0 ? st->run_ids[(step - 1) & 1] + (size_t)L0 * K : nullptr;
  hb.ids_out = st->pred_ids[(step + 1) % 3] + (size_t)(L0 + 1) * K;
  hb.w_out = st->pred_w[(step + 1) % 3] + (size_t)(L0 + 1) * K;
  if ((rc = launch_heads(hb, stream)) != EDGE0_OK) return rc;
  if (loop) {
    // one read-back per step: every prediction the heads committed, staged
    // for the next step on the copy stream (the host has waited for the
    // heads, so the copies may start at once)
    int32_t* pred = st->loop_host + (size_t)Lc * K;
    if (hipMemcpyAsync(pred, st->pred_ids[(step + 1) % 3], (size_t)Lc * K * 4,
                       hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return EDGE0_EHIP;
    for (int L = st->spec.owner_first; L <= st->spec.owner_last; ++L) {
      if (!ids_ok(pred + (size_t)(L + 1) * K, 1, K, E)) return EDGE0_ERANGE;
      if ((rc = edge0_stage_experts(sg, L + 1, step + 1, pred + (size_t)(L + 1) * K, K, nullptr,
                                    plan.copy_stream)) != EDGE0_OK)
        return rc;
    }
    return edge0_stager_flush(sg, stream);
  }
  if (!plan.next_ids_host) return EDGE0_OK;
  // the next step's predicted sets, known once the heads ran
  if (!st->ev_heads &&
      hipEventCreateWithFlags(&st->ev_heads, hipEventDisableTiming) != hipSuccess)
    return EDGE0_EHIP;
  if (hipEventRecord(st->ev_heads, stream) != hipSuccess ||
      hipStreamWaitEvent(plan.copy_stream, st->ev_heads, 0) != hipSuccess)
    return EDGE0_EHIP;
  for (int L = st->spec.owner_first; L <= st->spec.owner_last; ++L)
    if ((rc = edge0_stage_experts(sg, L + 1, step + 1, plan.next_ids_host + (size_t)(L + 1) * K,
                                  K, nullptr, plan.copy_stream)) != EDGE0_OK)
      return rc;
  // their slot-table updates, on the compute stream (ahead of their use)
  return edge0_stager_flush(sg, stream);
}

extern "C" int edge0_stack_step_staged(edge0_stack* st, edge0_stager* sg,
                                       const edge0_stage_plan* plan, const void* h0, void* h_out,
                                       int32_t step, hipStream_t stream) {
  if (!st || !sg || !plan || !h0 || !h_out || step < 0) return EDGE0_EINVAL;
  if (plan->ahead != 0 && plan->ahead != 1 && plan->ahead != EDGE0_STAGE_LOOP) return EDGE0_EINVAL;
  const bool loop = plan->ahead == EDGE0_STAGE_LOOP;
  if (!loop && (!plan->ids_dev || !plan->ids_host)) return EDGE0_EINVAL;
  if (step != 0 && step != st->last_step + 1) return EDGE0_EINVAL;
  const edge0_slot_pool sp = stager_pool(sg);
  const int Lc = st->spec.n_layers, K = st->shape.top_k, E = st->shape.n_experts;
  if (sp.base != st->pool.base || sp.slot_bytes != st->pool.slot_bytes ||
      sp.n_slots != st->pool.n_slots || stager_table(sg) != st->tables || stager_layers(sg) != Lc)
    return EDGE0_EINVAL;
  if (!loop && !ids_ok(plan->ids_host, Lc, K, E)) return EDGE0_EINVAL;
  if (plan->ahead == 1 && plan->next_ids_host && !ids_ok(plan->next_ids_host, Lc, K, E))
    return EDGE0_EINVAL;
  if (loop && !st->loop_host &&
      hipHostMalloc((void**)&st->loop_host, 2 * (size_t)Lc * K * 4, hipHostMallocDefault) !=
          hipSuccess)
    return EDGE0_ENOMEM;
  const size_t d = st->shape.d_model;
  if (hipMemcpyAsync(st->h, h0, d * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return EDGE0_EHIP;
  const int rc = enqueue_staged_step(st, sg, *plan, step, stream);
  if (rc != EDGE0_OK) return rc;
  if (hipMemcpyAsync(h_out, st->h + (size_t)Lc * d, d * 2, hipMemcpyDeviceToDevice, stream) !=
      hipSuccess)
    return EDGE0_EHIP;
  st->last_step = step;
  return EDGE0_OK;
}

extern "C" int edge0_stack_get_buffers(const edge0_stack* st, edge0_stack_buffers* out) {
  if (!st || !out || st->last_step < 0) return EDGE0_EINVAL;
  const int s = st->last_step;
  const int Lc = st->spec.n_layers, K = st->shape.top_k;
  out->x = st->x;
  out->y = st->y;
  out->h = st->h;
  out->ids = st->run_ids[s & 1];
  out->w = st->run_w[s & 1];
  out->pred_ids = st->pred_ids[(s + 1) % 3];
  out->pred_w = st->pred_w[(s + 1) % 3];
  (void)Lc;
  (void)K;
  return EDGE0_OK;
}

extern "C" int edge0_stack_set_timing(edge0_stack* st, int32_t kernel) {
  if (!st || kernel < 0 || kernel > 3) return EDGE0_EINVAL;
  const int n = st->spec.n_layers;
  while ((int)st->ev_start.size() < n) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return EDGE0_EHIP;
    st->ev_start.push_back(a);
    st->ev_stop.push_back(b);
  }
  st->timed_kernel = kernel;
  return EDGE0_OK;
}

extern "C" int edge0_stack_kernel_ms(edge0_stack* st, float* ms_out, int32_t cap, int32_t* n_out) {
  if (!st || !ms_out || !n_out || st->timed_kernel <= 0 || st->last_step < 0) return EDGE0_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return EDGE0_EHIP;
  const int n = (st->mode == EDGE0_STACK_PERSISTENT || st->mode == EDGE0_STACK_XCD)
                    ? (cap > 0 ? 1 : 0)
                                                   : (st->spec.n_layers < cap ? st->spec.n_layers : cap);
  for (int L = 0; L < n; ++L)
    if (hipEventElapsedTime(&ms_out[L], st->ev_start[L], st->ev_stop[L]) != hipSuccess)
      return EDGE0_EHIP;
  *n_out = n;
  return EDGE0_OK;
}

// device copy of the router pointers (persistent modes)
static int ensure_routers(edge0_stack* st) {
  if (st->flow_routers) return EDGE0_OK;
  const int Lc = st->spec.n_layers;
  if (hipMalloc((void**)&st->flow_routers, Lc * sizeof(void*)) != hipSuccess) return EDGE0_ENOMEM;
  if (hipMemcpy(st->flow_routers, st->routers.data(), Lc * sizeof(void*), hipMemcpyHostToDevice) !=
      hipSuccess)
    return EDGE0_EHIP;
  return EDGE0_OK;
}

extern "C" int edge0_stack_set_mode(edge0_stack* st, int32_t mode) {
  if (!st || (mode != EDGE0_STACK_GRAPHS && mode != EDGE0_STACK_PERSISTENT &&
              mode != EDGE0_STACK_XCD && mode != EDGE0_STACK_XLAYER))
    return EDGE0_EINVAL;
  // the one-launch and XCD-split modes read the adapters from the bundles
  if (mode != EDGE0_STACK_GRAPHS && !st->loras.empty()) return EDGE0_EINVAL;
  if (mode == EDGE0_STACK_XLAYER) {
    if (!xstep_shape_ok(st->shape, st->spec.n_layers)) return EDGE0_EINVAL;
    if (!st->xl_acc) {
      const size_t d = st->shape.d_model;
      const size_t nw = 2 * 8 * 768 + 2 * 8 * 256;
      const size_t ns = 2 * (size_t)st->spec.n_layers * st->shape.top_k;
      if (hipMalloc((void**)&st->xl_acc, 3 * d * 8) != hipSuccess ||
          hipMalloc((void**)&st->xl_words, nw * 8) != hipSuccess ||
          hipMalloc((void**)&st->xl_slots, ns * 4) != hipSuccess ||
          (!st->x_abort && hipMalloc((void**)&st->x_abort, 4) != hipSuccess))
        return EDGE0_ENOMEM;
      if (hipMemset(st->xl_acc, 0, 3 * d * 8) != hipSuccess ||
          hipMemset(st->xl_words, 0, nw * 8) != hipSuccess ||
          hipMemset(st->xl_slots, 0xFF, ns * 4) != hipSuccess ||
          hipMemset(st->x_abort, 0, 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return EDGE0_EHIP;
    }
  }
  // graphs captured in another mode hold other launches
  if (mode != st->mode)
    for (auto& g : st->graphs)
      if (g) {
        (void)hipGraphExecDestroy(g);
        g = nullptr;
      }
  if (mode == EDGE0_STACK_XCD) {
    if (!xstep_shape_ok(st->shape, st->spec.n_layers)) return EDGE0_EINVAL;
    int rc = xstep_coresident();
    if (rc != EDGE0_OK) return rc;
    if ((rc = ensure_routers(st)) != EDGE0_OK) return rc;
    if (!st->x_words) {
      // y partials [2][8][2048], y copies [8][1024], h slices [8][768],
      // logits [8][256]; tag 0 is never used, so zeroed words are stale
      const size_t words = 2 * 8 * 2048 + 8 * 1024 + 8 * 768 + 8 * 256;
      if (hipMalloc((void**)&st->x_words, words * 8) != hipSuccess ||
          hipMalloc((void**)&st->x_abort, 4) != hipSuccess)
        return EDGE0_ENOMEM;
      if (hipMemset(st->x_words, 0, words * 8) != hipSuccess ||
          hipMemset(st->x_abort, 0, 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        return EDGE0_EHIP;
      st->x_layers = 0;
    }
    st->mode = mode;
    return EDGE0_OK;
  }
  if (mode == EDGE0_STACK_PERSISTENT) {
    const int Lc = st->spec.n_layers;
    if (!flow_shape_ok(st->shape, Lc)) return EDGE0_EINVAL;
    int rc = flow_coresident(flow_grid(st->shape));
    if (rc != EDGE0_OK) return rc;
    if ((rc = ensure_routers(st)) != EDGE0_OK) return rc;
    if (!st->flow_cnt) {
      const size_t cnt_bytes = (size_t)kFlowMaxPhases * kFlowCounters * 64 * 4;
      if (hipMalloc((void**)&st->flow_cnt, cnt_bytes) != hipSuccess ||
          hipMalloc((void**)&st->flow_abort, 4) != hipSuccess)
        return EDGE0_ENOMEM;
      if (hipMemset(st->flow_cnt, 0, cnt_bytes) != hipSuccess ||
          hipMemset(st->flow_abort, 0, 4) != hipSuccess)
        return EDGE0_EHIP;
      st->flow_uses.assign(kFlowMaxPhases, 0u);
    }
  }
  st->mode = mode;
  return EDGE0_OK;
}

extern "C" int edge0_stack_set_trace(edge0_stack* st, int32_t layer, uint64_t* trace) {
  if (!st || (trace && (layer < 0 || layer >= st->spec.n_layers))) return EDGE0_EINVAL;
  st->x_trace = reinterpret_cast<unsigned long long*>(trace);
  st->x_trace_layer = layer;
  // the per-layer mode's step graphs hold the trace pointer in their arguments
  for (auto& g : st->graphs)
    if (g) {
      (void)hipGraphExecDestroy(g);
      g = nullptr;
    }
  return EDGE0_OK;
}

extern "C" int edge0_stack_set_head_schedule(edge0_stack* st, int32_t schedule) {
  if (!st || (schedule != EDGE0_HEADS_FOLDED && schedule != EDGE0_HEADS_AFTER_LAYERS))
    return EDGE0_EINVAL;
  if (schedule == st->head_schedule) return EDGE0_OK;
  // the step graphs hold the schedule: wait for any replay, then rebuild them
  if (hipDeviceSynchronize() != hipSuccess) return EDGE0_EHIP;
  st->head_schedule = schedule;
  for (auto& g : st->graphs)
    if (g) {
      (void)hipGraphExecDestroy(g);
      g = nullptr;
    }
  return EDGE0_OK;
}

extern "C" int edge0_stack_error(edge0_stack* st) {
  if (!st) return EDGE0_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return EDGE0_EHIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, st->ws, 4, hipMemcpyDeviceToHost) != hipSuccess) return EDGE0_EHIP;
  const uint32_t zero = 0;
  if (hipMemcpy(st->ws, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return EDGE0_EHIP;
  if (v & (uint32_t)(-EDGE0_EHIP)) return EDGE0_EHIP;
  return v ? EDGE0_ERANGE : EDGE0_OK;
}

extern "C" int edge0_stack_set_spin_limit(edge0_stack* st, int64_t polls) {
  if (!st || polls < 0) return EDGE0_EINVAL;
  st->spin = polls > 0 ? polls : kFlowDefaultSpin;
  // the step graphs hold the old limit in their launch arguments
  for (auto& g : st->graphs)
    if (g) {
      (void)hipGraphExecDestroy(g);
      g = nullptr;
    }
  return EDGE0_OK;
}

extern "C" void edge0_stack_destroy(edge0_stack* st) {
  if (!st) return;
  // the handle's launches (graphs, the persistent step, the capture stream)
  // may still be running on the device: let them finish before their
  // events, graphs, stream and buffers go
  (void)hipDeviceSynchronize();
  for (auto e : st->ev_start) (void)hipEventDestroy(e);
  for (auto e : st->ev_stop) (void)hipEventDestroy(e);
  for (auto& g : st->graphs)
    if (g) (void)hipGraphExecDestroy(g);
  if (st->cap) (void)hipStreamDestroy(st->cap);
  if (st->ev_heads) (void)hipEventDestroy(st->ev_heads);
  (void)hipFree(st->x_words);
  (void)hipFree(st->x_abort);
  if (st->loop_host) (void)hipHostFree(st->loop_host);
  (void)hipFree(st->xl_acc);
  (void)hipFree(st->xl_words);
  (void)hipFree(st->xl_slots);
  (void)hipFree(st->flow_cnt);
  (void)hipFree(st->flow_abort);
  (void)hipFree(const_cast<uint16_t**>(st->flow_routers));

  (void)hipFree(st->x);
  (void)hipFree(st->y);
  (void)hipFree(st->h);
  (void)hipFree(st->ws);
  for (int i = 0; i < 2; ++i) {
    (void)hipFree(st->run_ids[i]);
    (void)hipFree(st->run_w[i]);
  }
  (void)hipFree(st->logits);
  (void)hipFree(st->head_a);
  (void)hipFree(st->head_res);
  (void)hipFree(st->head_logits);
  (void)hipFree(st->head_cnt);
  for (int i = 0; i < 2; ++i) {
    (void)hipFree(st->exec_ids[i]);
    (void)hipFree(st->exec_w[i]);
  }
  for (int i = 0; i < 3; ++i) {
    (void)hipFree(st->pred_ids[i]);
    (void)hipFree(st->pred_w[i]);
  }
  delete st;
}
