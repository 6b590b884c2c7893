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
#include <new>
#include <vector>

#include "moe_internal.h"

namespace e0 {

// routing each layer executed at step s, gathered into one [L][K] array
__global__ void k_gather_routing(const int32_t* __restrict__ exec_ids,
                                 const float* __restrict__ exec_w,
                                 const int32_t* __restrict__ pred_ids,
                                 const float* __restrict__ pred_w, int n_layers, int K,
                                 int consumer_first, int consumer_last, int step,
                                 int32_t* __restrict__ ids, float* __restrict__ w) {
  for (int t = threadIdx.x; t < n_layers * K; t += blockDim.x) {
    const int L = t / K;
    const bool by_pred = L >= consumer_first && L <= consumer_last && step > 0;
    ids[t] = by_pred ? pred_ids[t] : exec_ids[t];
    w[t] = by_pred ? pred_w[t] : exec_w[t];
  }
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
  int32_t* run_ids;          // [L][K] routing executed in the last step
  float* run_w;
  void* ws;
  size_t ws_bytes;
  int32_t last_step;
  hipStream_t cap;           // capture stream
  hipStream_t cap_side;      // capture stream of the head branch
  hipStream_t side;          // head branch stream for direct (timed) enqueue
  std::vector<hipEvent_t> ev_fork;  // per layer: x and routing of the layer are ready
  hipEvent_t ev_join;
  int timed_kernel;          // measurement aid: which launch class carries events
  std::vector<hipEvent_t> ev_start, ev_stop;  // one pair per layer
  hipGraphExec_t graphs[8];  // [0] step 0, [1] step 1, [2 + s%6] later steps
};

static bool is_consumer(const edge0_stack_spec& s, int L) {
  return L >= s.consumer_first && L <= s.consumer_last;
}
static bool is_owner(const edge0_stack_spec& s, int L) {
  return L >= s.owner_first && L <= s.owner_last;
}

// enqueue all launches of decode step `step` (h[0] already holds h0).  The
// heads are off the step's critical path (their predictions are used at the
// next step), so they run on a forked branch that joins at the end.
static int enqueue_step(edge0_stack* st, int step, hipStream_t stream, hipStream_t side) {
  const edge0_moe_shape& sh = st->shape;
  const int d = sh.d_model, K = sh.top_k, Lc = st->spec.n_layers, E = sh.n_experts;
  for (int L = 0; L < Lc; ++L) {
    uint16_t* hL = st->h + (size_t)L * d;
    uint16_t* xL = st->x + (size_t)L * d;
    const bool by_pred = is_consumer(st->spec, L) && step > 0;
    int32_t* ids;
    float* w;
    if (by_pred) {
      ids = st->pred_ids[step % 3] + (size_t)L * K;
      w = st->pred_w[step % 3] + (size_t)L * K;
    } else {
      ids = st->exec_ids[step & 1] + (size_t)L * K;
      w = st->exec_w[step & 1] + (size_t)L * K;
      // the router launch also computes x_L = bf16(RMSNorm(h_L))
      const int rc = launch_router(&sh, st->routers[L], nullptr, hL, xL, st->spec.rms_eps, nullptr,
                                   ids, w, st->ws, stream);
      if (rc != EDGE0_OK) return rc;
    }
    MoeArgs a;
    int rc = fill_moe_args(&sh, &st->pool, st->tables + (size_t)L * E, ids, w, xL,
                           st->y + (size_t)L * d, st->ws, &a);
    if (rc != EDGE0_OK) return rc;
    a.h_res = hL;
    a.h_out = st->h + (size_t)(L + 1) * d;
    if (by_pred) {  // the first MoE launch computes x_L
      a.h_norm = hL;
      a.x_out = xL;
      a.eps = st->spec.rms_eps;
    }
    LaunchTiming lt{st->timed_kernel, nullptr, nullptr};
    if (st->timed_kernel > 0) {
      lt.start = st->ev_start[L];
      lt.stop = st->ev_stop[L];
    }
    rc = launch_moe(a, stream, st->timed_kernel > 0 ? &lt : nullptr);
    if (rc != EDGE0_OK) return rc;
    if (is_owner(st->spec, L)) {
      if (hipEventRecord(st->ev_fork[L], stream) != hipSuccess ||
          hipStreamWaitEvent(side, st->ev_fork[L], 0) != hipSuccess)
        return EDGE0_EHIP;
      const int32_t* prev = nullptr;
      if (step > 0) {
        const bool prev_pred = is_consumer(st->spec, L) && step - 1 > 0;
        prev = prev_pred ? st->pred_ids[(step - 1) % 3] + (size_t)L * K
                         : st->exec_ids[(step - 1) & 1] + (size_t)L * K;
      }
      rc = edge0_prerouter(&sh, &st->heads[L], xL, ids, prev, nullptr,
                           st->pred_ids[(step + 1) % 3] + (size_t)(L + 1) * K,
                           st->pred_w[(step + 1) % 3] + (size_t)(L + 1) * K, st->ws, side);
      if (rc != EDGE0_OK) return rc;
    }
  }
  if (st->spec.owner_first <= st->spec.owner_last &&
      (hipEventRecord(st->ev_join, side) != hipSuccess ||
       hipStreamWaitEvent(stream, st->ev_join, 0) != hipSuccess))
    return EDGE0_EHIP;
  k_gather_routing<<<1, 256, 0, stream>>>(st->exec_ids[step & 1], st->exec_w[step & 1],
                                          st->pred_ids[step % 3], st->pred_w[step % 3], Lc, K,
                                          st->spec.consumer_first, st->spec.consumer_last, step,
                                          st->run_ids, st->run_w);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

extern "C" int edge0_stack_create(edge0_stack** out, const edge0_moe_shape* shape,
                                  const edge0_stack_spec* spec, const edge0_slot_pool* pool,
                                  const int32_t* slot_tables, const void* const* routers,
                                  const edge0_head* heads) {
  if (!out || !shape || !shape_ok(shape) || !spec || !pool || !pool->base || !slot_tables ||
      !routers || !heads)
    return EDGE0_EINVAL;
  const int Lc = spec->n_layers;
  if (Lc < 1 || spec->rms_eps < 0.f) return EDGE0_EINVAL;
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
  st->last_step = -1;
  const size_t d = shape->d_model, K = shape->top_k;
  st->ws_bytes = edge0_workspace_bytes(shape);
  bool ok = hipMalloc((void**)&st->x, Lc * d * 2) == hipSuccess &&
            hipMalloc((void**)&st->y, Lc * d * 2) == hipSuccess &&
            hipMalloc((void**)&st->h, (Lc + 1) * d * 2) == hipSuccess &&
            hipMalloc(&st->ws, st->ws_bytes) == hipSuccess &&
            hipMalloc((void**)&st->run_ids, Lc * K * 4) == hipSuccess &&
            hipMalloc((void**)&st->run_w, Lc * K * 4) == hipSuccess;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipMalloc((void**)&st->exec_ids[i], Lc * K * 4) == hipSuccess &&
         hipMalloc((void**)&st->exec_w[i], Lc * K * 4) == hipSuccess;
  for (int i = 0; i < 3 && ok; ++i)
    ok = hipMalloc((void**)&st->pred_ids[i], Lc * K * 4) == hipSuccess &&
         hipMalloc((void**)&st->pred_w[i], Lc * K * 4) == hipSuccess;
  ok = ok && hipMemset(st->ws, 0, st->ws_bytes) == hipSuccess &&
       hipMemset(st->x, 0, Lc * d * 2) == hipSuccess &&
       hipMemset(st->y, 0, Lc * d * 2) == hipSuccess;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipMemset(st->exec_ids[i], 0, Lc * K * 4) == hipSuccess &&
         hipMemset(st->exec_w[i], 0, Lc * K * 4) == hipSuccess;
  for (int i = 0; i < 3 && ok; ++i)
    ok = hipMemset(st->pred_ids[i], 0, Lc * K * 4) == hipSuccess &&
         hipMemset(st->pred_w[i], 0, Lc * K * 4) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&st->cap, hipStreamNonBlocking) == hipSuccess &&
       hipStreamCreateWithFlags(&st->cap_side, hipStreamNonBlocking) == hipSuccess &&
       hipStreamCreateWithFlags(&st->side, hipStreamNonBlocking) == hipSuccess &&
       hipEventCreateWithFlags(&st->ev_join, hipEventDisableTiming) == hipSuccess;
  for (int L = 0; L < Lc && ok; ++L) {
    hipEvent_t e;
    ok = hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
    if (ok) st->ev_fork.push_back(e);
  }
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    edge0_stack_destroy(st);
    return EDGE0_ENOMEM;
  }
  *out = st;
  return EDGE0_OK;
}

extern "C" int edge0_stack_step(edge0_stack* st, const void* h0, void* h_out, int32_t step,
                                hipStream_t stream) {
  if (!st || !h0 || !h_out || step < 0) return EDGE0_EINVAL;
  if (step != 0 && step != st->last_step + 1) return EDGE0_EINVAL;  // steps run in order
  const size_t d = st->shape.d_model;
  if (hipMemcpyAsync(st->h, h0, d * 2, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return EDGE0_EHIP;
  if (st->timed_kernel > 0) {
    // measurement mode: the same launches enqueued directly (events cannot be
    // timed inside a graph), each layer's chosen launch bracketed by events
    const int rc = enqueue_step(st, step, stream, st->side);
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
    const int rc = enqueue_step(st, step, st->cap, st->cap_side);
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

extern "C" int edge0_stack_get_buffers(const edge0_stack* st, edge0_stack_buffers* out) {
  if (!st || !out || st->last_step < 0) return EDGE0_EINVAL;
  const int s = st->last_step;
  const int Lc = st->spec.n_layers, K = st->shape.top_k;
  out->x = st->x;
  out->y = st->y;
  out->h = st->h;
  out->ids = st->run_ids;
  out->w = st->run_w;
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
  const int n = st->spec.n_layers < cap ? st->spec.n_layers : cap;
  for (int L = 0; L < n; ++L)
    if (hipEventElapsedTime(&ms_out[L], st->ev_start[L], st->ev_stop[L]) != hipSuccess)
      return EDGE0_EHIP;
  *n_out = n;
  return EDGE0_OK;
}

extern "C" void edge0_stack_destroy(edge0_stack* st) {
  if (!st) return;
  for (auto e : st->ev_start) (void)hipEventDestroy(e);
  for (auto e : st->ev_stop) (void)hipEventDestroy(e);
  for (auto& g : st->graphs)
    if (g) (void)hipGraphExecDestroy(g);
  if (st->cap) (void)hipStreamDestroy(st->cap);
  if (st->cap_side) (void)hipStreamDestroy(st->cap_side);
  if (st->side) (void)hipStreamDestroy(st->side);
  for (auto e : st->ev_fork) (void)hipEventDestroy(e);
  if (st->ev_join) (void)hipEventDestroy(st->ev_join);
  (void)hipFree(st->x);
  (void)hipFree(st->y);
  (void)hipFree(st->h);
  (void)hipFree(st->ws);
  (void)hipFree(st->run_ids);
  (void)hipFree(st->run_w);
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
