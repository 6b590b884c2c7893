// Routing kernels: the plain router GEMV, the prerouter head and the commit
// (softmax-top-K or sigmoid-group).
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction".  Routing math: §2 "MoE routing" and
// App. A "Softmax-topk", "Sigmoid-group"; head: §3.2 "Head",
// "Prediction-as-routing".
//
// The GEMVs here are small (router E x d bf16; head fc1 H x d fp16 plus the
// residual E x d, fc2 E x H) and HBM-bound: one wave per output row, 16-byte
// loads per lane, fp32 accumulation, a wave butterfly for the row sum.  The
// top-K runs in the last workgroup to finish (completion counter in the
// workspace), so a router or head call is one or two launches.
#include "heads_dev.h"
#include "moe_internal.h"

namespace e0 {

// ---------------------------------------------------------------- router
// With h_norm set, every workgroup computes x = bf16(RMSNorm(h_norm)) into LDS
// and workgroup 0 stores it to x_out.
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ wr,
                                                const uint16_t* __restrict__ x_in,
                                                const uint16_t* __restrict__ h_norm,
                                                uint16_t* __restrict__ x_out, float eps, int d,
                                                int E, int K, RouteRule rr,
                                                float* __restrict__ logits,
                                                int32_t* __restrict__ ids, float* __restrict__ w,
                                                uint32_t* __restrict__ counter) {
  __shared__ uint16_t xs[kMaxD];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  RowPref pf;
  const bool pref = row < E && d <= 64 * kPrefChunks * 8;
  if (pref) row_prefetch(wr + (size_t)row * d, d, pf);   // in flight during the norm
  const uint16_t* x = x_in;
  if (h_norm != nullptr) {
    rmsnorm_to_lds(h_norm, xs, d, eps);
    if (blockIdx.x == 0)
      for (int j = threadIdx.x; j < d; j += blockDim.x) x_out[j] = xs[j];
    x = xs;
  }
  if (row < E) {
    const float s = pref ? row_dot_pref(pf, x, d) : row_dot<false, false>(wr + (size_t)row * d, x, d);
    if ((threadIdx.x & 63) == 0) st_dev(logits + row, s);
  }
  if (last_arrival(counter, gridDim.x)) {
    if (wave == 0) wave_commit<true>(logits, E, K, rr, ids, w);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ prerouter
// Heads run batched: one launch covers the fc1 (and residual) rows of every
// head of the batch, one the fc2 rows and each head's top-K (the last
// workgroup of a head, per-head completion counter).  A batch of one is the
// single-head call; the stack runs the heads of all owner layers of a step
// as one batch after the step's layers ("one flush per step").
// fc1 rows [0, H) of head i and its residual rows [H, H+E): one wave per row
__global__ __launch_bounds__(256) void k_heads_fc1(HeadBatch hb) {
  const int per = (hb.H + (hb.has_res ? hb.E : 0) + 3) / 4;
  const int i = blockIdx.x / per;
  head_fc1_row(head_part(hb, i), (blockIdx.x % per) * 4 + (threadIdx.x >> 6));
}

// fc2 rows and each head's commit: a workgroup covers 8 * kFc2Waves rows of
// one head, so a head spreads over E / 16 compute units; the logits go to
// memory and the head's last workgroup to finish commits the top-K.
constexpr int kFc2Waves = 2;
__global__ __launch_bounds__(64 * kFc2Waves) void k_heads_fc2(HeadBatch hb) {
  const int parts = (hb.E + 8 * kFc2Waves - 1) / (8 * kFc2Waves);
  const int i = blockIdx.x / parts;
  head_fc2_part(head_part(hb, i), blockIdx.x % parts, parts);
}

int launch_heads(const HeadBatch& hb, hipStream_t stream, bool fc1) {
  if (hb.n < 1 || hb.n > kMaxHeads) return EDGE0_EINVAL;
  if (fc1) {
    const int per1 = (hb.H + (hb.has_res ? hb.E : 0) + 3) / 4;
    k_heads_fc1<<<hb.n * per1, 256, 0, stream>>>(hb);
    E0_CHECK_LAUNCH();
  }
  k_heads_fc2<<<hb.n * ((hb.E + 8 * kFc2Waves - 1) / (8 * kFc2Waves)), 64 * kFc2Waves, 0,
                stream>>>(hb);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

}  // namespace e0

using namespace e0;

namespace e0 {
RouteRule route_rule(const edge0_moe_shape* shape, const float* bias) {
  RouteRule rr{};
  rr.kind = shape->routing;
  rr.n_groups = shape->n_groups;
  rr.top_groups = shape->top_groups;
  rr.scale = shape->route_scale;
  rr.bias = bias;
  return rr;
}

int launch_router(const edge0_moe_shape* shape, const void* w_router, const float* route_bias,
                  const void* x, const uint16_t* h_norm, uint16_t* x_out, float eps,
                  float* logits_out, int32_t* ids_out, float* w_out, void* workspace,
                  hipStream_t stream) {
  const WsLayout L = ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.logits);
  const int E = shape->n_experts;
  k_router<<<(E + 3) / 4, 256, 0, stream>>>(
      static_cast<const uint16_t*>(w_router), static_cast<const uint16_t*>(x), h_norm, x_out, eps,
      shape->d_model, E, shape->top_k, route_rule(shape, route_bias), logits, ids_out, w_out,
      reinterpret_cast<uint32_t*>(ws + L.cnt_router));
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
}  // namespace e0

extern "C" int edge0_router(const edge0_moe_shape* shape, const void* w_router,
                            const float* route_bias, const void* x, float* logits_out,
                            int32_t* ids_out, float* w_out, void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !w_router || !x || !ids_out || !w_out || !workspace)
    return EDGE0_EINVAL;
  return launch_router(shape, w_router, route_bias, x, nullptr, nullptr, 0.f, logits_out, ids_out,
                       w_out, workspace, stream);
}

extern "C" int edge0_prerouter(const edge0_moe_shape* shape, const edge0_head* head,
                               const float* route_bias, const void* x, const int32_t* ids_now,
                               const int32_t* ids_prev, float* logits_out, int32_t* ids_out,
                               float* w_out, void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !head || !head->w1x || !head->w1oh || !head->w2 || !x ||
      !ids_now || !ids_out || !w_out || !workspace || shape->head_hidden <= 0)
    return EDGE0_EINVAL;
  const WsLayout L = ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  HeadBatch hb{};
  hb.n = 1;
  hb.d = shape->d_model;
  hb.E = shape->n_experts;
  hb.K = shape->top_k;
  hb.H = shape->head_hidden;
  hb.has_res = head->wl != nullptr;
  hb.w1x[0] = static_cast<const uint16_t*>(head->w1x);
  hb.w1oh[0] = static_cast<const uint16_t*>(head->w1oh);
  hb.b1[0] = static_cast<const uint16_t*>(head->b1);
  hb.w2[0] = static_cast<const uint16_t*>(head->w2);
  hb.b2[0] = static_cast<const uint16_t*>(head->b2);
  hb.wl[0] = static_cast<const uint16_t*>(head->wl);
  hb.x = static_cast<const uint16_t*>(x);
  hb.ids_now = ids_now;
  hb.ids_prev = ids_prev;
  hb.a = reinterpret_cast<float*>(ws + L.head_a);
  hb.res = reinterpret_cast<float*>(ws + L.head_res);
  hb.logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.head_logits);
  hb.counters = reinterpret_cast<uint32_t*>(ws + L.cnt_head);
  hb.ids_out = ids_out;
  hb.w_out = w_out;
  hb.err = reinterpret_cast<uint32_t*>(ws + L.err);
  hb.rule = route_rule(shape, route_bias);
  return launch_heads(hb, stream);
}

namespace e0 {
__global__ __launch_bounds__(64) void k_commit(const float* __restrict__ logits, int E, int K,
                                               RouteRule rr, int32_t* __restrict__ ids,
                                               float* __restrict__ w) {
  wave_commit<false>(logits, E, K, rr, ids, w);
}
}  // namespace e0

namespace e0 {
int launch_commit(const float* logits, int E, int K, const RouteRule& rr, int32_t* ids, float* w,
                  hipStream_t stream) {
  k_commit<<<1, 64, 0, stream>>>(logits, E, K, rr, ids, w);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
}  // namespace e0

extern "C" int edge0_route_commit(const edge0_moe_shape* shape, const float* logits,
                                  const float* route_bias, int32_t* ids_out, float* w_out,
                                  hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !logits || !ids_out || !w_out) return EDGE0_EINVAL;
  k_commit<<<1, 64, 0, stream>>>(logits, shape->n_experts, shape->top_k,
                                 route_rule(shape, route_bias), ids_out, w_out);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
