// Routing kernels: the plain router GEMV, the prerouter head and the
// softmax-top-K commit.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction".  Routing math: §2 "MoE routing" and
// App. A "Softmax-topk"; head: §3.2 "Head", "Prediction-as-routing".
//
// The GEMVs here are small (router E x d bf16; head fc1 H x d fp16 plus the
// residual E x d, fc2 E x H) and HBM-bound: one wave per output row, 16-byte
// loads per lane, fp32 accumulation, a wave butterfly for the row sum.  The
// top-K runs in the last workgroup to finish (completion counter in the
// workspace), so a router or head call is one or two launches.
#include "common.h"

namespace e0 {

// ------------------------------------------------------------------ top-K
__device__ void wave_topk(const float* logits, int E, int K, int32_t* ids_out, float* w_out) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kMaxPer = 16;  // E <= 1024
  float v[kMaxPer];
  const int nper = (E + kWave - 1) / kWave;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int idx = lane + kWave * j;
    float x = -INFINITY;
    if (j < nper && idx < E) {
      x = ld_dev(logits + idx);
      if (x != x) x = -INFINITY;
    }
    v[j] = x;
  }
  uint32_t taken = 0;  // bit j: element lane + 64 j already selected
  float my_v = -INFINITY;  // lane kk keeps the kk-th selection
  int my_i = 0;
  for (int kk = 0; kk < K; ++kk) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      const int idx = lane + kWave * j;
      const bool ok = (j < nper) && (idx < E) && !((taken >> j) & 1u);
      if (ok && (v[j] > bv || (v[j] == bv && idx < bi))) {
        bv = v[j];
        bi = idx;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == kk) {
      my_v = bv;
      my_i = bi;
    }
  }
  const float m = __shfl(my_v, 0, kWave);
  const float ex = lane < K ? expf(my_v - m) : 0.f;
  float den = 0.f;
  for (int j = 0; j < K; ++j) den += __shfl(ex, j, kWave);  // fixed order
  if (lane < K) {
    ids_out[lane] = my_i;
    w_out[lane] = ex / den;
  }
}

// ---------------------------------------------------------------- router
// With h_norm set, every workgroup computes x = bf16(RMSNorm(h_norm)) into LDS
// and workgroup 0 stores it to x_out.
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ wr,
                                                const uint16_t* __restrict__ x_in,
                                                const uint16_t* __restrict__ h_norm,
                                                uint16_t* __restrict__ x_out, float eps, int d,
                                                int E, int K, float* __restrict__ logits,
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
    if (wave == 0) wave_topk(logits, E, K, ids, w);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ prerouter
// fc1 rows [0, H): a[h] = gelu(w1x[h] . x + sum of the one-hot columns + b1[h]);
// residual rows [H, H+E): res[e] = wl[e] . x
__global__ __launch_bounds__(256) void k_head_fc1(
    const uint16_t* __restrict__ w1x, const uint16_t* __restrict__ w1oh,
    const uint16_t* __restrict__ b1, const uint16_t* __restrict__ wl,
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids_now,
    const int32_t* __restrict__ ids_prev, int d, int E, int K, int H, float* __restrict__ a,
    float* __restrict__ res, uint32_t* __restrict__ err) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row < H) {
    float s = row_dot<true, false>(w1x + (size_t)row * d, x, d);
    // gather of the one-hot columns: lane j < K this token's ids, lane
    // K <= j < 2K the previous token's (block offset E)
    float g = 0.f;
    if (lane < 2 * K) {
      const bool prev = lane >= K;
      const int32_t* src = prev ? ids_prev : ids_now;
      if (src != nullptr) {
        const int id = src[prev ? lane - K : lane];
        if (id >= 0 && id < E) {
          g = h2f(w1oh[(size_t)(prev ? E + id : id) * H + row]);
        } else {
          set_error(err, EDGE0_ERANGE);
        }
      }
    }
    // fixed-order sum of the gathered columns (lanes 0..2K-1 in order)
    float gs = 0.f;
    for (int j = 0; j < 2 * K; ++j) gs += __shfl(g, j, kWave);
    s += gs;
    if (b1 != nullptr) s += h2f(b1[row]);
    if (lane == 0) a[row] = 0.5f * s * (1.f + erff(s * 0.70710678118654752440f));
  } else if (wl != nullptr && row < H + E) {
    const int e = row - H;
    const float s = row_dot<true, false>(wl + (size_t)e * d, x, d);
    if (lane == 0) res[e] = s;
  }
}

// logits[e] = w2[e] . a + b2[e] + res[e]; then top-K in the last workgroup
__global__ __launch_bounds__(256) void k_head_fc2(
    const uint16_t* __restrict__ w2, const uint16_t* __restrict__ b2,
    const float* __restrict__ a, const float* __restrict__ res, int E, int K, int H,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w,
    uint32_t* __restrict__ counter) {
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row < E) {
    float s = row_dot<true, true>(w2 + (size_t)row * H, a, H);
    if (b2 != nullptr) s += h2f(b2[row]);
    if (res != nullptr) s += res[row];
    if ((threadIdx.x & 63) == 0) st_dev(logits + row, s);
  }
  if (last_arrival(counter, gridDim.x)) {
    if (wave == 0) wave_topk(logits, E, K, ids, w);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace e0

using namespace e0;

namespace e0 {
int launch_router(const edge0_moe_shape* shape, const void* w_router, const void* x,
                  const uint16_t* h_norm, uint16_t* x_out, float eps, float* logits_out,
                  int32_t* ids_out, float* w_out, void* workspace, hipStream_t stream) {
  const WsLayout L = ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.logits);
  const int E = shape->n_experts;
  k_router<<<(E + 3) / 4, 256, 0, stream>>>(
      static_cast<const uint16_t*>(w_router), static_cast<const uint16_t*>(x), h_norm, x_out, eps,
      shape->d_model, E, shape->top_k, logits, ids_out, w_out,
      reinterpret_cast<uint32_t*>(ws + L.cnt_router));
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
}  // namespace e0

extern "C" int edge0_router(const edge0_moe_shape* shape, const void* w_router, const void* x,
                            float* logits_out, int32_t* ids_out, float* w_out, void* workspace,
                            hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !w_router || !x || !ids_out || !w_out || !workspace)
    return EDGE0_EINVAL;
  return launch_router(shape, w_router, x, nullptr, nullptr, 0.f, logits_out, ids_out, w_out,
                       workspace, stream);
}

extern "C" int edge0_prerouter(const edge0_moe_shape* shape, const edge0_head* head,
                               const void* x, const int32_t* ids_now, const int32_t* ids_prev,
                               float* logits_out, int32_t* ids_out, float* w_out,
                               void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !head || !head->w1x || !head->w1oh || !head->w2 || !x ||
      !ids_now || !ids_out || !w_out || !workspace || shape->head_hidden <= 0)
    return EDGE0_EINVAL;
  const WsLayout L = ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.head_logits);
  float* a = reinterpret_cast<float*>(ws + L.head_a);
  float* res = reinterpret_cast<float*>(ws + L.head_res);
  const int d = shape->d_model, E = shape->n_experts, K = shape->top_k, H = shape->head_hidden;
  const int rows1 = H + (head->wl ? E : 0);
  k_head_fc1<<<(rows1 + 3) / 4, 256, 0, stream>>>(
      static_cast<const uint16_t*>(head->w1x), static_cast<const uint16_t*>(head->w1oh),
      static_cast<const uint16_t*>(head->b1), static_cast<const uint16_t*>(head->wl),
      static_cast<const uint16_t*>(x), ids_now, ids_prev, d, E, K, H, a, res,
      reinterpret_cast<uint32_t*>(ws + L.err));
  E0_CHECK_LAUNCH();
  k_head_fc2<<<(E + 3) / 4, 256, 0, stream>>>(
      static_cast<const uint16_t*>(head->w2), static_cast<const uint16_t*>(head->b2), a,
      head->wl ? res : nullptr, E, K, H, logits, ids_out, w_out,
      reinterpret_cast<uint32_t*>(ws + L.cnt_head));
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
