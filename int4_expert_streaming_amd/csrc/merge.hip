// Merging the LoRA into the int4 weights, the alternative the pages reject:
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction", §3.3 "Recovery LoRA: Unmerged by
// Design" and its footnote 2.  The LoRA delta (alpha/r) B A is added to the
// dequantised weight and the sum is requantised to int4 with the format's
// affine scheme; what survives is measured as sum(actual * delta) /
// sum(delta^2) per projection.
//
// One thread per (projection, row, group of g inputs): it rebuilds the
// group's weights s q + b (exact in fp32), adds delta (r products of bf16
// factors, summed in rank order in fp32), takes the group's min and max,
// rounds s' = (max - min) / 15 and b' = min to bf16 (nearest, ties to even),
// codes q' = round((w - b') / s') to nearest-even clipped to 0..15 (q' = 0
// when s' is 0), writes them into the merged bundle (the LoRA-free layout
// of the same shape), and keeps sum(actual delta) and sum(delta^2) of its
// group in fp64.  Each workgroup writes its six partial sums; one more
// launch adds them in workgroup order, so the figures do not depend on
// scheduling.
#include "moe_internal.h"

namespace e0 {

constexpr int kMergeThreads = 256;

struct MergeArgs {
  const uint8_t* src;  // bundle with its LoRA
  uint8_t* dst;        // bundle in the LoRA-free layout
  edge0_bundle_layout ls, ld;
  int d, I, g, r;
  float scale;
  int n_gate, n_up, n_down;  // groups per projection
  double* partial;           // [gridDim][6]
};

// word w (8 inputs) of group G of row o: index into the projection's u32
// array (row-major [out][in/8] for gate/up, 1 KiB tiles [d/64][I/32][64][4]
// for down)
__device__ __forceinline__ size_t merge_word(int proj, int o, int G, int w, int d, int I, int g) {
  const int j = G * g + 8 * w;  // first input of the word
  if (proj < 2) return (size_t)o * (d / 8) + (size_t)(j >> 3);
  return (((size_t)(o >> 6) * (I / 32) + (j >> 5)) * 64 + (o & 63)) * 4 + ((j & 31) >> 3);
}

__global__ __launch_bounds__(kMergeThreads) void k_merge_requant(MergeArgs a) {
  __shared__ double red[kMergeThreads / 64][6];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * kMergeThreads + tid;
  const int d = a.d, I = a.I, g = a.g, r = a.r;
  double sad = 0.0, sdd = 0.0;
  int proj = -1;
  if (t < a.n_gate + a.n_up + a.n_down) {
    proj = t < a.n_gate ? 0 : (t < a.n_gate + a.n_up ? 1 : 2);
    const int u = t - (proj == 0 ? 0 : (proj == 1 ? a.n_gate : a.n_gate + a.n_up));
    const int n_in = proj < 2 ? d : I;  // inputs per row
    const int gpr = n_in / g;           // groups per row
    const int o = u / gpr, G = u % gpr; // row, group
    const edge0_bundle_layout& ls = a.ls;
    const edge0_bundle_layout& ld = a.ld;
    const int64_t oq = proj == 0 ? ls.gate_q : (proj == 1 ? ls.up_q : ls.down_q);
    const int64_t os = proj == 0 ? ls.gate_s : (proj == 1 ? ls.up_s : ls.down_s);
    const int64_t ob = proj == 0 ? ls.gate_b : (proj == 1 ? ls.up_b : ls.down_b);
    const int64_t dq = proj == 0 ? ld.gate_q : (proj == 1 ? ld.up_q : ld.down_q);
    const int64_t ds = proj == 0 ? ld.gate_s : (proj == 1 ? ld.up_s : ld.down_s);
    const int64_t db = proj == 0 ? ld.gate_b : (proj == 1 ? ld.up_b : ld.down_b);
    const int64_t oa = proj == 0 ? ls.a_gate : (proj == 1 ? ls.a_up : ls.a_down);
    const int64_t obb = proj == 0 ? ls.b_gate : (proj == 1 ? ls.b_up : ls.b_down);
    const uint32_t* qs = reinterpret_cast<const uint32_t*>(a.src + oq);
    uint32_t* qd = reinterpret_cast<uint32_t*>(a.dst + dq);
    const size_t si = proj < 2 ? (size_t)o * gpr + G : (size_t)G * d + o;  // scale/bias index
    const uint16_t* A = r > 0 ? reinterpret_cast<const uint16_t*>(a.src + oa) : nullptr;
    const uint16_t* B = r > 0 ? reinterpret_cast<const uint16_t*>(a.src + obb) + (size_t)o * r : nullptr;
    const float s = bf2f(reinterpret_cast<const uint16_t*>(a.src + os)[si]);
    const float b = bf2f(reinterpret_cast<const uint16_t*>(a.src + ob)[si]);
    // delta of input i (fp32, rank order), the same in both passes
    auto delta = [&](int i) {
      float dl = 0.f;
      for (int k = 0; k < r; ++k) dl += bf2f(B[k]) * bf2f(A[(size_t)k * n_in + i]);
      return dl * a.scale;
    };
    const int nw = g / 8;
    float lo = INFINITY, hi = -INFINITY;
    for (int w = 0; w < nw; ++w) {
      const uint32_t word = qs[merge_word(proj, o, G, w, d, I, g)];
      for (int e = 0; e < 8; ++e) {
        const float Wm = (s * (float)((word >> (4 * e)) & 15u) + b) + delta(G * g + 8 * w + e);
        lo = fminf(lo, Wm);
        hi = fmaxf(hi, Wm);
      }
    }
    const uint32_t s2b = f2bf((hi - lo) / 15.f), b2b = f2bf(lo);
    const float s2 = bf2f(s2b), b2 = bf2f(b2b);
    reinterpret_cast<uint16_t*>(a.dst + ds)[si] = (uint16_t)s2b;
    reinterpret_cast<uint16_t*>(a.dst + db)[si] = (uint16_t)b2b;
    for (int w = 0; w < nw; ++w) {
      const size_t wi = merge_word(proj, o, G, w, d, I, g);
      const uint32_t word = qs[wi];
      uint32_t out = 0;
      for (int e = 0; e < 8; ++e) {
        const float W = s * (float)((word >> (4 * e)) & 15u) + b;  // exact
        const float dl = delta(G * g + 8 * w + e);
        const float Wm = W + dl;
        float qf = s2 > 0.f ? rintf((Wm - b2) / s2) : 0.f;
        qf = fminf(fmaxf(qf, 0.f), 15.f);
        const uint32_t q2 = (uint32_t)qf;
        out |= q2 << (4 * e);
        const double act = ((double)s2 * (double)q2 + (double)b2) - (double)W;
        sad += act * (double)dl;
        sdd += (double)dl * (double)dl;
      }
      qd[wi] = out;
    }
  }
  // per-projection sums of the workgroup, in lane then wave order
  double v[6];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    v[2 * p] = proj == p ? sad : 0.0;
    v[2 * p + 1] = proj == p ? sdd : 0.0;
  }
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    double x = v[q];
    for (int o2 = 32; o2 >= 1; o2 >>= 1) x += __shfl_xor(x, o2, kWave);
    if (lane == 0) red[wave][q] = x;
  }
  __syncthreads();
  if (tid < 6) {
    double x = 0.0;
    for (int w2 = 0; w2 < kMergeThreads / 64; ++w2) x += red[w2][tid];
    a.partial[(size_t)blockIdx.x * 6 + tid] = x;
  }
}

__global__ void k_merge_sum(const double* partial, int n, double* out) {
  if (threadIdx.x < 6) {
    double x = 0.0;
    for (int i = 0; i < n; ++i) x += partial[(size_t)i * 6 + threadIdx.x];
    out[threadIdx.x] = x;
  }
}

}  // namespace e0

using namespace e0;

extern "C" size_t edge0_merge_workspace_bytes(const edge0_moe_shape* shape) {
  if (!shape || !shape_ok(shape)) return 0;
  const size_t groups = (size_t)shape->d_inter * (shape->d_model / shape->group_size) * 2 +
                        (size_t)shape->d_model * (shape->d_inter / shape->group_size);
  return ((groups + kMergeThreads - 1) / kMergeThreads) * 6 * sizeof(double);
}

extern "C" int edge0_merge_requant(const edge0_moe_shape* shape, const void* src_bundle,
                                   void* dst_bundle, double* stats_out, void* workspace,
                                   hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !src_bundle || !dst_bundle ||
      !stats_out || !workspace || src_bundle == dst_bundle)
    return EDGE0_EINVAL;
  MergeArgs a{};
  edge0_moe_shape s0 = *shape;
  s0.lora_rank = 0;
  if (bundle_layout(shape, &a.ls) != EDGE0_OK || bundle_layout(&s0, &a.ld) != EDGE0_OK)
    return EDGE0_EINVAL;
  a.src = static_cast<const uint8_t*>(src_bundle);
  a.dst = static_cast<uint8_t*>(dst_bundle);
  a.d = shape->d_model;
  a.I = shape->d_inter;
  a.g = shape->group_size;
  a.r = shape->lora_rank;
  a.scale = a.r > 0 ? shape->lora_alpha / (float)a.r : 0.f;
  a.n_gate = a.I * (a.d / a.g);
  a.n_up = a.n_gate;
  a.n_down = a.d * (a.I / a.g);
  a.partial = static_cast<double*>(workspace);
  const int n = a.n_gate + a.n_up + a.n_down;
  const int grid = (n + kMergeThreads - 1) / kMergeThreads;
  k_merge_requant<<<grid, kMergeThreads, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  k_merge_sum<<<1, 64, 0, stream>>>(a.partial, grid, stats_out);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
