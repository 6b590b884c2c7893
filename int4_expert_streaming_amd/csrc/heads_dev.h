// Prerouter head rows ([Edge0] = "The Other Half of the Memory Wall: Serving
// 35B MoEs from SSD with Trained Routing Prediction", §3.2 "Head",
// "Prediction-as-routing"), shared by the batched head kernels and the
// stack's folded head schedule, which runs the fc1 rows as workgroups of
// the down projections' launches.
#pragma once
#include "moe_internal.h"

namespace e0 {

__device__ __forceinline__ float gelu_erf_f(float z) {
  return 0.5f * z * (1.f + erff(z * 0.70710678118654752440f));
}

// One wave: fc1 row `row` of head h.  Rows [0, H): a[row] = gelu(w1x[row] .
// x + the one-hot columns of this token's and the previous token's ids +
// b1[row]); rows [H, H+E) when the head has the residual: res[row - H] =
// wl[row - H] . x.  Other rows do nothing.
// NCH > 0: d = 512 NCH, lane l takes the row's 16-byte chunks l + 64 m; the
// loads go out in this order, fenced so the compiler keeps it (loads return
// in order): the ids, the row, the one-hot columns the ids select, then x
// and b1, so the columns are read while the row is in flight and nothing
// waits before every load is issued.  NCH = 0: any d (the generic row dot).
template <int NCH>
__device__ __forceinline__ void head_fc1_row_t(const HeadPart& h, int row) {
  const int lane = threadIdx.x & 63;
  const int H = h.H, E = h.E, K = h.K, d = h.d;
  const bool fc1 = row < H;
  const bool resrow = !fc1 && h.has_res && row < H + E;
  if (!fc1 && !resrow) return;
  const uint16_t* wrow = fc1 ? h.w1x + (size_t)row * d : h.wl + (size_t)(row - H) * d;
  // one-hot columns: lane j < K this token's ids, K <= j < 2K the previous
  // token's (block offset E)
  const bool prev = lane >= K;
  const int32_t* src = prev ? h.ids_prev : h.ids_now;
  int id = -1;
  if (fc1 && lane < 2 * K && src != nullptr) id = src[prev ? lane - K : lane];
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  uint4 wv[NCH > 0 ? NCH : 1];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int m = 0; m < NCH; ++m) wv[m] = reinterpret_cast<const uint4*>(wrow)[lane + 64 * m];
  }
  // the lane's column entry (fp16 bits), read at a clamped id by every lane
  // and kept only where it adds a column (no branch around the load, so
  // nothing waits for it before x is requested)
  // (on every row: a residual row's entry is read at row H - 1 and dropped)
  // the blocks are binary multi-hots, so an id listed twice in one block
  // sets its entry once: only its first listing in that block adds the column
  bool first = true;
  for (int j = 0; j < 2 * K; ++j) {
    const int other = __shfl(id, j, kWave);
    if (j < lane && (j >= K) == prev && other == id) first = false;
  }
  const bool listed = fc1 && lane < 2 * K && first && src != nullptr;
  const bool in = id >= 0 && id < E;
  if (listed && !in) set_error(h.err, EDGE0_ERANGE);
  const bool adds = listed && in;
  const int idc = min(max(id, 0), E - 1);
  const uint32_t graw = h.w1oh[(size_t)(prev ? E + idc : idc) * H + min(row, H - 1)];
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // b1 read on every row (a valid address when there is none; dropped then)
  const uint32_t b1raw = *(h.b1 != nullptr ? h.b1 + min(row, H - 1) : h.w1oh);
  float s;
  if constexpr (NCH > 0) {
    uint4 xv[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) xv[m] = reinterpret_cast<const uint4*>(h.x)[lane + 64 * m];
    asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const uint32_t ww[4] = {wv[m].x, wv[m].y, wv[m].z, wv[m].w};
      const uint32_t xx[4] = {xv[m].x, xv[m].y, xv[m].z, xv[m].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(h2f(ww[q] & 0xFFFFu), bf_lo(xx[q]), acc);
        acc = fmaf(h2f(ww[q] >> 16), bf_hi(xx[q]), acc);
      }
    }
    s = wave_sum(acc);
  } else {
    s = row_dot<true, false>(wrow, h.x, d);
  }
  if (fc1) {
    const float g = adds ? h2f(graw) : 0.f;
    float gs = 0.f;
    for (int j = 0; j < 2 * K; ++j) gs += __shfl(g, j, kWave);  // fixed order
    const float b1 = h.b1 != nullptr ? h2f(b1raw) : 0.f;
    if (lane == 0) h.a[row] = gelu_erf_f(s + (gs + b1));
  } else {
    if (lane == 0) h.res[row - H] = s;
  }
}
__device__ __forceinline__ void head_fc1_row(const HeadPart& h, int row) {
  switch (h.d) {
    case 2048: head_fc1_row_t<4>(h, row); break;
    case 4096: head_fc1_row_t<8>(h, row); break;
    default: head_fc1_row_t<0>(h, row); break;
  }
}

// One wave: fc2 rows rb .. rb + 7 of head h, logits[e] = w2[e] . a + b2[e]
// + res[e], stored device-coherent for the commit.  One 16-byte chunk of
// each fp16 row per lane, the 8 row sums reduced together.
__device__ __forceinline__ void head_fc2_rows(const HeadPart& h, int rb) {
  const int lane = threadIdx.x & 63;
  const int H = h.H, E = h.E;
  if (rb >= E) return;
  const int nch = H / 8;  // 16-byte chunks per row
  float v[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) v[m] = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const float4 a0 = reinterpret_cast<const float4*>(h.a + 8 * c)[0];
    const float4 a1 = reinterpret_cast<const float4*>(h.a + 8 * c)[1];
    uint4 q[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      q[m] = rb + m < E ? reinterpret_cast<const uint4*>(h.w2 + (size_t)(rb + m) * H)[c]
                        : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float s = v[m];
      s = fmaf(h2f(q[m].x & 0xFFFFu), a0.x, s);
      s = fmaf(h2f(q[m].x >> 16), a0.y, s);
      s = fmaf(h2f(q[m].y & 0xFFFFu), a0.z, s);
      s = fmaf(h2f(q[m].y >> 16), a0.w, s);
      s = fmaf(h2f(q[m].z & 0xFFFFu), a1.x, s);
      s = fmaf(h2f(q[m].z >> 16), a1.y, s);
      s = fmaf(h2f(q[m].w & 0xFFFFu), a1.z, s);
      s = fmaf(h2f(q[m].w >> 16), a1.w, s);
      v[m] = s;
    }
  }
  // row rb + m ends up in lane 8 m
  const float sum = wave_sums8(v);
  if ((lane & 7) == 0) {
    const int e = rb + (lane >> 3);
    if (e < E) {
      float s = sum;
      if (h.b2 != nullptr) s += h2f(h.b2[e]);
      if (h.has_res) s += h.res[e];
      st_dev(h.logits + e, s);
    }
  }
}

// Workgroup `part` of the `parts` that cover head h's fc2 (8 rows per wave),
// then the commit of the head's routing by the last of them to finish
// (completion counter, reset by that workgroup).  Every thread of the
// workgroup calls it.
__device__ __forceinline__ void head_fc2_part(const HeadPart& h, int part, int parts) {
  const int waves = blockDim.x / 64, wave = threadIdx.x >> 6;
  head_fc2_rows(h, (part * waves + wave) * 8);
  if (last_arrival(h.counter, parts)) {
    if (wave == 0) wave_commit<true>(h.logits, h.E, h.K, h.rule, h.ids_out, h.w_out);
    if (threadIdx.x == 0) __hip_atomic_store(h.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace e0
