// Internal helpers shared by the HIP kernels and the C ABI of libedge0.
// gfx950 (CDNA4): wave64, 160 KiB LDS per CU, 256 CUs in 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "edge0.h"

namespace e0 {

constexpr int kWave = 64;

// ------------------------------------------------------------------ dtypes
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float h2f(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
// a.lo*b.lo + a.hi*b.hi + c with bf16 operands and fp32 accumulation
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// int4 nibble pairs as exact bf16 "128 + q": for s in 0..3 the pair holds
// (element 8m+s, element 8m+s+4) of word m.  0x4300 is bf16 128.0 and q < 16
// fills the low mantissa bits, so the value is exactly 128 + q.
__device__ __forceinline__ uint32_t q4pair(uint32_t word, int s) {
  return ((word >> (4 * s)) & 0x000F000Fu) | 0x43004300u;
}

// Activation pairs matching q4pair: from the raw bf16 words of 8 consecutive
// elements w0=(x0,x1) w1=(x2,x3) w2=(x4,x5) w3=(x6,x7) build (x0,x4),
// (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ void pair_perm8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                           uint32_t out[4]) {
  // v_perm_b32(a, b, sel): bytes 0-3 from b, 4-7 from a
  out[0] = __builtin_amdgcn_perm(w2, w0, 0x05040100u);  // lo(w0), lo(w2)
  out[1] = __builtin_amdgcn_perm(w2, w0, 0x07060302u);  // hi(w0), hi(w2)
  out[2] = __builtin_amdgcn_perm(w3, w1, 0x05040100u);  // lo(w1), lo(w3)
  out[3] = __builtin_amdgcn_perm(w3, w1, 0x07060302u);  // hi(w1), hi(w3)
}

// Sum over the 32 inputs of one 16-byte chunk of packed weights against the
// matching 16 activation pairs: returns sum (128 + q_i) * x_i.
__device__ __forceinline__ float chunk_dot128(uint4 q, const uint32_t* xp) {
  float acc = 0.f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = dot2bf(q4pair(w[m], s), xp[4 * m + s], acc);
  }
  return acc;
}

// -------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// sums over aligned segments of `seg` lanes (power of two); every lane of a
// segment gets the segment's sum
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = SEG / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// -------------------------------------------------------------- row dots
// One wave: sum_j w[j] * v[j] over n elements (n % 8 == 0); w is bf16 or
// fp16, v is bf16 or fp32.  Every lane returns the (identical) total.
template <bool W_FP16, bool V_F32>
__device__ __forceinline__ float row_dot(const uint16_t* __restrict__ w, const void* __restrict__ v,
                                         int n) {
  const int lane = threadIdx.x & (kWave - 1);
  float acc = 0.f;
  const int nc = n >> 3;
  for (int c = lane; c < nc; c += kWave) {
    const uint4 wq = *reinterpret_cast<const uint4*>(w + 8 * c);
    const uint32_t ww[4] = {wq.x, wq.y, wq.z, wq.w};
    float vf[8];
    if (V_F32) {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(v) + 8 * c);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(v) + 8 * c + 4);
      vf[0] = a.x; vf[1] = a.y; vf[2] = a.z; vf[3] = a.w;
      vf[4] = b.x; vf[5] = b.y; vf[6] = b.z; vf[7] = b.w;
    } else {
      const uint4 xq = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v) + 8 * c);
      const uint32_t xx[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        vf[2 * m] = bf_lo(xx[m]);
        vf[2 * m + 1] = bf_hi(xx[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float w0, w1;
      if (W_FP16) {
        w0 = h2f(ww[m] & 0xFFFFu);
        w1 = h2f(ww[m] >> 16);
      } else {
        w0 = bf_lo(ww[m]);
        w1 = bf_hi(ww[m]);
      }
      acc = fmaf(w0, vf[2 * m], acc);
      acc = fmaf(w1, vf[2 * m + 1], acc);
    }
  }
  return wave_sum(acc);
}

// Top-K of logits[0..E) by one wave, ranked by (value descending, index
// ascending); NaN ranks as -inf.  Weights: w_k = exp(l_k - l_max) / sum over
// the selected.  Lane 0 writes ids_out[K], w_out[K].  E <= 1024, K <= 16.
__device__ void wave_topk(const float* logits, int E, int K, int32_t* ids_out, float* w_out);

// Completion counting across workgroups: every thread fences its global
// stores, then one atomic per workgroup.  Returns true (in every thread) in
// the workgroup whose arrival makes the count reach `target`; that workgroup
// then sees all stores the others made before arriving.  The caller resets
// the counter to zero when done.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t target) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(counter, 1u);
    s_last = (old == target - 1);
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------- error word
__device__ __forceinline__ void set_error(uint32_t* err, int code) {
  atomicOr(err, (uint32_t)(-code));
}

// ------------------------------------------------------------------ host
struct WsLayout {
  size_t err, cnt_router, cnt_head, cnt_down;     // u32 words / counters
  size_t logits, head_a, head_res;                // fp32
  size_t t_in;                                    // fp32 [K][2][r]
  size_t hf;                                      // fp32 [K][I]
  size_t hp_hi, hp_lo;                            // u16 [K][I]
  size_t hs;                                      // fp32 [K][I/16]
  size_t tdpart;                                  // fp32 [K][I/16][r]
  size_t dpart;                                   // fp32 [d/64][K][I/32][64]
  size_t total;
};

bool shape_ok(const edge0_moe_shape* s);
WsLayout ws_layout(const edge0_moe_shape* s);
int bundle_layout(const edge0_moe_shape* s, edge0_bundle_layout* out);
int hip_status(hipError_t e);

#define E0_CHECK_LAUNCH()                                 \
  do {                                                    \
    hipError_t _e = hipGetLastError();                    \
    if (_e != hipSuccess) return EDGE0_EHIP;              \
  } while (0)

}  // namespace e0
