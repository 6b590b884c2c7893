// Internal helpers shared by the HIP kernels and the C ABI of libedge0.
// gfx950 (CDNA4): wave64, 160 KiB LDS per CU, 256 CUs in 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "edge0.h"

namespace e0 {

constexpr int kWave = 64;

// threadIdx.x through an empty asm: index arithmetic derived from it is
// recomputed where it is used instead of being hoisted out of a long loop
// and kept live (or spilled) across it
__device__ __forceinline__ int tid_here() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

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

// The nibble-pair mask and exponent word held in registers: a pair is then
// one v_and_or_b32 (a three-operand instruction, which cannot take two
// literal constants) instead of an AND and an OR.  Take them once per kernel
// section and pass them to every chunk_dot128 that shares a weight word, so
// the unpacked pairs are shared too.
struct Q4Consts {
  uint32_t m, c;
};
__device__ __forceinline__ Q4Consts q4_consts() {
  Q4Consts k{0x000F000Fu, 0x43004300u};
  asm volatile("" : "+v"(k.m), "+v"(k.c));
  return k;
}
__device__ __forceinline__ float chunk_dot128(uint4 q, const uint32_t* xp, Q4Consts k) {
  float acc = 0.f;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = dot2bf(((w[m] >> (4 * s)) & k.m) | k.c, xp[4 * m + s], acc);
  }
  return acc;
}

// Activation chunk `col` (32 bf16 of x): raw load, then the 16 pairs
// chunk_dot128 expects and its fp32 sum.
struct XRaw {
  uint4 v[4];
};
__device__ __forceinline__ void load_x_raw(const uint16_t* __restrict__ x, int col, XRaw& r) {
  const uint4* src = reinterpret_cast<const uint4*>(x + 32 * col);
#pragma unroll
  for (int m = 0; m < 4; ++m) r.v[m] = src[m];
}
__device__ __forceinline__ float x_pairs(const XRaw& r, uint32_t xp[16]) {
  const uint4* v = r.v;
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    pair_perm8(v[m].x, v[m].y, v[m].z, v[m].w, xp + 4 * m);
    sum += bf_lo(v[m].x) + bf_hi(v[m].x) + bf_lo(v[m].y) + bf_hi(v[m].y) + bf_lo(v[m].z) +
           bf_hi(v[m].z) + bf_lo(v[m].w) + bf_hi(v[m].w);
  }
  return sum;
}

// -------------------------------------------------------------- reductions
// DPP data movement within a wave (no LDS crossbar): quad permutes, row
// mirrors and the row broadcasts of GFX9.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}
// sum over each aligned group of 16 lanes, every lane of the group gets it
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(0.f, v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(0.f, v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(0.f, v);  // row_half_mirror
  v += dpp_f<0x140>(0.f, v);  // row_mirror
  return v;
}
// full-wave sum, the same value in every lane (fixed order)
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp_f<0x142, 0xa>(0.f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(0.f, v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Eight wave sums at once: halving exchanges across lane bits 5, 4, 3 (each
// lane keeps half of its values and adds its partner's copy of that half),
// then a sum over lane bits 0-2.  The sum of v[m] ends up in lanes 8m..8m+7.
__device__ __forceinline__ float wave_sums8(const float (&v)[8]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1;
  float w4[4], w2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = b5 ? v[4 + i] : v[i], send = b5 ? v[i] : v[4 + i];
    w4[i] = keep + __shfl_xor(send, 32, kWave);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = b4 ? w4[2 + i] : w4[i], send = b4 ? w4[i] : w4[2 + i];
    w2[i] = keep + __shfl_xor(send, 16, kWave);
  }
  const float keep = b3 ? w2[1] : w2[0], send = b3 ? w2[0] : w2[1];
  float w1 = keep + dpp_f<0x128>(0.f, send);  // row_ror:8 = lane ^ 8 within a row
  w1 += dpp_f<0xB1>(0.f, w1);                 // quad_perm [1,0,3,2]
  w1 += dpp_f<0x4E>(0.f, w1);                 // quad_perm [2,3,0,1]
  w1 += dpp_f<0x141>(0.f, w1);                // row_half_mirror
  return w1;
}

// sums over aligned segments of SEG lanes (8, 16 or 32); every lane of a
// segment gets the segment's sum
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
  v += dpp_f<0xB1>(0.f, v);
  v += dpp_f<0x4E>(0.f, v);
  v += dpp_f<0x141>(0.f, v);
  if constexpr (SEG >= 16) v += dpp_f<0x140>(0.f, v);
  if constexpr (SEG >= 32) {
    v += dpp_f<0x142, 0xa>(0.f, v);                    // lanes 31 and 63 hold the sums
    v = __shfl(v, (int)(threadIdx.x & 63) | 31, kWave);
  }
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

// Two-phase row dot for rows of up to 64*kPrefChunks*8 elements: the row's
// 16-byte chunks are loaded into registers first (so the loads are in flight
// while the caller prepares the vector), then dotted with a bf16 vector.
constexpr int kPrefChunks = 8;  // n <= 4096
struct RowPref {
  uint4 c[kPrefChunks];
};
__device__ __forceinline__ void row_prefetch(const uint16_t* __restrict__ w, int n, RowPref& p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nc = n >> 3;
#pragma unroll
  for (int m = 0; m < kPrefChunks; ++m) {
    const int c = lane + kWave * m;
    if (c < nc) p.c[m] = *reinterpret_cast<const uint4*>(w + 8 * c);
  }
}
// bf16 (or, with W_FP16, fp16) row (prefetched) . bf16 vector v (global or LDS)
template <bool W_FP16 = false>
__device__ __forceinline__ float row_dot_pref(const RowPref& p, const uint16_t* v, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nc = n >> 3;
  // every chunk of v this lane needs is requested before the first is used
  // (past the end at a clamped index), so the loads are in flight together
  // rather than one round trip each
  uint4 xv[kPrefChunks];
#pragma unroll
  for (int m = 0; m < kPrefChunks; ++m)
    if (kWave * m < nc) xv[m] = *reinterpret_cast<const uint4*>(v + 8 * min(lane + kWave * m, nc - 1));
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < kPrefChunks; ++m) {
    const int c = lane + kWave * m;
    if (kWave * m < nc && c < nc) {
      const uint4 xq = xv[m];
      const uint32_t ww[4] = {p.c[m].x, p.c[m].y, p.c[m].z, p.c[m].w};
      const uint32_t xx[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float w0 = W_FP16 ? h2f(ww[q] & 0xFFFFu) : bf_lo(ww[q]);
        const float w1 = W_FP16 ? h2f(ww[q] >> 16) : bf_hi(ww[q]);
        acc = fmaf(w0, bf_lo(xx[q]), acc);
        acc = fmaf(w1, bf_hi(xx[q]), acc);
      }
    }
  }
  return wave_sum(acc);
}

// Device-coherent stores and loads for data handed between workgroups of one
// kernel: agent-scope atomic accesses are performed at the device coherence
// point (across all XCDs), so no cache-wide write-back or invalidate is
// needed to publish or observe them.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ top-K
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
// Top-K ranking key: (value descending, index ascending) as one unsigned
// 64-bit order, larger first.  The value's bits are mapped to an order-
// preserving unsigned word (NaN ranks as -inf, -0 as +0); the low word is
// ~index, so of equal values the lower index ranks first.  0 is below every
// key and marks a taken element.
__device__ __forceinline__ unsigned long long topk_key(float x, int idx) {
  if (x != x) x = -INFINITY;
  if (x == 0.f) x = 0.f;
  uint32_t u = __float_as_uint(x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)~idx;
}
__device__ __forceinline__ float topk_value(unsigned long long key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ void keymax_dpp(unsigned long long& k) {
  const int hi = (int)(k >> 32), lo = (int)(uint32_t)k;
  const uint32_t ohi = (uint32_t)dpp_i<CTRL, ROW_MASK>(hi, hi);
  const uint32_t olo = (uint32_t)dpp_i<CTRL, ROW_MASK>(lo, lo);
  const unsigned long long o = ((unsigned long long)ohi << 32) | olo;
  k = o > k ? o : k;
}
// wave-wide largest key; every lane gets it
__device__ __forceinline__ unsigned long long wave_keymax(unsigned long long k) {
  keymax_dpp<0xB1>(k);        // quad_perm [1,0,3,2]
  keymax_dpp<0x4E>(k);        // quad_perm [2,3,0,1]
  keymax_dpp<0x141>(k);       // row_half_mirror
  keymax_dpp<0x140>(k);       // row_mirror
  keymax_dpp<0x142, 0xa>(k);  // row_bcast:15
  keymax_dpp<0x143, 0xc>(k);  // row_bcast:31
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(k >> 32), 63);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  return ((unsigned long long)hi << 32) | lo;
}

// Top-K of logits[0..E) by one wave, E <= 64 NPER: lane l ranks elements
// l + 64 j by key; each of the K picks is the wave's largest remaining key.
// Branch-free apart from the uniform loop over the picks.
template <int NPER, bool COHERENT>
__device__ __forceinline__ void wave_topk_n(const float* logits, int E, int K, int32_t* ids_out,
                                            float* w_out) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned long long key[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int idx = lane + kWave * j;
    float x = -INFINITY;
    if (idx < E) x = COHERENT ? ld_dev(logits + idx) : logits[idx];
    key[j] = idx < E ? topk_key(x, idx) : 0ull;  // past E: below every element
  }
  unsigned long long mine = 0;  // lane kk keeps the kk-th pick
  for (int kk = 0; kk < K; ++kk) {
    unsigned long long best = key[0];
#pragma unroll
    for (int j = 1; j < NPER; ++j) best = key[j] > best ? key[j] : best;
    best = wave_keymax(best);
#pragma unroll
    for (int j = 0; j < NPER; ++j) key[j] = key[j] == best ? 0ull : key[j];
    mine = lane == kk ? best : mine;
  }
  const float my_v = topk_value(mine);
  const int my_i = (int)~(uint32_t)mine;
  const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
  const float ex = lane < K ? expf(my_v - m) : 0.f;
  float den = 0.f;
  for (int j = 0; j < K; ++j)  // fixed order
    den += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < K) {
    ids_out[lane] = my_i;
    w_out[lane] = ex / den;
  }
}

// Top-K of logits[0..E) by one wave, ranked by (value descending, index
// ascending); NaN ranks as -inf.  Weights: w_k = exp(l_k - l_max) / sum over
// the selected.  Lanes < K write ids_out[lane], w_out[lane] (global or LDS).
// E <= 1024, K <= 16.  COHERENT: logits were written by other workgroups of
// the running kernel with st_dev, so they are read with ld_dev.
template <bool COHERENT>
__device__ __forceinline__ void wave_topk(const float* logits, int E, int K, int32_t* ids_out,
                                          float* w_out) {
  if (E <= 128) {
    wave_topk_n<2, COHERENT>(logits, E, K, ids_out, w_out);
  } else if (E <= 256) {
    wave_topk_n<4, COHERENT>(logits, E, K, ids_out, w_out);
  } else {
    wave_topk_n<16, COHERENT>(logits, E, K, ids_out, w_out);
  }
}

// Routing rule of a commit ([Edge0] App. A): kind 0 = softmax-top-K,
// kind 1 = sigmoid-group with n_groups contiguous groups of E / n_groups
// experts, top_groups of them surviving, weights scaled by `scale`, and an
// optional per-expert selection bias (fp32 [E], NULL = 0).
struct RouteRule {
  int kind;
  int n_groups, top_groups;
  float scale;
  const float* bias;
};

__device__ __forceinline__ float sigmoid_f(float l) { return 1.f / (1.f + expf(-l)); }

// Sigmoid-group commit by one wave ([Edge0] App. A "Sigmoid-group"; §2 "MoE
// routing"): sigma = sigmoid(l); selection score c = sigma + bias; a group's
// score is the sum of its two largest c; the top_groups groups survive
// (score descending, lower group first on ties); ids = the K largest c of
// the survivors (lower index first on ties), listed in rank order;
// w = scale * sigma[ids] / (sum of those sigma + 1e-20).  Decisions in fp32;
// NaN scores rank lowest.  E = NPER * 64 at most, n_groups <= 64, K <= 16,
// K <= top_groups * E / n_groups (checked by the caller).
template <int NPER, bool COHERENT>
__device__ __forceinline__ void wave_sigmoid_group_n(const float* logits, int E, int K,
                                                     const RouteRule& rr, int32_t* ids_out,
                                                     float* w_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = rr.n_groups, gs = E / n;
  auto score = [&](int e) {
    const float l = COHERENT ? ld_dev(logits + e) : logits[e];
    return sigmoid_f(l) + (rr.bias != nullptr ? rr.bias[e] : 0.f);
  };
  // group scores: lane i scans group i
  unsigned long long gkey = 0ull;
  if (lane < n) {
    float t1 = -INFINITY, t2 = -INFINITY;
    for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
      const float c = score(e);
      if (c > t1) {
        t2 = t1;
        t1 = c;
      } else if (c > t2) {
        t2 = c;
      }
    }
    gkey = topk_key(t1 + t2, lane);
  }
  unsigned long long alive = 0ull;  // bit i: group i survives
  for (int gg = 0; gg < rr.top_groups; ++gg) {
    const unsigned long long best = wave_keymax(gkey);
    alive |= 1ull << (int)~(uint32_t)best;
    gkey = gkey == best ? 0ull : gkey;
  }
  unsigned long long key[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int idx = lane + kWave * j;
    key[j] = (idx < E && ((alive >> (idx / gs)) & 1ull)) ? topk_key(score(idx), idx) : 0ull;
  }
  unsigned long long mine = 0;  // lane kk keeps the kk-th pick
  for (int kk = 0; kk < K; ++kk) {
    unsigned long long best = key[0];
#pragma unroll
    for (int j = 1; j < NPER; ++j) best = key[j] > best ? key[j] : best;
    best = wave_keymax(best);
#pragma unroll
    for (int j = 0; j < NPER; ++j) key[j] = key[j] == best ? 0ull : key[j];
    mine = lane == kk ? best : mine;
  }
  const int my_i = (int)~(uint32_t)mine;
  float sg = 0.f;
  if (lane < K) sg = sigmoid_f(COHERENT ? ld_dev(logits + my_i) : logits[my_i]);
  float den = 0.f;
  for (int j = 0; j < K; ++j)  // fixed order
    den += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sg), j));
  if (lane < K) {
    ids_out[lane] = my_i;
    w_out[lane] = rr.scale * sg / (den + 1e-20f);
  }
}

// The commit a rule names, by one wave (E <= 1024, K <= 16).
template <bool COHERENT>
__device__ __forceinline__ void wave_commit(const float* logits, int E, int K, const RouteRule& rr,
                                            int32_t* ids_out, float* w_out) {
  if (rr.kind == 0) {
    wave_topk<COHERENT>(logits, E, K, ids_out, w_out);
  } else if (E <= 128) {
    wave_sigmoid_group_n<2, COHERENT>(logits, E, K, rr, ids_out, w_out);
  } else if (E <= 256) {
    wave_sigmoid_group_n<4, COHERENT>(logits, E, K, rr, ids_out, w_out);
  } else {
    wave_sigmoid_group_n<16, COHERENT>(logits, E, K, rr, ids_out, w_out);
  }
}

// Weights of a routing whose ids are given: w_k = exp(l[id_k] - m) /
// sum_j exp(l[id_j] - m), m the largest of the K logits (g[ids] / sum g[ids]
// for g = softmax(l)).  Lanes 0..K-1 of one wave; an id outside [0, E) gets
// weight 0 and records EDGE0_ERANGE.
__device__ __forceinline__ void wave_softmax_at(const float* logits, const int32_t* ids, int E,
                                                int K, float* w_out, uint32_t* err) {
  const int lane = threadIdx.x & (kWave - 1);
  float v = -INFINITY;
  bool ok = true;
  if (lane < K) {
    const int id = ids[lane];
    ok = id >= 0 && id < E;
    if (ok) v = logits[id];
  }
  float m = -INFINITY;
  for (int j = 0; j < K; ++j) m = fmaxf(m, __shfl(v, j, kWave));
  const float ex = (lane < K && ok) ? expf(v - m) : 0.f;
  float den = 0.f;
  for (int j = 0; j < K; ++j) den += __shfl(ex, j, kWave);  // fixed order
  if (lane < K) w_out[lane] = den > 0.f ? ex / den : 0.f;
  if (lane < K && !ok) atomicOr(err, (uint32_t)(-EDGE0_ERANGE));
}

// Completion counting across workgroups.  Data that the last workgroup will
// read must have been written with st_dev.  Every wave waits for its stores
// to complete, the workgroup synchronises, and one atomic per workgroup
// counts the arrival.  Returns true (in every thread) in the workgroup whose
// arrival makes the count reach `target`; it then reads the others' data with
// ld_dev.  The caller resets the counter to zero when done.
__device__ __forceinline__ bool last_arrival(uint32_t* counter, uint32_t target) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == target - 1);
  }
  __syncthreads();
  return s_last != 0;
}

// Down-projection partial sums are accumulated in 64-bit fixed point (32
// fractional bits): integer addition is associative, so the sum is exact and
// the same in any arrival order.
constexpr float kFixScale = 4294967296.0f;  // 2^32
__device__ __forceinline__ unsigned long long to_fix(float v) {
  const float c = fminf(fmaxf(v * kFixScale, -9.2e18f), 9.2e18f);
  return (unsigned long long)__float2ll_rn(c);
}
// the value as fp32: hi * 2^32 + lo (two's complement words) is exact in fp64
// while |v| < 2^53 (|value| < 2^21), so the result is rounded once, as a
// direct 64-bit conversion would be; the scaling is a power of two
__device__ __forceinline__ float from_fix(unsigned long long v) {
  const double dv = fma((double)(int)(uint32_t)(v >> 32), 4294967296.0, (double)(uint32_t)v);
  return (float)(dv * (1.0 / kFixScale));
}

// x = bf16(h / sqrt(mean(h^2) + eps)) into LDS by one workgroup (fixed
// summation order, so every workgroup computes the same x)
__device__ __forceinline__ void rmsnorm_to_lds(const uint16_t* __restrict__ h, uint16_t* xs, int d,
                                               float eps) {
  __shared__ float red[256];
  float s = 0.f;
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    const float v = bf2f(h[j]);
    s = fmaf(v, v, s);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv = 1.f / sqrtf(red[0] / (float)d + eps);
  for (int j = threadIdx.x; j < d; j += blockDim.x) xs[j] = (uint16_t)f2bf(bf2f(h[j]) * inv);
  __syncthreads();
}

constexpr int kMaxD = 8192;

// ---------------------------------------------------------- error word
__device__ __forceinline__ void set_error(uint32_t* err, int code) {
  atomicOr(err, (uint32_t)(-code));
}

// ------------------------------------------------------------------ host
struct WsLayout {
  size_t err, cnt_router, cnt_head, cnt_down;     // u32 words / counters
  size_t logits, head_a, head_res;                // fp32
  size_t t_in;                                    // fp32 [K][2][r]
  size_t t_hand;                                  // fp32 [K][2r] LoRA A x handed between workgroups
  size_t lg_hand;                                 // fp32 [2][E] router logits handed between workgroups
  size_t gu_pre;                                  // fp32 [K][2][I] gate/up rows before LoRA
  size_t hp_hi, hp_lo;                            // u16 [K][I]
  size_t hs;                                      // fp32 [K][I/16]
  size_t tdpart;                                  // fp32 [K][I/16][r]
  size_t slots;                                   // int32 [K]
  size_t head_logits;                             // fp32 [E]
  size_t acc;                                     // int64 [2][d] fixed-point y
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
