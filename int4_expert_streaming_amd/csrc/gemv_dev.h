// Device helpers of the int4 gate/up GEMV shared by the per-layer kernels
// and the persistent step kernel: the wide-row weight loads, the batched
// wave reductions and the SwiGLU row epilogue.
#pragma once

#include "moe_internal.h"

namespace e0 {

// position of element i of h in the pair-permuted order of its 8-group
__device__ __forceinline__ int pair_pos(int i) {
  const int s = i & 7;
  return (i & ~7) + (s < 4 ? 2 * s : 2 * (s - 4) + 1);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

// store one row of h as its bf16 hi/lo split (hi = bf16(h), lo = bf16(h - hi));
// returns hi + lo, the value the down GEMV sees
__device__ __forceinline__ float store_h(const MoeArgs& a, int k, int i, float h) {
  const uint32_t hi = f2bf(h);
  const uint32_t lo = f2bf(h - bf2f(hi));
  const size_t base = (size_t)k * a.I;
  a.hp_hi[base + pair_pos(i)] = (uint16_t)hi;
  a.hp_lo[base + pair_pos(i)] = (uint16_t)lo;
  return bf2f(hi) + bf2f(lo);
}

// Wide rows (d >= 2048): 8 waves of 2 row pairs per 16-row workgroup (two
// waves per SIMD hide each other's latency); narrow rows: 4 waves.
constexpr int kWideRowsPerWave = 2;
constexpr int gate_up_threads(int cpr) { return cpr >= 64 ? 64 * 16 / kWideRowsPerWave : 256; }

// Wide rows: d/32 = 64*NJ chunks per row; lane l owns chunks l + 64 j of both
// the gate and the up row of the wave's R row pairs.  gu_load issues every
// weight load of the wave (int4 words, scales, biases, LoRA B rows);
// gu_finish takes x (global or LDS) and the lane's LoRA t, and computes.
template <int NJ, int RR = kWideRowsPerWave>
struct GuW {
  static constexpr int R = RR;
  uint4 qg[R][NJ], qu[R][NJ];
  uint32_t sg[R][NJ], bg[R][NJ], su[R][NJ], bu[R][NJ];
  uint32_t Bg[R], Bu[R];
};

// `wave` selects the rows (R * wave ..): a wave that only needs the loads
// issued in order (not their values) passes the index of another wave
template <int NJ, int RR = kWideRowsPerWave>
__device__ __forceinline__ void gu_load(const MoeArgs& a, const uint8_t* b, int i0,
                                        GuW<NJ, RR>& w, int wave = tid_here() >> 6, int k = 0,
                                        int e = -1) {
  constexpr int R = RR;
  const int lane = tid_here() & 63;
  const int d = a.d, g = a.g, ng = d / g, r = a.r;
  const int row0 = i0 + R * wave;
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s);
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(b + a.lay.up_s);
  const uint16_t* ub = reinterpret_cast<const uint16_t*>(b + a.lay.up_b);
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    const int row = row0 + ii;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = lane + 64 * j;
      w.qg[ii][j] = reinterpret_cast<const uint4*>(gq + (size_t)row * (d / 8))[col];
      w.qu[ii][j] = reinterpret_cast<const uint4*>(uq + (size_t)row * (d / 8))[col];
      const int grp = (32 * col) / g;
      w.sg[ii][j] = gs[row * ng + grp];
      w.bg[ii][j] = gb[row * ng + grp];
      w.su[ii][j] = us[row * ng + grp];
      w.bu[ii][j] = ub[row * ng + grp];
    }
  }
  // LoRA: lane rr < r holds B[row][rr] of the R rows (r <= 64).  Loaded
  // without a branch (lanes >= r, or r = 0, read an in-bundle word that is
  // never used), so no control flow separates these loads from their uses.
  const int rc = r > 0 ? r : 1;
  // (adapters given apart: expert e's, or routed expert k's when e < 0)
  const uint16_t* Bgp = reinterpret_cast<const uint16_t*>(
      r > 0 ? E0_LORA_E(a, b, (e >= 0 ? e : (a).ids[k]), 1, a.lay.b_gate) : b);
  const uint16_t* Bup = reinterpret_cast<const uint16_t*>(
      r > 0 ? E0_LORA_E(a, b, (e >= 0 ? e : (a).ids[k]), 3, a.lay.b_up) : b);
  const int rl = lane % rc;
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    w.Bg[ii] = Bgp[(size_t)(row0 + ii) * rc + rl];
    w.Bu[ii] = Bup[(size_t)(row0 + ii) * rc + rl];
  }
}

// Sums of 2R per-lane values over the wave at once: halving exchanges across
// the top lane bits (each lane keeps half of its values and adds its
// partner's copy of that half), then a sum over the remaining low lane bits.
// Value v is then in lane (64 / 2R) * v.
template <int R>
__device__ __forceinline__ float wave_sums_2r(const float (&v)[2 * R]) {
  const int lane = tid_here() & 63;
  const int b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1;
  float w1;
  if constexpr (R == 1) {
    const float keep = b5 ? v[1] : v[0], send = b5 ? v[0] : v[1];
    w1 = row16_sum(keep + __shfl_xor(send, 32, kWave));
    w1 += __shfl_xor(w1, 16, kWave);
  } else if constexpr (R == 2) {
    float w2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b5 ? v[2 + i] : v[i], send = b5 ? v[i] : v[2 + i];
      w2[i] = keep + __shfl_xor(send, 32, kWave);
    }
    const float keep = b4 ? w2[1] : w2[0], send = b4 ? w2[0] : w2[1];
    w1 = row16_sum(keep + __shfl_xor(send, 16, kWave));
  } else {
    static_assert(R == 4, "1, 2 or 4");
    const int b3 = (lane >> 3) & 1;
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
    w1 = keep + dpp_f<0x128>(0.f, send);  // row_ror:8 = lane ^ 8 within a row
    w1 += dpp_f<0xB1>(0.f, w1);   // quad_perm [1,0,3,2]
    w1 += dpp_f<0x4E>(0.f, w1);   // quad_perm [2,3,0,1]
    w1 += dpp_f<0x141>(0.f, w1);  // row_half_mirror
  }
  return w1;
}

// Per-lane partials of the wave's R gate rows (v[0..R-1]) and R up rows
// (v[R..2R-1]) on x (global or LDS), without the LoRA term.
template <int NJ, int RR>
__device__ __forceinline__ void gu_base(const GuW<NJ, RR>& w, const uint16_t* xsrc,
                                        float (&v)[2 * RR]) {
  constexpr int R = RR;
  const int lane = tid_here() & 63;
  XRaw xr[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) load_x_raw(xsrc, lane + 64 * j, xr[j]);
  uint32_t xp[NJ][16];
  float X[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) X[j] = x_pairs(xr[j], xp[j]);
  const Q4Consts kq = q4_consts();
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    float G = 0.f, U = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float s1 = bf2f(w.sg[ii][j]), b1 = bf2f(w.bg[ii][j]);
      const float s2 = bf2f(w.su[ii][j]), b2 = bf2f(w.bu[ii][j]);
      G += s1 * chunk_dot128(w.qg[ii][j], xp[j], kq) + (b1 - 128.f * s1) * X[j];
      U += s2 * chunk_dot128(w.qu[ii][j], xp[j], kq) + (b2 - 128.f * s2) * X[j];
    }
    v[ii] = G;
    v[R + ii] = U;
  }
}

// The LoRA term (lane rr < r adds scale * B[row][rr] * t[rr]), the sums over
// the wave and the SwiGLU of the R rows.  STORE: rows of h go to the
// workspace (store_h); otherwise only h_s and hrep_s (hi + lo, the value the
// down GEMV sees) are written and the caller publishes them.
template <int NJ, int RR, bool STORE>
__device__ __forceinline__ void gu_epilogue(const MoeArgs& a, const GuW<NJ, RR>& w, int k,
                                            int i0, float (&v)[2 * RR], float tg, float tu,
                                            float* h_s, float* hrep_s) {
  constexpr int R = RR;
  const int lane = tid_here() & 63, wave = tid_here() >> 6;
  const int row0 = i0 + R * wave;
  if (a.r > 0 && lane < a.r) {
#pragma unroll
    for (int ii = 0; ii < R; ++ii) {
      v[ii] += a.scale * (bf2f(w.Bg[ii]) * tg);
      v[R + ii] += a.scale * (bf2f(w.Bu[ii]) * tu);
    }
  }
  // lane (64/2R) * ii holds G of row ii, lane 32 + (64/2R) * ii its U
  const float w1 = wave_sums_2r<R>(v);
  const float Uo = __shfl_xor(w1, 32, kWave);
  constexpr int kSpan = 64 / (2 * R);
  if (lane < 32 && (lane % kSpan) == 0) {
    const int ii = lane / kSpan;
    const float h = silu_f(w1) * Uo;
    h_s[R * wave + ii] = h;
    if constexpr (STORE) {
      hrep_s[R * wave + ii] = store_h(a, k, row0 + ii, h);
    } else {
      const uint32_t hi = f2bf(h);
      hrep_s[R * wave + ii] = bf2f(hi) + bf2f(f2bf(h - bf2f(hi)));
    }
  }
}

// gate/up of the wave's R row pairs: gu_base then gu_epilogue
template <int NJ, int RR = kWideRowsPerWave, bool STORE = true>
__device__ __forceinline__ void gu_finish(const MoeArgs& a, const GuW<NJ, RR>& w, int k, int i0,
                                          const uint16_t* xsrc, float tg, float tu, float* h_s,
                                          float* hrep_s) {
  float v[2 * RR];
  gu_base<NJ, RR>(w, xsrc, v);
  gu_epilogue<NJ, RR, STORE>(a, w, k, i0, v, tg, tu, h_s, hrep_s);
}


}  // namespace e0
