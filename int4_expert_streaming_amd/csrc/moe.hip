// The int4 gather kernels of one MoE layer: fused dequant-GEMV of the
// committed experts' gate/up/down projections, SwiGLU, the unmerged LoRA
// deltas and the weighted combine.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction": §3.1 "Math contract" (down(silu(gate(x))
// * up(x)) over the routed experts), §2 "Quantization" (int4 affine, group
// 64), §3.1 "Executor paths" (nine arrays per expert, slot table), §3.3
// (LoRA served unmerged as a parallel delta).
//
// Three launches per layer, all HBM-bound at batch 1:
//   k_lora_in : t = A x for the gate and up adapters of the K experts
//               (K*2*r bf16 rows of length d), one wave per row.
//   k_gate_up : gate and up rows of the K experts, one wave per row pair
//               (row-major weights; each lane owns 32-input chunks and keeps
//               its activation chunk in registers), LoRA B t, SwiGLU.  Writes
//               h as bf16 hi/lo pairs for the down GEMV, per-16-row sums of
//               h, and per-16-row partials of A_down h.
//   k_down    : tiled down weights (1 KiB tile = 64 rows x 32 inputs; lane =
//               output row, the tile's activation chunk is wave-uniform);
//               units split the K*I reduction into slices; the last unit of
//               a 64-row block sums the slices in a fixed order, adds the
//               LoRA-down term and the routing weights, and rounds to bf16.
//
// Int4 arithmetic: each 32-input chunk accumulates sum (128 + q) x with
// v_dot2_f32_bf16 on exact bf16 "128 + q" nibble pairs, and the group affine
// is applied per chunk as s * acc + (b - 128 s) * sum(x), which equals
// sum (s q + b) x.  Everything after the loads is fp32.
#include "moe_internal.h"

namespace e0 {

__device__ __forceinline__ const uint8_t* slot_of(const MoeArgs& a, int k) {
  const int e = a.ids[k];
  if (e < 0 || e >= a.E) return nullptr;
  const int s = a.table[e];
  if (s < 0 || s >= a.n_slots) return nullptr;
  return a.pool + (size_t)s * (size_t)a.slot_bytes;
}

// -------------------------------------------------------------- k_lora_in
// t[k][p][rr] = A_p(e_k)[rr] . x.  With h_norm set, every workgroup first
// computes x = bf16(RMSNorm(h_norm)) into LDS and workgroup 0 stores it.
__global__ __launch_bounds__(256) void k_lora_in(MoeArgs a) {
  __shared__ uint16_t xs[kMaxD];
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  const int nrows = a.K * 2 * a.r;
  const bool active = row < nrows;
  const int k = active ? row / (2 * a.r) : 0;
  const int p = active ? (row / a.r) & 1 : 0;
  const int rr = active ? row % a.r : 0;
  const uint8_t* b = active ? slot_of(a, k) : nullptr;
  const uint16_t* A = nullptr;
  if (b != nullptr)
    A = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.a_up : a.lay.a_gate)) + (size_t)rr * a.d;
  RowPref pf;
  const bool pref = A != nullptr && a.d <= 64 * kPrefChunks * 8;
  if (pref) row_prefetch(A, a.d, pf);          // in flight during the norm
  const uint16_t* x = a.x;
  if (a.h_norm != nullptr) {
    rmsnorm_to_lds(a.h_norm, xs, a.d, a.eps);
    if (blockIdx.x == 0)
      for (int j = threadIdx.x; j < a.d; j += blockDim.x) a.x_out[j] = xs[j];
    x = xs;
  }
  if (!active) return;
  float t = 0.f;
  if (A != nullptr) {
    t = pref ? row_dot_pref(pf, x, a.d) : row_dot<false, false>(A, x, a.d);
  } else if ((threadIdx.x & 63) == 0) {
    set_error(a.err, EDGE0_ERANGE);
  }
  if ((threadIdx.x & 63) == 0) a.t_in[row] = t;
}

// -------------------------------------------------------------- k_gate_up
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

// position of element i of h in the pair-permuted order of its 8-group
__device__ __forceinline__ int pair_pos(int i) {
  const int s = i & 7;
  return (i & ~7) + (s < 4 ? 2 * s : 2 * (s - 4) + 1);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

// store one row of h: fp32, the bf16 hi/lo split (hi = bf16(h), lo = bf16(h - hi));
// returns hi + lo, the value the down GEMV sees
__device__ __forceinline__ float store_h(const MoeArgs& a, int k, int i, float h) {
  const uint32_t hi = f2bf(h);
  const uint32_t lo = f2bf(h - bf2f(hi));
  const size_t base = (size_t)k * a.I;
  a.hf[base + i] = h;
  a.hp_hi[base + pair_pos(i)] = (uint16_t)hi;
  a.hp_lo[base + pair_pos(i)] = (uint16_t)lo;
  return bf2f(hi) + bf2f(lo);
}

// Wide rows: d/32 = 64*NJ chunks per row; lane l owns chunks l + 64 j of both
// the gate and the up row; 4 row pairs per wave.  Every global load of the
// wave (weights, scales, biases, LoRA B rows and t) is issued before any math.
template <int NJ>
__device__ __forceinline__ void gate_up_wide(const MoeArgs& a, const uint8_t* b, int k, int i0,
                                             float* h_s, float* hrep_s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, g = a.g, ng = d / g, r = a.r;
  constexpr int R = 4;
  const int row0 = i0 + 4 * wave;
  XRaw xr[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) load_x_raw(a.x, lane + 64 * j, xr[j]);
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s);
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(b + a.lay.up_s);
  const uint16_t* ub = reinterpret_cast<const uint16_t*>(b + a.lay.up_b);
  uint4 qg[R][NJ], qu[R][NJ];
  uint32_t sg[R][NJ], bg[R][NJ], su[R][NJ], bu[R][NJ];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    const int row = row0 + ii;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = lane + 64 * j;
      qg[ii][j] = reinterpret_cast<const uint4*>(gq + (size_t)row * (d / 8))[col];
      qu[ii][j] = reinterpret_cast<const uint4*>(uq + (size_t)row * (d / 8))[col];
      const int grp = (32 * col) / g;
      sg[ii][j] = gs[row * ng + grp];
      bg[ii][j] = gb[row * ng + grp];
      su[ii][j] = us[row * ng + grp];
      bu[ii][j] = ub[row * ng + grp];
    }
  }
  // LoRA: lane rr < r holds B[row][rr] for the 4 rows and t[rr] (r <= 64)
  uint32_t Bg[R], Bu[R];
  float tg = 0.f, tu = 0.f;
  const bool has_l = r > 0 && lane < r;
  if (has_l) {
    const uint16_t* Bgp = reinterpret_cast<const uint16_t*>(b + a.lay.b_gate);
    const uint16_t* Bup = reinterpret_cast<const uint16_t*>(b + a.lay.b_up);
#pragma unroll
    for (int ii = 0; ii < R; ++ii) {
      Bg[ii] = Bgp[(size_t)(row0 + ii) * r + lane];
      Bu[ii] = Bup[(size_t)(row0 + ii) * r + lane];
    }
    tg = a.t_in[(size_t)(k * 2 + 0) * r + lane];
    tu = a.t_in[(size_t)(k * 2 + 1) * r + lane];
  }
  uint32_t xp[NJ][16];
  float X[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) X[j] = x_pairs(xr[j], xp[j]);
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    float G = 0.f, U = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float s1 = bf2f(sg[ii][j]), b1 = bf2f(bg[ii][j]);
      const float s2 = bf2f(su[ii][j]), b2 = bf2f(bu[ii][j]);
      G += s1 * chunk_dot128(qg[ii][j], xp[j]) + (b1 - 128.f * s1) * X[j];
      U += s2 * chunk_dot128(qu[ii][j], xp[j]) + (b2 - 128.f * s2) * X[j];
    }
    if (has_l) {
      G += a.scale * (bf2f(Bg[ii]) * tg);
      U += a.scale * (bf2f(Bu[ii]) * tu);
    }
    G = wave_sum(G);
    U = wave_sum(U);
    const float h = silu_f(G) * U;
    if (lane == 0) {
      h_s[4 * wave + ii] = h;
      hrep_s[4 * wave + ii] = store_h(a, k, row0 + ii, h);
    }
  }
}

// Narrow rows: d/32 = CPR in {8, 16, 32} chunks per row; a step covers
// R = 32/CPR row pairs; lane -> (row of the step, gate/up, chunk).
template <int CPR>
__device__ __forceinline__ void gate_up_narrow(const MoeArgs& a, const uint8_t* b, int k, int i0,
                                               float* h_s, float* hrep_s) {
  constexpr int R = 32 / CPR;
  constexpr int STEPS = 4 / R;
  constexpr int LPR = (64 + CPR - 1) / CPR;  // LoRA terms per lane, r <= 64
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rloc = lane / (2 * CPR);
  const int p = (lane / CPR) & 1;
  const int col = lane % CPR;
  const int d = a.d, g = a.g, ng = d / g, r = a.r;
  XRaw xr;
  load_x_raw(a.x, col, xr);
  const uint32_t* q = reinterpret_cast<const uint32_t*>(b + (p ? a.lay.up_q : a.lay.gate_q));
  const uint16_t* sp = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.up_s : a.lay.gate_s));
  const uint16_t* bp = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.up_b : a.lay.gate_b));
  uint4 qq[STEPS];
  uint32_t ss[STEPS], bb[STEPS];
  uint32_t Bl[STEPS][LPR];
  float tl[LPR];
  const int grp = (32 * col) / g;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int row = i0 + 4 * wave + st * R + rloc;
    qq[st] = reinterpret_cast<const uint4*>(q + (size_t)row * (d / 8))[col];
    ss[st] = sp[row * ng + grp];
    bb[st] = bp[row * ng + grp];
  }
  if (r > 0) {
    const uint16_t* B = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.b_up : a.lay.b_gate));
    const float* t = a.t_in + (size_t)(k * 2 + p) * r;
#pragma unroll
    for (int m = 0; m < LPR; ++m) {
      const int rr = col + m * CPR;
      tl[m] = rr < r ? t[rr] : 0.f;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const int row = i0 + 4 * wave + st * R + rloc;
        Bl[st][m] = rr < r ? B[(size_t)row * r + rr] : 0u;
      }
    }
  }
  uint32_t xp[16];
  const float X = x_pairs(xr, xp);
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int row = i0 + 4 * wave + st * R + rloc;
    const float s = bf2f(ss[st]), bv = bf2f(bb[st]);
    float v = s * chunk_dot128(qq[st], xp) + (bv - 128.f * s) * X;
    if (r > 0) {
      float dl = 0.f;
#pragma unroll
      for (int m = 0; m < LPR; ++m) dl += bf2f(Bl[st][m]) * tl[m];
      v += a.scale * dl;
    }
    v = seg_sum<CPR>(v);                       // G (p = 0) or U (p = 1) of this row
    const float U = __shfl(v, (lane + CPR) & 63, kWave);
    if (p == 0 && col == 0) {
      const float h = silu_f(v) * U;
      const int loc = 4 * wave + st * R + rloc;
      h_s[loc] = h;
      hrep_s[loc] = store_h(a, k, row, h);
    }
  }
}

// One workgroup = 16 consecutive rows of one expert's gate and up.  Also
// writes the 16-row sum of h and the 16-row partial of A_down h.
template <int CPR>
__global__ __launch_bounds__(256) void k_gate_up(MoeArgs a) {
  __shared__ float h_s[16];
  __shared__ float hrep_s[16];
  const int nblk = a.I / 16;
  const int k = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int i0 = blk * 16;
  const int r = a.r;
  const uint8_t* b = slot_of(a, k);
  if (b == nullptr) {
    // unresolvable expert: zero activations, flag the error
    for (int t = threadIdx.x; t < 16; t += blockDim.x) store_h(a, k, i0 + t, 0.f);
    if ((int)threadIdx.x < r) a.tdpart[((size_t)k * nblk + blk) * r + threadIdx.x] = 0.f;
    if (threadIdx.x == 0) {
      a.hs[(size_t)k * nblk + blk] = 0.f;
      set_error(a.err, EDGE0_ERANGE);
    }
    return;
  }
  // A_down columns of these rows, loaded early (threads rr < r), used raw later
  uint4 ad0 = make_uint4(0, 0, 0, 0), ad1 = ad0;
  if ((int)threadIdx.x < r) {
    const uint4* src = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(b + a.lay.a_down) + (size_t)threadIdx.x * a.I + i0);
    ad0 = src[0];
    ad1 = src[1];
  }
  if constexpr (CPR >= 64) {
    gate_up_wide<CPR / 64>(a, b, k, i0, h_s, hrep_s);
  } else {
    gate_up_narrow<CPR>(a, b, k, i0, h_s, hrep_s);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int t = 0; t < 16; ++t) s += hrep_s[t];
    a.hs[(size_t)k * nblk + blk] = s;
  }
  if ((int)threadIdx.x < r) {
    const uint32_t w[8] = {ad0.x, ad0.y, ad0.z, ad0.w, ad1.x, ad1.y, ad1.z, ad1.w};
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) s += bf_lo(w[m]) * h_s[2 * m] + bf_hi(w[m]) * h_s[2 * m + 1];
    a.tdpart[((size_t)k * nblk + blk) * r + threadIdx.x] = s;
  }
}

// ------------------------------------------------------------------ k_down
// Unit (rb, k, sl): rows 64 rb .. 64 rb + 63 of expert k's down projection
// over input chunks of slice sl, times the routing weight w_k; the sl = 0
// unit adds the LoRA-down delta.  The last unit of a row block sums the
// K*S partials in a fixed order, rounds to bf16 and applies the residual.
constexpr int kDownTiles = 4;  // tiles per wave per batch of loads

constexpr int kMaxSliceChunks = 64;  // chunks per slice (cps) staged in LDS

__device__ __forceinline__ void down_tile_loads(const uint4* dq, const uint16_t* ds,
                                                const uint16_t* db, int rb, int NC, int d, int g,
                                                int o, int lane, int base, int c1, uint4* q,
                                                uint32_t* sv, uint32_t* bv) {
#pragma unroll
  for (int m = 0; m < kDownTiles; ++m) {
    const int c = base + 4 * m;
    if (c < c1) {
      q[m] = dq[((size_t)rb * NC + c) * 64 + lane];
      const int grp = (32 * c) / g;
      sv[m] = ds[(size_t)grp * d + o];
      bv[m] = db[(size_t)grp * d + o];
    }
  }
}

__global__ __launch_bounds__(256) void k_down(MoeArgs a) {
  __shared__ float red[4][64];
  __shared__ uint32_t hp_s[kMaxSliceChunks][32];  // hi pairs then lo pairs of each chunk
  __shared__ float hsum_s[kMaxSliceChunks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K, S = a.S, I = a.I, d = a.d, r = a.r;
  const int NC = I / 32;
  const int u = blockIdx.x;
  const int rb = u / (K * S);
  const int k = (u / S) % K;
  const int sl = u % S;
  const int cps = (NC + S - 1) / S;
  const int c0 = sl * cps;
  const int c1 = min(NC, c0 + cps);
  const int o = rb * 64 + lane;
  const uint8_t* b = slot_of(a, k);  // uniform over the workgroup
  const float wk = a.w[k];
  const uint4* dq = nullptr;
  const uint16_t *ds = nullptr, *db = nullptr;
  uint4 q[kDownTiles];
  uint32_t sv[kDownTiles], bv[kDownTiles];
  // LoRA-down delta for these rows (slice 0 only, wave 0): t_down = sum over
  // the 16-row partials of A_down h, where element t = blk*r + rr of the
  // partials goes to lane t % 64 (which always holds rr = lane % r, r
  // dividing 64), and B_down row o (r bf16).  Loaded before the tiles.
  const bool lora_here = b != nullptr && r > 0 && sl == 0 && wave == 0;
  const int ntd = (I / 16) * r;
  constexpr int kTd = 16;
  float tdr[kTd];
  uint4 bdr[8];
  if (b != nullptr) {
    dq = reinterpret_cast<const uint4*>(b + a.lay.down_q);
    ds = reinterpret_cast<const uint16_t*>(b + a.lay.down_s);
    db = reinterpret_cast<const uint16_t*>(b + a.lay.down_b);
    if (lora_here) {
      const float* tp = a.tdpart + (size_t)k * ntd;
#pragma unroll
      for (int m = 0; m < kTd; ++m) tdr[m] = (lane + 64 * m < ntd) ? tp[lane + 64 * m] : 0.f;
      const uint4* Bdp = reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint16_t*>(b + a.lay.b_down) + (size_t)o * r);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (8 * m < r) bdr[m] = Bdp[m];
    }
    // first batch of this wave's tiles: in flight while the slice's
    // activation pairs and chunk sums are staged in LDS
    down_tile_loads(dq, ds, db, rb, NC, d, a.g, o, lane, c0 + wave, c1, q, sv, bv);
    const uint32_t* hph = reinterpret_cast<const uint32_t*>(a.hp_hi + (size_t)k * I);
    const uint32_t* hpl = reinterpret_cast<const uint32_t*>(a.hp_lo + (size_t)k * I);
    const float* hs = a.hs + (size_t)k * (I / 16);
    const int ncs = c1 - c0;
    for (int t = threadIdx.x; t < ncs * 32; t += blockDim.x) {
      const int cc = t >> 5, j = t & 31;
      hp_s[cc][j] = j < 16 ? hph[16 * (c0 + cc) + j] : hpl[16 * (c0 + cc) + j - 16];
    }
    for (int t = threadIdx.x; t < ncs; t += blockDim.x)
      hsum_s[t] = hs[2 * (c0 + t)] + hs[2 * (c0 + t) + 1];
  } else if (threadIdx.x == 0) {
    set_error(a.err, EDGE0_ERANGE);
  }
  __syncthreads();  // every thread, unconditionally
  float part = 0.f;
  if (b != nullptr) {
    for (int base = c0 + wave; base < c1; base += 4 * kDownTiles) {
      if (base != c0 + wave)
        down_tile_loads(dq, ds, db, rb, NC, d, a.g, o, lane, base, c1, q, sv, bv);
#pragma unroll
      for (int m = 0; m < kDownTiles; ++m) {
        const int c = base + 4 * m;
        if (c < c1) {
          const float s = bf2f(sv[m]), bb = bf2f(bv[m]);
          const uint32_t* hp = hp_s[c - c0];
          const float acc = chunk_dot128(q[m], hp) + chunk_dot128(q[m], hp + 16);
          part += s * acc + (bb - 128.f * s) * hsum_s[c - c0];
        }
      }
    }
    if (lora_here) {
      float tdv = 0.f;
#pragma unroll
      for (int m = 0; m < kTd; ++m) tdv += tdr[m];
      for (int t = lane + 64 * kTd; t < ntd; t += 64) tdv += a.tdpart[(size_t)k * ntd + t];
      for (int off = r; off < 64; off <<= 1) tdv += __shfl_xor(tdv, off, kWave);
      float dl = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (8 * m < r) {
          const uint32_t bw[4] = {bdr[m].x, bdr[m].y, bdr[m].z, bdr[m].w};
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            dl += bf_lo(bw[q2]) * __shfl(tdv, 8 * m + 2 * q2, kWave);
            dl += bf_hi(bw[q2]) * __shfl(tdv, 8 * m + 2 * q2 + 1, kWave);
          }
        }
      }
      part += a.scale * dl;
    }
  }
  red[wave][lane] = part;
  __syncthreads();
  if (wave == 0) {
    const float t = (red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane]) * wk;
    a.dpart[(((size_t)rb * K + k) * S + sl) * 64 + lane] = t;
  }
}

// y[o] = bf16(sum over experts k and slices s of the down partials, in that
// fixed order); optional residual h_out = bf16(h_res + y)
__global__ __launch_bounds__(256) void k_combine(MoeArgs a) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= a.d) return;
  const int rb = o / 64, lane = o % 64;
  const float* p = a.dpart + (size_t)rb * a.K * a.S * 64 + lane;
  const int n = a.K * a.S;
  float yv = 0.f;
  for (int j0 = 0; j0 < n; j0 += 16) {
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = (j0 + m < n) ? p[(size_t)(j0 + m) * 64] : 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) yv += v[m];
  }
  const uint32_t yb = f2bf(yv);
  a.y[o] = (uint16_t)yb;
  if (a.h_out != nullptr) a.h_out[o] = (uint16_t)f2bf(bf2f(a.h_res[o]) + bf2f(yb));
}

// ------------------------------------------------------------ bundle pack
// down_q: logical u32 [d][I/8] -> tiled [d/64][I/32][64][4]
__global__ void k_tile_down(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int d,
                            int I) {
  const int NC = I / 32;
  const size_t n = (size_t)d * I / 8;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n;
       t += (size_t)gridDim.x * blockDim.x) {
    const size_t tile = t / 256;
    const int within = (int)(t % 256);
    const int rb = (int)(tile / NC), c = (int)(tile % NC);
    const int o = rb * 64 + within / 4, word = within % 4;
    dst[t] = src[(size_t)o * (I / 8) + 4 * c + word];
  }
}

// down scales/biases: logical bf16 [d][I/g] -> group-major [I/g][d]
__global__ void k_transpose_sb(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                               int d, int ng) {
  const size_t n = (size_t)d * ng;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n;
       t += (size_t)gridDim.x * blockDim.x) {
    const int grp = (int)(t / d), o = (int)(t % d);
    dst[t] = src[(size_t)o * ng + grp];
  }
}

// ------------------------------------------------------------ host side
int fill_moe_args(const edge0_moe_shape* sh, const edge0_slot_pool* pool, const int32_t* table,
                  const int32_t* ids, const float* w, const void* x, void* y, void* workspace,
                  MoeArgs* a) {
  edge0_bundle_layout lay;
  if (bundle_layout(sh, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  if (!pool || !pool->base || pool->n_slots <= 0 || pool->slot_bytes < lay.bytes ||
      pool->slot_bytes % 256 != 0 || !table || !ids || !w || !x || !y || !workspace || x == y)
    return EDGE0_EINVAL;
  const WsLayout L = ws_layout(sh);
  char* ws = static_cast<char*>(workspace);
  a->pool = static_cast<const uint8_t*>(pool->base);
  a->slot_bytes = pool->slot_bytes;
  a->n_slots = pool->n_slots;
  a->table = table;
  a->ids = ids;
  a->w = w;
  a->x = static_cast<const uint16_t*>(x);
  a->y = static_cast<uint16_t*>(y);
  a->h_res = nullptr;
  a->h_out = nullptr;
  a->h_norm = nullptr;
  a->x_out = nullptr;
  a->eps = 0.f;
  a->d = sh->d_model;
  a->E = sh->n_experts;
  a->I = sh->d_inter;
  a->K = sh->top_k;
  a->g = sh->group_size;
  a->r = sh->lora_rank;
  a->scale = sh->lora_rank > 0 ? sh->lora_alpha / (float)sh->lora_rank : 0.f;
  a->lay = lay;
  a->err = reinterpret_cast<uint32_t*>(ws + L.err);
  a->cnt_down = reinterpret_cast<uint32_t*>(ws + L.cnt_down);
  a->t_in = reinterpret_cast<float*>(ws + L.t_in);
  a->hf = reinterpret_cast<float*>(ws + L.hf);
  a->hp_hi = reinterpret_cast<uint16_t*>(ws + L.hp_hi);
  a->hp_lo = reinterpret_cast<uint16_t*>(ws + L.hp_lo);
  a->hs = reinterpret_cast<float*>(ws + L.hs);
  a->tdpart = reinterpret_cast<float*>(ws + L.tdpart);
  a->td = reinterpret_cast<float*>(ws + L.td);
  a->cnt_td = reinterpret_cast<uint32_t*>(ws + L.cnt_td);
  a->dpart = reinterpret_cast<float*>(ws + L.dpart);
  const int RB = a->d / 64, NC = a->I / 32;
  int S = (512 + RB * a->K - 1) / (RB * a->K);
  S = S < 1 ? 1 : (S > NC ? NC : S);
  const int min_s = (NC + kMaxSliceChunks - 1) / kMaxSliceChunks;  // slice fits the LDS stage
  a->S = S < min_s ? min_s : S;
  return EDGE0_OK;
}

int launch_moe(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing) {
  auto mark = [&](int which, bool start) {
    if (timing && timing->which == which)
      (void)hipEventRecord(start ? timing->start : timing->stop, stream);
  };
  if (a.r > 0 || a.h_norm != nullptr) {
    const int rows = a.K * 2 * a.r;
    mark(3, true);
    k_lora_in<<<rows > 0 ? (rows + 3) / 4 : 1, 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
    mark(3, false);
  }
  const int cpr = a.d / 32;
  const int grid2 = a.K * (a.I / 16);
  mark(1, true);
  switch (cpr) {
    case 8: k_gate_up<8><<<grid2, 256, 0, stream>>>(a); break;
    case 16: k_gate_up<16><<<grid2, 256, 0, stream>>>(a); break;
    case 32: k_gate_up<32><<<grid2, 256, 0, stream>>>(a); break;
    case 64: k_gate_up<64><<<grid2, 256, 0, stream>>>(a); break;
    case 128: k_gate_up<128><<<grid2, 256, 0, stream>>>(a); break;
    case 192: k_gate_up<192><<<grid2, 256, 0, stream>>>(a); break;
    case 256: k_gate_up<256><<<grid2, 256, 0, stream>>>(a); break;
    default: return EDGE0_EINVAL;
  }
  E0_CHECK_LAUNCH();
  mark(1, false);
  const int grid3 = (a.d / 64) * a.K * a.S;
  mark(2, true);
  k_down<<<grid3, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  mark(2, false);
  k_combine<<<(a.d + 255) / 256, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

}  // namespace e0

using namespace e0;

extern "C" int edge0_moe_layer(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                               const int32_t* slot_table, const int32_t* ids, const float* w,
                               const void* x, void* y, void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape)) return EDGE0_EINVAL;
  MoeArgs a;
  const int rc = fill_moe_args(shape, pool, slot_table, ids, w, x, y, workspace, &a);
  if (rc != EDGE0_OK) return rc;
  return launch_moe(a, stream);
}

extern "C" int edge0_pack_bundle(const edge0_moe_shape* shape, const edge0_expert_arrays* src,
                                 void* bundle_dst, hipStream_t stream) {
  edge0_bundle_layout lay;
  if (!shape || !src || !bundle_dst || bundle_layout(shape, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  if (reinterpret_cast<uintptr_t>(bundle_dst) % 256 != 0) return EDGE0_EINVAL;
  const int d = shape->d_model, I = shape->d_inter, g = shape->group_size, r = shape->lora_rank;
  const void* req[] = {src->gate_q, src->gate_s, src->gate_b, src->up_q, src->up_s,
                       src->up_b, src->down_q, src->down_s, src->down_b};
  for (const void* p : req)
    if (!p) return EDGE0_EINVAL;
  if (r > 0 && (!src->a_gate || !src->b_gate || !src->a_up || !src->b_up || !src->a_down ||
                !src->b_down))
    return EDGE0_EINVAL;
  char* dst = static_cast<char*>(bundle_dst);
  const size_t qb = (size_t)I * d / 2, sb = (size_t)I * (d / g) * 2, dsb = (size_t)d * (I / g) * 2;
  struct {
    int64_t off;
    const void* p;
    size_t n;
  } copies[] = {
      {lay.gate_q, src->gate_q, qb}, {lay.gate_s, src->gate_s, sb}, {lay.gate_b, src->gate_b, sb},
      {lay.up_q, src->up_q, qb},     {lay.up_s, src->up_s, sb},     {lay.up_b, src->up_b, sb},
  };
  for (auto& c : copies)
    if (hipMemcpyAsync(dst + c.off, c.p, c.n, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return EDGE0_EHIP;
  k_tile_down<<<256, 256, 0, stream>>>(static_cast<const uint32_t*>(src->down_q),
                                       reinterpret_cast<uint32_t*>(dst + lay.down_q), d, I);
  E0_CHECK_LAUNCH();
  k_transpose_sb<<<64, 256, 0, stream>>>(static_cast<const uint16_t*>(src->down_s),
                                         reinterpret_cast<uint16_t*>(dst + lay.down_s), d, I / g);
  E0_CHECK_LAUNCH();
  k_transpose_sb<<<64, 256, 0, stream>>>(static_cast<const uint16_t*>(src->down_b),
                                         reinterpret_cast<uint16_t*>(dst + lay.down_b), d, I / g);
  E0_CHECK_LAUNCH();
  (void)dsb;
  if (r > 0) {
    struct {
      int64_t off;
      const void* p;
      size_t n;
    } lc[] = {{lay.a_gate, src->a_gate, (size_t)r * d * 2}, {lay.b_gate, src->b_gate, (size_t)I * r * 2},
              {lay.a_up, src->a_up, (size_t)r * d * 2},     {lay.b_up, src->b_up, (size_t)I * r * 2},
              {lay.a_down, src->a_down, (size_t)r * I * 2}, {lay.b_down, src->b_down, (size_t)d * r * 2}};
    for (auto& c : lc)
      if (hipMemcpyAsync(dst + c.off, c.p, c.n, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return EDGE0_EHIP;
  }
  return EDGE0_OK;
}
