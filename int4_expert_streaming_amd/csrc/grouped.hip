// Several tokens through one MoE layer, grouped by expert: every routed
// expert's weights are read once per call however many tokens chose it.
//
// The result is defined token by token, exactly as the single-token layer
// ([Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction", §3.1 "Math contract", §3.3 unmerged
// LoRA, Figure 1 sum node); the grouping only reorders the work.
//
// Launches (all on the caller's stream):
//   k_grp_route_lora : workgroup 0 buckets the T*K (token, k) pairs by
//                   expert (counting sort, stable in pair order, so by
//                   token), lists the active experts with their first pair
//                   and count, and resolves each active expert's slot once;
//                   the other workgroups compute t = A x for every pair's
//                   gate and up adapters.
//   k_grp_gu_tile : one workgroup = 16 rows of one active expert's gate and
//                   up for a tile of up to 16 of its tokens, on MFMA
//                   (16x16x32 bf16 against the exact 128 + q nibble values);
//                   SwiGLU; h stored as bf16 hi/lo pairs, per-16-row sums,
//                   and A_down h accumulated in fixed point per pair.
//   k_grp_gate_up : the same as multi-token GEMVs (rows in registers, at most
//                   8 tokens per workgroup), for calls of few tokens.
//   k_grp_down_tile / k_grp_down : one workgroup = 128 output rows of one
//                   active expert for a tile of its tokens on MFMA, or 64
//                   rows for at most 8 tokens as GEMVs; the LoRA-down delta;
//                   each token's weighted row added to its fixed-point
//                   output.
//   k_grp_out     : y = bf16 of each token's accumulator; clears the
//                   accumulators for the next call.
// Int4 arithmetic is the single-token path's: exact bf16 "128 + q" nibble
// pairs against pair-permuted activations, the group affine folded per
// 32-input chunk (per group on MFMA), fp32 accumulation, one bf16 rounding
// of y.
#include <algorithm>

#include "moe_internal.h"

namespace e0 {

constexpr int kGrpMaxTokens = 64;

struct GrpArgs {
  const uint8_t* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  const int32_t* table;
  const int32_t* ids;  // [T][K]
  const float* w;      // [T][K]
  const uint16_t* x;   // [T][d]
  uint16_t* y;         // [T][d]
  int T, d, E, I, K, g, r;
  float scale;
  edge0_bundle_layout lay;
  int Amax;  // grid bound on the number of active experts: min(E, T*K)
  int P;     // T*K
  // workspace
  uint32_t* err;
  int32_t* info;      // [0] active experts, [1] valid pairs
  int32_t* act_e;     // [Amax]
  int32_t* act_off;   // [Amax] first sorted pair
  int32_t* act_cnt;   // [Amax]
  int32_t* act_slot;  // [Amax] slot, or -1
  int32_t* pair_tok;  // [P] token of each sorted pair
  int32_t* pair_src;  // [P] each sorted pair's unsorted index (token * K + k)
  float* pair_w;      // [P] routing weight of each sorted pair
  float* t_in;        // [P][2][r] by unsorted pair
  uint16_t* hp_hi;    // [P][I] pair-permuted
  uint16_t* hp_lo;
  float* hs;                   // [P][I/16]
  unsigned long long* tdown;   // [P][r] A_down h, fixed point
  unsigned long long* acc;     // [T][d] y, fixed point
  // prefill: the list of (active expert, 64-pair tile),
  // info[3] entries; each token's activation sum per input group [T][d/g];
  // each pair's weighted output row, by unsorted pair [P][d] (fp32); the
  // kept expert of each unsorted pair, or -1 (dropped repeat, invalid id)
  const int2* tiles64;
  const float* xsum;
  float* ypair;
  const int32_t* keep;
  // adapters given apart from the bundles (the _lora calls): factor i
  // (a_gate, b_gate, a_up, b_up, a_down, b_down) of expert e at lo_base[i] +
  // e * lo_stride bytes; when lora_sep is false each expert's factors are in
  // its bundle at the layout's offsets
  bool lora_sep;
  const uint8_t* lo_base[6];
  int64_t lo_stride;
};

// LoRA factor i of expert e (its bundle b, offset off in the bundle)
__device__ __forceinline__ const uint8_t* grp_lora(const GrpArgs& a, const uint8_t* b, int e, int i,
                                                   int64_t off) {
  return a.lora_sep ? a.lo_base[i] + (size_t)max(0, min(e, a.E - 1)) * a.lo_stride : b + off;
}

// ------------------------------------------------------------- bucketing
// inclusive prefix sum over a wave
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// One workgroup of 1024 threads, one expert per thread (E <= 1024): counts
// by LDS atomics, exclusive scans of the counts and of the "active" flags,
// then each pair's destination = its expert's first sorted position + the
// number of earlier pairs of the same expert (stable).  An id repeated
// within one token's routing is kept once, at its first k, with the
// repeats' weights added to it in k order (w1 D(x) + w2 D(x) = (w1 + w2)
// D(x)), so an expert holds at most one pair per token.
__device__ __forceinline__ void grp_route(const GrpArgs& a) {
  __shared__ unsigned long long tok_mask[1024];  // per expert: the tokens that chose it
  __shared__ int first[1024];
  __shared__ int ids_s[kGrpMaxTokens * 16];
  __shared__ float w_s[kGrpMaxTokens * 16];
  __shared__ int wtot[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.P, K = a.K;
  // every global read up front: pair tid's id and weight (P <= 1024), expert
  // tid's slot (E <= 1024)
  int e = -1;
  float w = 0.f;
  if (tid < P) {
    e = a.ids[tid];
    w = a.w[tid];
    if (e < 0 || e >= E) {
      set_error(a.err, EDGE0_ERANGE);
      e = -1;
    }
    ids_s[tid] = e;
    w_s[tid] = w;
  }
  const int slot = tid < E ? a.table[tid] : -1;
  tok_mask[tid] = 0ull;
  __syncthreads();
  // repeats within a token: the first k keeps the summed weight; each kept
  // pair marks its token in its expert's mask (at most one pair per token)
  const int t = tid / K;
  if (e >= 0) {
    const int k0 = tid - tid % K;
    bool dup = false;
    for (int q = k0; q < tid; ++q) dup |= ids_s[q] == e;
    for (int q = tid + 1; q < k0 + K; ++q)
      if (ids_s[q] == e) w += w_s[q];
    if (dup) e = -1;
    else atomicOr(&tok_mask[e], 1ull << t);
  }
  __syncthreads();
  const int c = tid < E ? __popcll(tok_mask[tid]) : 0;
  const int f = c > 0 ? 1 : 0;
  const int ic = wave_incl_scan(c), iff = wave_incl_scan(f);
  if (lane == 63) {
    wtot[0][wave] = ic;
    wtot[1][wave] = iff;
  }
  __syncthreads();
  int bc = 0, bf = 0, tc = 0, tf = 0;
  for (int v = 0; v < 16; ++v) {
    if (v < wave) {
      bc += wtot[0][v];
      bf += wtot[1][v];
    }
    tc += wtot[0][v];
    tf += wtot[1][v];
  }
  const int xc = bc + ic - c, xf = bf + iff - f;  // exclusive prefixes
  if (tid < E) {
    first[tid] = xc;
    if (f) {
      a.act_e[xf] = tid;
      a.act_off[xf] = xc;
      a.act_cnt[xf] = c;
      const bool ok = slot >= 0 && slot < a.n_slots;
      a.act_slot[xf] = ok ? slot : -1;
      if (!ok) set_error(a.err, EDGE0_ERANGE);
    }
  }
  if (tid == 0) {
    a.info[0] = tf;
    a.info[1] = tc;
  }
  __syncthreads();
  if (e >= 0) {
    // rank among the expert's pairs = its earlier tokens (pairs are in token order)
    const int dst = first[e] + __popcll(tok_mask[e] & ((1ull << t) - 1ull));
    a.pair_tok[dst] = t;
    a.pair_src[dst] = tid;
    a.pair_w[dst] = w;
  }
}

// ------------------------------------------------------------ LoRA A x
// t = A x for every (token, k) pair in the callers' order, which needs only
// the ids and the slot table: these workgroups run beside the bucketing in
// the same launch.  One wave per row (pair p, projection j, rank row rr).
__device__ __forceinline__ void grp_lora_in(const GrpArgs& a, int wg) {
  const int r = a.r;
  const int row = wg * 16 + (threadIdx.x >> 6);
  const int p = row / (2 * r), j = (row / r) & 1, rr = row % r;
  if (p >= a.P) return;
  const int e = a.ids[p];
  const int s = (e >= 0 && e < a.E) ? a.table[e] : -1;
  float t = 0.f;
  if (s >= 0 && s < a.n_slots) {  // otherwise the bucketing reports the pair
    const uint8_t* b = a.pool + (size_t)s * (size_t)a.slot_bytes;
    const uint16_t* wrow =
        reinterpret_cast<const uint16_t*>(grp_lora(a, b, e, j ? 2 : 0, j ? a.lay.a_up : a.lay.a_gate)) +
        (size_t)rr * a.d;
    t = row_dot<false, false>(wrow, a.x + (size_t)(p / a.K) * a.d, a.d);
  }
  if ((threadIdx.x & 63) == 0) a.t_in[row] = t;
}

// workgroup 0: the bucketing; workgroups 1.. (16 waves each): LoRA A x
__global__ __launch_bounds__(1024) void k_grp_route_lora(GrpArgs a) {
  if (blockIdx.x == 0) grp_route(a);
  else if (a.r > 0) grp_lora_in(a, blockIdx.x - 1);
}

// position of element i of h in the pair-permuted order of its 8-group
__device__ __forceinline__ int grp_pair_pos(int i) {
  const int s = i & 7;
  return (i & ~7) + (s < 4 ? 2 * s : 2 * (s - 4) + 1);
}
__device__ __forceinline__ float grp_silu(float z) { return z / (1.f + expf(-z)); }

// One token's h for one row: stored as hi/lo bf16 pairs; returns hi + lo.
__device__ __forceinline__ float grp_store_h(const GrpArgs& a, int q, int i, float h) {
  const uint32_t hi = f2bf(h);
  const uint32_t lo = f2bf(h - bf2f(hi));
  const size_t base = (size_t)q * a.I + grp_pair_pos(i);
  a.hp_hi[base] = (uint16_t)hi;
  a.hp_lo[base] = (uint16_t)lo;
  return bf2f(hi) + bf2f(lo);
}

// Per-16-row epilogue of one token: the sum of h over the rows and the
// partial A_down h (threads rr < r), added in fixed point.
__device__ __forceinline__ void grp_rows_epilogue(const GrpArgs& a, int q, int blk, int i0,
                                                  const float* h_s, const float* hrep_s,
                                                  const uint4& ad0, const uint4& ad1) {
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int t = 0; t < 16; ++t) s += hrep_s[t];
    a.hs[(size_t)q * (a.I / 16) + blk] = s;
  }
  if ((int)threadIdx.x < a.r) {
    const uint32_t w[8] = {ad0.x, ad0.y, ad0.z, ad0.w, ad1.x, ad1.y, ad1.z, ad1.w};
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) s += bf_lo(w[m]) * h_s[2 * m] + bf_hi(w[m]) * h_s[2 * m + 1];
    atomicAdd(a.tdown + (size_t)q * a.r + threadIdx.x, to_fix(s));
  }
  (void)i0;
}

// ------------------------------------------------------- gate/up (GEMV)
// Token batches staged in LDS: kGrpXBytes of activations per batch.
constexpr int kGrpXBytes = 32768;

// NJ = ceil(d/32 / 64) chunks per lane; lane l owns chunks l + 64 j (< d/32)
// of 4 row pairs of its wave.  Workgroup (slice, expert, 16-row block) takes
// the expert's tokens [ts * slice, ts * slice + ts): an expert chosen by many
// tokens is spread over several workgroups (each reads its rows again) and
// no longer sets the time alone.
// FULL: d = 2048 NJ, every lane's chunks exist (no per-lane guard on the
// loads, which the compiler would turn into branches that wait for them).
template <int NJ, bool FULL>
__global__ __launch_bounds__(256) void k_grp_gate_up(GrpArgs a, int min_cnt, int max_cnt,
                                                     int ts) {
  __shared__ uint16_t xs[kGrpXBytes / 2];
  __shared__ float h_s[16];
  __shared__ float hrep_s[16];
  const int nblk = a.I / 16;
  const int sl = blockIdx.x / (a.Amax * nblk);
  const int act = (blockIdx.x / nblk) % a.Amax;
  const int blk = blockIdx.x % nblk;
  // everything the start depends on, in one round trip
  const int n_act = a.info[0], n = a.act_cnt[act], slot = a.act_slot[act], q0 = a.act_off[act];
  asm volatile("" ::"s"(n_act), "s"(n), "s"(slot), "s"(q0));
  const int t_lo = sl * ts, t_hi = min(n, t_lo + ts);  // n <= T: the slices cover it
  if (act >= n_act || n < min_cnt || n > max_cnt || t_lo >= n || slot < 0) return;
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, g = a.g, ng = d / g, r = a.r, cpr = d / 32;
  const int i0 = blk * 16, row0 = i0 + 4 * wave;
  // the wave's 4 gate and 4 up rows, with their scales and biases
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q);
  const uint16_t* gsp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s);
  const uint16_t* gbp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b);
  const uint16_t* usp = reinterpret_cast<const uint16_t*>(b + a.lay.up_s);
  const uint16_t* ubp = reinterpret_cast<const uint16_t*>(b + a.lay.up_b);
  uint4 qg[4][NJ], qu[4][NJ];
  float sg[4][NJ], cg[4][NJ], su[4][NJ], cu[4][NJ];  // s and (b - 128 s)
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int row = row0 + ii;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = lane + 64 * j;
      const bool on = FULL || col < cpr;
      const int cc = on ? col : 0;
      qg[ii][j] = on ? reinterpret_cast<const uint4*>(gq + (size_t)row * (d / 8))[cc]
                     : make_uint4(0, 0, 0, 0);
      qu[ii][j] = on ? reinterpret_cast<const uint4*>(uq + (size_t)row * (d / 8))[cc]
                     : make_uint4(0, 0, 0, 0);
      const int grp = (32 * cc) / g;
      const float s1 = bf2f(gsp[row * ng + grp]), b1 = bf2f(gbp[row * ng + grp]);
      const float s2 = bf2f(usp[row * ng + grp]), b2 = bf2f(ubp[row * ng + grp]);
      sg[ii][j] = on ? s1 : 0.f;
      cg[ii][j] = on ? b1 - 128.f * s1 : 0.f;
      su[ii][j] = on ? s2 : 0.f;
      cu[ii][j] = on ? b2 - 128.f * s2 : 0.f;
    }
  }
  const bool has_l = r > 0 && lane < r;
  const int e = a.lora_sep ? a.act_e[act] : 0;  // the expert, for adapters given apart
  float Bg[4] = {0.f, 0.f, 0.f, 0.f}, Bu[4] = {0.f, 0.f, 0.f, 0.f};
  if (has_l) {
    const uint16_t* Bgp = reinterpret_cast<const uint16_t*>(grp_lora(a, b, e, 1, a.lay.b_gate));
    const uint16_t* Bup = reinterpret_cast<const uint16_t*>(grp_lora(a, b, e, 3, a.lay.b_up));
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      Bg[ii] = bf2f(Bgp[(size_t)(row0 + ii) * r + lane]);
      Bu[ii] = bf2f(Bup[(size_t)(row0 + ii) * r + lane]);
    }
  }
  uint4 ad0 = make_uint4(0, 0, 0, 0), ad1 = ad0;
  if ((int)threadIdx.x < r) {
    const uint4* src = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(grp_lora(a, b, e, 4, a.lay.a_down)) +
        (size_t)threadIdx.x * a.I + i0);
    ad0 = src[0];
    ad1 = src[1];
  }
  const int bt = kGrpXBytes / (2 * d) < 1 ? 1 : kGrpXBytes / (2 * d);  // tokens per batch
  for (int j0 = t_lo; j0 < t_hi; j0 += bt) {
    const int nb = t_hi - j0 < bt ? t_hi - j0 : bt;
    __syncthreads();  // previous batch fully consumed
    // stage the batch's activations: 16 bytes per thread per step
    const int n16 = nb * d / 8;
    for (int t = threadIdx.x; t < n16; t += 256) {
      const int jj = t / (d / 8), c8 = t % (d / 8);
      const int tok = a.pair_tok[q0 + j0 + jj];
      reinterpret_cast<uint4*>(xs)[t] =
          reinterpret_cast<const uint4*>(a.x + (size_t)tok * d)[c8];
    }
    __syncthreads();
    for (int jj = 0; jj < nb; ++jj) {
      const int q = q0 + j0 + jj;
      uint32_t xp[NJ][16];
      float X[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = lane + 64 * j;
        XRaw xr;
        if (FULL || col < cpr) {
          const uint4* src = reinterpret_cast<const uint4*>(xs + (size_t)jj * d + 32 * col);
#pragma unroll
          for (int m = 0; m < 4; ++m) xr.v[m] = src[m];
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) xr.v[m] = make_uint4(0, 0, 0, 0);
        }
        X[j] = x_pairs(xr, xp[j]);
      }
      float tg = 0.f, tu = 0.f;
      if (has_l) {
        const int src = a.pair_src[q];
        tg = a.t_in[((size_t)src * 2 + 0) * r + lane];
        tu = a.t_in[((size_t)src * 2 + 1) * r + lane];
      }
      const Q4Consts kq = q4_consts();
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float G = 0.f, U = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          G += sg[ii][j] * chunk_dot128(qg[ii][j], xp[j], kq) + cg[ii][j] * X[j];
          U += su[ii][j] * chunk_dot128(qu[ii][j], xp[j], kq) + cu[ii][j] * X[j];
        }
        if (has_l) {
          G += a.scale * (Bg[ii] * tg);
          U += a.scale * (Bu[ii] * tu);
        }
        G = wave_sum(G);
        U = wave_sum(U);
        if (lane == 0) {
          const float h = grp_silu(G) * U;
          h_s[4 * wave + ii] = h;
          hrep_s[4 * wave + ii] = grp_store_h(a, q, row0 + ii, h);
        }
      }
      __syncthreads();
      grp_rows_epilogue(a, q, blk, i0, h_s, hrep_s, ad0, ad1);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------- down (GEMV)
// CPW = 32-input chunks per wave: wave w owns chunks w, w + 4, ... of the
// tiled down weights of 64 output rows (lane = row).  Tokens in batches of
// kGrpBT; wave 0 adds the LoRA-down delta and scatters the weighted rows.
// Workgroup (slice, expert, row block) takes the expert's tokens
// [ts * slice, ts * slice + ts), as in k_grp_gate_up.
constexpr int kGrpBT = 8;
constexpr int kGrpMaxNC = 32;  // d_inter <= 1024

template <int CPW>
__global__ __launch_bounds__(256) void k_grp_down(GrpArgs a, int min_cnt, int max_cnt, int ts) {
  __shared__ uint32_t hp_s[kGrpBT][kGrpMaxNC][32];  // hi pairs then lo pairs of each chunk
  __shared__ float hsum_s[kGrpBT][kGrpMaxNC];
  __shared__ float red[4][kGrpBT][64];
  __shared__ float td_s[kGrpBT][64];
  const int nrb = a.d / 64;
  const int sl = blockIdx.x / (a.Amax * nrb);
  const int act = (blockIdx.x / nrb) % a.Amax;
  const int rb = blockIdx.x % nrb;
  // everything the start depends on, in one round trip
  const int n_act = a.info[0], n = a.act_cnt[act], slot = a.act_slot[act], q0 = a.act_off[act];
  asm volatile("" ::"s"(n_act), "s"(n), "s"(slot), "s"(q0));
  const int t_lo = sl * ts, t_hi = min(n, t_lo + ts);
  if (act >= n_act || n < min_cnt || n > max_cnt || t_lo >= n || slot < 0) return;
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, I = a.I, r = a.r, NC = I / 32;
  const int o = rb * 64 + lane;
  uint4 qv[CPW];
  float sv[CPW], cv[CPW];
#pragma unroll
  for (int m = 0; m < CPW; ++m) {
    const int c = wave + 4 * m;
    const bool on = c < NC;
    const int cc = on ? c : 0;
    qv[m] = reinterpret_cast<const uint4*>(b + a.lay.down_q)[((size_t)rb * NC + cc) * 64 + lane];
    const int grp = (32 * cc) / a.g;
    const float s = bf2f(reinterpret_cast<const uint16_t*>(b + a.lay.down_s)[(size_t)grp * d + o]);
    const float bb = bf2f(reinterpret_cast<const uint16_t*>(b + a.lay.down_b)[(size_t)grp * d + o]);
    sv[m] = on ? s : 0.f;
    cv[m] = on ? bb - 128.f * s : 0.f;
  }
  // LoRA-down row o (wave 0): r <= 64 bf16 as packed pairs
  uint32_t bd[32];
  if (wave == 0) {
    const int e = a.lora_sep ? a.act_e[act] : 0;  // the expert, for adapters given apart
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(grp_lora(a, b, e, 5, a.lay.b_down)) + (size_t)o * (r / 2);
#pragma unroll
    for (int m = 0; m < 32; ++m) bd[m] = 2 * m < r ? src[m] : 0u;
  }
  for (int j0 = t_lo; j0 < t_hi; j0 += kGrpBT) {
    const int nb = t_hi - j0 < kGrpBT ? t_hi - j0 : kGrpBT;
    __syncthreads();  // previous batch consumed
    {
      // the batch's h pairs, 16 bytes per thread and step: every load (at a
      // clamped, in-range index) before any store
      constexpr int kPer = kGrpBT * kGrpMaxNC * 32 / 4 / 256;
      const int n4 = nb * NC * 8;  // 16-byte pieces
      uint4 hv[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int t = min((int)threadIdx.x + 256 * u, n4 - 1);
        const int jj = t / (NC * 8), rem = t % (NC * 8);
        const int c = rem >> 3, w4 = rem & 7;  // pieces 0-3 hi pairs, 4-7 lo pairs
        const uint4* src = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint32_t*>(w4 < 4 ? a.hp_hi : a.hp_lo) +
            (size_t)(q0 + j0 + jj) * (I / 2) + 16 * c);
        hv[u] = src[w4 & 3];
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int t = threadIdx.x + 256 * u;
        if (t < n4) {
          const int jj = t / (NC * 8), rem = t % (NC * 8);
          reinterpret_cast<uint4*>(hp_s[jj][rem >> 3])[rem & 7] = hv[u];
        }
      }
    }
    for (int t = threadIdx.x; t < nb * NC; t += 256) {
      const int jj = t / NC, c = t % NC;
      const float* hs = a.hs + (size_t)(q0 + j0 + jj) * (I / 16);
      hsum_s[jj][c] = hs[2 * c] + hs[2 * c + 1];
    }
    for (int t = threadIdx.x; t < nb * r; t += 256) {
      const int jj = t / r, rr = t % r;
      td_s[jj][rr] = from_fix(a.tdown[(size_t)(q0 + j0 + jj) * r + rr]);
    }
    __syncthreads();
    const Q4Consts kq = q4_consts();
#pragma unroll
    for (int jj = 0; jj < kGrpBT; ++jj) {
      float part = 0.f;
      if (jj < nb) {
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
          const int c = wave + 4 * m;
          if (c < NC) {
            const uint32_t* hp = hp_s[jj][c];
            const float accv = chunk_dot128(qv[m], hp, kq) + chunk_dot128(qv[m], hp + 16, kq);
            part += sv[m] * accv + cv[m] * hsum_s[jj][c];
          }
        }
      }
      red[wave][jj][lane] = part;
    }
    __syncthreads();
    if (wave == 0) {
      for (int jj = 0; jj < nb; ++jj) {
        float tot = red[0][jj][lane] + red[1][jj][lane] + red[2][jj][lane] + red[3][jj][lane];
        if (r > 0) {
          float dl = 0.f;
#pragma unroll
          for (int m = 0; m < 32; ++m)
            if (2 * m < r) dl += bf_lo(bd[m]) * td_s[jj][2 * m] + bf_hi(bd[m]) * td_s[jj][2 * m + 1];
          tot += a.scale * dl;
        }
        const int q = q0 + j0 + jj;
        atomicAdd(a.acc + (size_t)a.pair_tok[q] * d + o, to_fix(a.pair_w[q] * tot));
      }
    }
  }
}

// ------------------------------------------------ MFMA token tiles
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
// activations as the MFMA operand: 8 consecutive bf16 in the pair order
// (e0,e4,e1,e5,e2,e6,e3,e7) of the packed int4 words
__device__ __forceinline__ bf16x8_t x_operand(uint4 raw) {
  uint32_t o[4];
  pair_perm8(raw.x, raw.y, raw.z, raw.w, o);
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}
// Every active expert on v_mfma_f32_16x16x32_bf16, whatever its token
// count: A = up to 16 of the expert's tokens x 32 inputs, B = 32 inputs x 16
// weight rows.  Lane l = (n = l % 16, j = l / 16) supplies token n's and
// weight row n's inputs k0 .. k0 + 7 (the same inputs for both operands, so
// the product does not depend on how the unit orders k inside the lanes);
// accumulator v of lane l is C[token 4 j + v][row n].  Within a group of g
// inputs quad j takes the g/4 inputs from j g/4 on, one packed word (8
// inputs) per step, WPG = g/32 steps; per group the products start from
// zero and are folded in fp32 as s * acc + (b - 128 s) * (the group's
// activation sum).  The int4 operand is expanded once per tile of up to 16
// tokens, so an expert's cost barely grows with its token count.  Rows
// staged in LDS are swizzled (16-byte chunk c of token m at c ^ (m & 15)),
// so the 16 lanes of a quad read 16 different banks.  A workgroup's first
// loads (its expert's count, slot and first pair) go out together.
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t q4_operand_k(uint32_t w, Q4Consts k) {
  const uint4 v = make_uint4((w & k.m) | k.c, ((w >> 4) & k.m) | k.c, ((w >> 8) & k.m) | k.c,
                             ((w >> 12) & k.m) | k.c);
  return __builtin_bit_cast(bf16x8_t, v);
}
constexpr int kTileTok = 16;   // tokens per MFMA tile at most
constexpr int kTileRank = 16;  // LoRA rank bound of the tile kernels
constexpr int kTileMinCall = 3;  // default: tiles for calls of >= 3 tokens (measured crossover)
constexpr int kDownNT = 2;  // 64-row blocks per down workgroup (a 16-row n-tile each per wave)

// N consecutive 32-bit words from p (p aligned to min(N, 4) words)
template <int N>
__device__ __forceinline__ void load_u32s(const uint32_t* p, uint32_t* w) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int u = 0; u < N / 4; ++u) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[u];
      w[4 * u] = v.x;
      w[4 * u + 1] = v.y;
      w[4 * u + 2] = v.z;
      w[4 * u + 3] = v.w;
    }
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    w[0] = p[0];
  }
}
__device__ __forceinline__ float bf_at(const uint32_t* w, int i) {
  return (i & 1) ? bf_hi(w[i >> 1]) : bf_lo(w[i >> 1]);
}
// element offset of input k of staged row m (rows of len bf16, len % 128 == 0)
__device__ __forceinline__ int swz(int m, int len, int k) {
  return m * len + ((((k >> 3) ^ (m & 15))) << 3) + (k & 7);
}

// The tile's pair tokens through the scalar cache: pair_tok is not written
// while the tile kernels run, so it may be read as constant memory, and a
// wait for these loads does not wait for the vector loads in flight.
__device__ __forceinline__ int tile_pair_tok(const GrpArgs& a, int q) {
  const __attribute__((address_space(4))) int32_t* p =
      (const __attribute__((address_space(4))) int32_t*)a.pair_tok;
  return p[q];
}
__device__ __forceinline__ int tile_pair_src(const GrpArgs& a, int q) {
  const __attribute__((address_space(4))) int32_t* p =
      (const __attribute__((address_space(4))) int32_t*)a.pair_src;
  return p[q];
}

// Gate/up: workgroup (tile, active expert, 16-row block).  The 4 waves split
// the d inputs into quarters of GW groups (NW = GW * WPG words per lane per
// matrix, loaded once); each lane reads its token's activations straight
// from memory (the quarters do not overlap, so staging them would save
// nothing), and a third MFMA per step against a ones operand gives each
// group's activation sum for the fold.  The partial 16 x 16 gate and up
// tiles meet in LDS; then one thread per (token, row): LoRA B t, SwiGLU, h
// as bf16 hi/lo pairs, 16-row sums of h, and A_down h added in fixed point
// per (pair, rank).  An expert holds at most T pairs (one per token), so
// the grid's ceil(T / tm) tiles cover it and a workgroup has one tile:
// straight-line code, nothing loop-carried.
struct GuTileLds {
  float4 red[kTileTok][kTileTok][2];  // [token][row]: gate then up partials of the 4 waves
  float bl[2][kTileTok][kTileRank];
  float tl[kTileTok][2][kTileRank];
  float h[kTileTok][kTileTok];  // read back as whole rows (float4)
};

template <int GW, int WPG>
__device__ __forceinline__ void gu_tile(const GrpArgs& a, const uint8_t* b, int e, int q0, int t0,
                                        int mt, int blk, const uint32_t (&wg)[GW * WPG],
                                        const uint32_t (&wu)[GW * WPG], Q4Consts kq,
                                        GuTileLds& sm) {
  constexpr int NW = GW * WPG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, g = a.g, ng = d / g, r = a.r, I = a.I;
  const int i0 = blk * 16, row = i0 + n;
  const bool lora = r > 0;
  // this lane's A row: token n of the tile (rows past the tile repeat its
  // last token; their results are dropped)
  int tok = tile_pair_tok(a, q0 + t0);
#pragma unroll
  for (int i = 1; i < kTileTok; ++i) {
    const int ti = tile_pair_tok(a, q0 + t0 + min(i, mt - 1));
    tok = n == i ? ti : tok;
  }
  const uint4* xp =
      reinterpret_cast<const uint4*>(a.x + (size_t)tok * d + wave * (d / 4) + j * (g / 4));
  uint4 xa[NW];
#pragma unroll
  for (int gl = 0; gl < GW; ++gl)
#pragma unroll
    for (int s = 0; s < WPG; ++s) xa[gl * WPG + s] = xp[(gl * g + 8 * s) / 8];
  // scales and biases of this lane's row and groups; A_down[rr][i0 .. i0+15]
  // for thread (token, rr = tid % 16), rank clamped
  uint32_t sgw[GW / 2], gbw[GW / 2], suw[GW / 2], ubw[GW / 2];
  {
    const size_t so = ((size_t)row * ng + wave * GW) / 2;  // in words
    load_u32s<GW / 2>(reinterpret_cast<const uint32_t*>(b + a.lay.gate_s) + so, sgw);
    load_u32s<GW / 2>(reinterpret_cast<const uint32_t*>(b + a.lay.gate_b) + so, gbw);
    load_u32s<GW / 2>(reinterpret_cast<const uint32_t*>(b + a.lay.up_s) + so, suw);
    load_u32s<GW / 2>(reinterpret_cast<const uint32_t*>(b + a.lay.up_b) + so, ubw);
  }
  const int rr = tid & 15;
  const uint4* adp = reinterpret_cast<const uint4*>(
      lora ? grp_lora(a, b, e, 4, a.lay.a_down) + ((size_t)min(rr, r - 1) * I + i0) * 2
           : b + a.lay.gate_q);
  const uint4 ad0 = adp[0], ad1 = adp[1];
  if (lora) {
    // rank entries past r are zero, so the epilogue's dot runs over
    // kTileRank entries with every read issued at once
    for (int t = tid; t < 2 * 16 * kTileRank; t += 256) {
      const int p = t / (16 * kTileRank), rw = (t / kTileRank) % 16, k = t % kTileRank;
      const uint16_t* B = reinterpret_cast<const uint16_t*>(
          grp_lora(a, b, e, p ? 3 : 1, p ? a.lay.b_up : a.lay.b_gate));
      sm.bl[p][rw][k] = k < r ? bf2f(B[(size_t)(i0 + rw) * r + k]) : 0.f;
    }
    for (int t = tid; t < kTileTok * 2 * kTileRank; t += 256) {
      const int m = t / (2 * kTileRank), p = (t / kTileRank) & 1, k = t % kTileRank;
      const int src = tile_pair_src(a, q0 + t0 + min(m, mt - 1));
      sm.tl[m][p][k] = m < mt && k < r ? a.t_in[((size_t)src * 2 + p) * r + k] : 0.f;
    }
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u,
                                                                0x3F803F80u, 0x3F803F80u));
  f32x4_t accG = {0.f, 0.f, 0.f, 0.f}, accU = accG;
#pragma unroll
  for (int gl = 0; gl < GW; ++gl) {
    f32x4_t cg = {0.f, 0.f, 0.f, 0.f}, cu = cg, cx = cg;
#pragma unroll
    for (int s = 0; s < WPG; ++s) {
      const bf16x8_t xo = x_operand(xa[gl * WPG + s]);
      cg = mfma16(xo, q4_operand_k(wg[gl * WPG + s], kq), cg);
      cu = mfma16(xo, q4_operand_k(wu[gl * WPG + s], kq), cu);
      cx = mfma16(xo, ones, cx);
    }
    const float sg = bf_at(sgw, gl), cbg = bf_at(gbw, gl) - 128.f * sg;
    const float su = bf_at(suw, gl), cbu = bf_at(ubw, gl) - 128.f * su;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      accG[v] += sg * cg[v] + cbg * cx[v];
      accU[v] += su * cu[v] + cbu * cx[v];
    }
    // one group at a time: expanding every group's operands ahead would
    // take more registers than the occupancy allows
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    reinterpret_cast<float*>(&sm.red[4 * j + v][n][0])[wave] = accG[v];
    reinterpret_cast<float*>(&sm.red[4 * j + v][n][1])[wave] = accU[v];
  }
  __syncthreads();
  const int m = tid >> 4, rn = tid & 15;  // the 16 threads of token m are one DPP row
  {
    const float4 pg = sm.red[m][rn][0], pu = sm.red[m][rn][1];
    float Gv = pg.x + pg.y + pg.z + pg.w;
    float Uv = pu.x + pu.y + pu.z + pu.w;
    if (lora) {
      float dg = 0.f, du = 0.f;
#pragma unroll
      for (int k = 0; k < kTileRank; ++k) {
        dg += sm.bl[0][rn][k] * sm.tl[m][0][k];
        du += sm.bl[1][rn][k] * sm.tl[m][1][k];
      }
      Gv += a.scale * dg;
      Uv += a.scale * du;
    }
    const float h = grp_silu(Gv) * Uv;
    const bool ok = m < mt;
    float hr = 0.f;
    if (ok) hr = grp_store_h(a, q0 + t0 + m, i0 + rn, h);
    sm.h[m][rn] = ok ? h : 0.f;
    const float s16 = row16_sum(hr);
    if (rn == 0 && ok) a.hs[(size_t)(q0 + t0 + m) * (I / 16) + blk] = s16;
  }
  __syncthreads();  // h written
  if (lora && m < mt && rr < r) {
    const uint32_t w8[8] = {ad0.x, ad0.y, ad0.z, ad0.w, ad1.x, ad1.y, ad1.z, ad1.w};
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += bf_lo(w8[u]) * sm.h[m][2 * u] + bf_hi(w8[u]) * sm.h[m][2 * u + 1];
    atomicAdd(a.tdown + (size_t)(q0 + t0 + m) * r + rr, to_fix(s));
  }
}

template <int GW, int WPG>
__global__ __launch_bounds__(256, 3) void k_grp_gu_tile(GrpArgs a, int tm, int min_cnt) {
  constexpr int NW = GW * WPG;
  __shared__ GuTileLds sm;
  const int nblk = a.I / 16;
  const int blk = blockIdx.x % nblk;
  const int tt = blockIdx.x / (a.Amax * nblk), act = (blockIdx.x / nblk) % a.Amax;
  // everything the start depends on, in one round trip
  const int n_act = a.info[0], cnt = a.act_cnt[act], slot = a.act_slot[act], q0 = a.act_off[act];
  asm volatile("" ::"s"(n_act), "s"(cnt), "s"(slot), "s"(q0));
  const int t_first = tt * tm;
  if (act >= n_act || t_first >= cnt || cnt < min_cnt || slot < 0) return;
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, g = a.g;
  const int row = blk * 16 + n;
  // this lane's weight words: groups wave * GW + gl, quad j
  uint32_t wg[NW], wu[NW];
  {
    const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q) + (size_t)row * (d / 8);
    const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q) + (size_t)row * (d / 8);
#pragma unroll
    for (int gl = 0; gl < GW; ++gl) {
      const int off = (wave * GW + gl) * (g / 8) + j * WPG;
      load_u32s<WPG>(gq + off, wg + gl * WPG);
      load_u32s<WPG>(uq + off, wu + gl * WPG);
    }
  }
  const Q4Consts kq = q4_consts();
  const int e = a.lora_sep ? a.act_e[act] : 0;  // the expert, for adapters given apart
  gu_tile<GW, WPG>(a, b, e, q0, t_first, min(tm, cnt - t_first), blk, wg, wu, kq, sm);
}

// Down: workgroup (tile, active expert, kDownNT blocks of 64 output rows);
// wave w owns rows 16 w .. 16 w + 15 of each block (one 16-row n-tile per
// block) over all I inputs (NW = I / 32 words per lane and n-tile, GD =
// NW / WPG groups, loaded once), two MFMAs per step and n-tile (h as its hi
// and lo bf16 halves, pair-permuted as stored) against rows staged in LDS
// once for the workgroup; then the LoRA-down delta and each token's
// weighted row added to its fixed-point output.  Dynamic LDS: hi and lo h
// of tm pairs, rows of I bf16.  One tile per workgroup, as for gate/up.
template <int NW, int WPG>
__device__ __forceinline__ void down_tile(const GrpArgs& a, const uint8_t* b, int e, int q0,
                                          int t0, int mt, int tm, int rb,
                                          const uint32_t (&wd)[kDownNT][NW], Q4Consts kq,
                                          uint16_t* hsm, float (&gsum)[kTileTok][NW / WPG],
                                          float (&td_s)[kTileTok][kTileRank]) {
  constexpr int GD = NW / WPG, NT = kDownNT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, g = a.g, I = a.I, r = a.r;
  const bool lora = r > 0;
  uint16_t* hh = hsm;
  uint16_t* hl = hsm + (size_t)tm * I;
  const int cpt = I / 8;  // 16-byte chunks per h row
  // hi and lo h of the tile's pairs (contiguous rows): NW / 2 chunks per
  // thread at tm = 16, all loads first
  uint4 v[NW / 2];
#pragma unroll
  for (int u = 0; u < NW / 2; ++u) {
    const int idx = tid + 256 * u;
    const int half = idx / (tm * cpt), rem = idx % (tm * cpt);  // half: 0 hi, 1 lo
    const uint16_t* src = half == 1 ? a.hp_lo : a.hp_hi;
    v[u] = reinterpret_cast<const uint4*>(
        src + ((size_t)(q0 + t0 + min(rem / cpt, mt - 1))) * I)[rem % cpt];
  }
  // per output row o of each n-tile: scales, biases and B_down (pair index
  // clamped; r is even); the lane's 4 pairs' tokens and routing weights
  uint32_t sdr[NT][GD], dbr[NT][GD], bdw[NT][kTileRank / 2];
  {
    const uint16_t* ds = reinterpret_cast<const uint16_t*>(b + a.lay.down_s);
    const uint16_t* db = reinterpret_cast<const uint16_t*>(b + a.lay.down_b);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int o = (rb * NT + t) * 64 + 16 * wave + n;
#pragma unroll
      for (int G = 0; G < GD; ++G) {
        sdr[t][G] = ds[(size_t)G * d + o];
        dbr[t][G] = db[(size_t)G * d + o];
      }
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          lora ? grp_lora(a, b, e, 5, a.lay.b_down) + (size_t)o * r * 2 : b + a.lay.down_q);
#pragma unroll
      for (int k = 0; k < kTileRank / 2; ++k) bdw[t][k] = src[lora ? min(k, r / 2 - 1) : 0];
    }
  }
  int ptok[4];
  float pw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = q0 + t0 + min(4 * j + u, mt - 1);
    ptok[u] = a.pair_tok[q];
    pw[u] = a.pair_w[q];
  }
#pragma unroll
  for (int u = 0; u < NW / 2; ++u) {
    const int idx = tid + 256 * u;
    const int half = idx / (tm * cpt), rem = idx % (tm * cpt);
    if (half < 2)
      *reinterpret_cast<uint4*>((half ? hl : hh) + swz(rem / cpt, I, 8 * (rem % cpt))) =
          rem / cpt < mt ? v[u] : make_uint4(0, 0, 0, 0);
  }
  const int bpg = g / 16;  // 16-row sums per group
  for (int t = tid; t < tm * GD; t += 256) {
    const int m = t / GD, G = t % GD;
    float s = 0.f;
    if (m < mt) {
      const float* hs = a.hs + (size_t)(q0 + t0 + m) * (I / 16) + G * bpg;
      for (int u = 0; u < bpg; ++u) s += hs[u];
    }
    gsum[m][G] = s;
  }
  if (lora) {
    for (int t = tid; t < tm * kTileRank; t += 256) {
      const int m = t / kTileRank, k = t % kTileRank;
      td_s[m][k] = m < mt && k < r ? from_fix(a.tdown[(size_t)(q0 + t0 + m) * r + k]) : 0.f;
    }
  }
  __syncthreads();
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nr = min(n, tm - 1);
#pragma unroll
  for (int G = 0; G < GD; ++G) {
    f32x4_t c[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) c[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < WPG; ++s) {
      const int e = swz(nr, I, G * g + j * (g / 4) + 8 * s);
      const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(hh + e));
      const bf16x8_t al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(hl + e));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8_t wo = q4_operand_k(wd[t][G * WPG + s], kq);
        c[t] = mfma16(ah, wo, c[t]);
        c[t] = mfma16(al, wo, c[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float sd = bf2f(sdr[t][G]), cbd = bf2f(dbr[t][G]) - 128.f * sd;
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[t][u] += sd * c[t][u] + cbd * gsum[min(4 * j + u, tm - 1)][G];
    }
    __builtin_amdgcn_sched_barrier(0);  // one group's LDS reads at a time
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int m = 4 * j + u;
    if (m < mt) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float tot = acc[t][u];
        if (lora) {
          float dl = 0.f;
#pragma unroll
          for (int k = 0; k < kTileRank / 2; ++k)
            dl += bf_lo(bdw[t][k]) * td_s[m][2 * k] + bf_hi(bdw[t][k]) * td_s[m][2 * k + 1];
          tot += a.scale * dl;
        }
        const int o = (rb * NT + t) * 64 + 16 * wave + n;
        atomicAdd(a.acc + (size_t)ptok[u] * d + o, to_fix(pw[u] * tot));
      }
    }
  }
}

template <int NW, int WPG>
__global__ __launch_bounds__(256, 2) void k_grp_down_tile(GrpArgs a, int tm, int min_cnt) {
  constexpr int GD = NW / WPG;
  extern __shared__ __align__(16) uint16_t hsm[];
  __shared__ float gsum[kTileTok][GD];
  __shared__ float td_s[kTileTok][kTileRank];  // zero past the rank
  const int nrb = a.d / (64 * kDownNT);
  const int rb = blockIdx.x % nrb;
  const int tt = blockIdx.x / (a.Amax * nrb), act = (blockIdx.x / nrb) % a.Amax;
  const int n_act = a.info[0], cnt = a.act_cnt[act], slot = a.act_slot[act], q0 = a.act_off[act];
  asm volatile("" ::"s"(n_act), "s"(cnt), "s"(slot), "s"(q0));
  const int t_first = tt * tm;
  if (act >= n_act || t_first >= cnt || cnt < min_cnt || slot < 0) return;
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int g = a.g, NC = a.I / 32;
  uint32_t wd[kDownNT][NW];
  {
    const uint32_t* dq = reinterpret_cast<const uint32_t*>(b + a.lay.down_q);
#pragma unroll
    for (int t = 0; t < kDownNT; ++t)
#pragma unroll
      for (int G = 0; G < GD; ++G) {
        const int k0 = G * g + j * (g / 4);
        load_u32s<WPG>(dq + (((size_t)(rb * kDownNT + t) * NC + (k0 >> 5)) * 64 + 16 * wave + n) * 4 +
                           ((k0 & 31) >> 3),
                       wd[t] + G * WPG);
      }
  }
  const Q4Consts kq = q4_consts();
  const int e = a.lora_sep ? a.act_e[act] : 0;  // the expert, for adapters given apart
  down_tile<NW, WPG>(a, b, e, q0, t_first, min(tm, cnt - t_first), tm, rb, wd, kq, hsm, gsum,
                     td_s);
}

// ------------------------------------------------------------ output
__global__ __launch_bounds__(256) void k_grp_out(GrpArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < a.T * a.d) {
    a.y[i] = (uint16_t)f2bf(from_fix(a.acc[i]));
    a.acc[i] = 0ull;
  }
  for (int j = i; j < a.P * a.r; j += gridDim.x * 256) a.tdown[j] = 0ull;
}

// ------------------------------------------------------------ prefill
// The whole-layer path for a prompt chunk ([Edge0] §3.1 "Executor paths",
// whole-layer; §3.2 "Two consumption profiles": prefill hits every expert of
// a layer).  Token by token the same result as the grouped call, for up to
// kPfMaxTokens tokens: the bucketing runs over many workgroups and lists
// the (expert, tile) units that exist (16-pair tiles for the LoRA A x on
// MFMA, 64-pair tiles for the gate/up and down GEMMs), so the grids cover
// those units rather than every (tile, expert) combination.  Pairs are
// placed in an expert's run in arrival order; a pair's results do not depend
// on its place (every MFMA output element is its own row's dot product, and
// a token's K rows are added in k order), so calls are bit-reproducible.
constexpr int kPfMaxTokens = 4096;

// pass 1: per pair, an id repeated within its token is dropped (its first
// listing keeps the weights summed in k order); kept pairs counted per
// expert, in LDS per workgroup of kPfPairsPerWg pairs first (the global
// counters then take at most E additions per workgroup: a few thousand
// pairs adding one by one into E counters serialise on them)
constexpr int kPfPairsPerWg = 4096;
__global__ __launch_bounds__(1024) void k_pf_count(GrpArgs a, int32_t* cnt, int32_t* keep,
                                                   float* keep_w) {
  __shared__ int hist[1024];  // E <= 1024
  for (int e = threadIdx.x; e < a.E; e += 1024) hist[e] = 0;
  __syncthreads();
  const int K = a.K;
  for (int p = blockIdx.x * kPfPairsPerWg + threadIdx.x;
       p < min(a.P, (blockIdx.x + 1) * kPfPairsPerWg); p += 1024) {
    const int k0 = p - p % K;
    int e = a.ids[p];
    float w = a.w[p];
    if (e < 0 || e >= a.E) {
      set_error(a.err, EDGE0_ERANGE);
      e = -1;
    } else {
      bool dup = false;
      for (int q = k0; q < p; ++q) dup |= a.ids[q] == e;
      for (int q = p + 1; q < k0 + K; ++q)
        if (a.ids[q] == e) w += a.w[q];
      if (dup) e = -1;
    }
    keep[p] = e;
    keep_w[p] = w;
    if (e >= 0) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += 1024)
    if (hist[e] != 0) atomicAdd(cnt + e, hist[e]);
}

// pass 2 (one workgroup, one expert per thread): exclusive scans of the
// counts, the active flags and the 64-pair tiles per expert; the active
// list, each expert's first free position, the tile list; the counts
// cleared
constexpr int kPfTile = 64;  // pairs per prefill GEMM tile (4 waves x 16)
__global__ __launch_bounds__(1024) void k_pf_scan(GrpArgs a, int32_t* cnt, int32_t* fill,
                                                  int2* tiles64) {
  __shared__ int wtot[3][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const int c = tid < E ? cnt[tid] : 0;
  const int f = c > 0 ? 1 : 0;
  const int n64 = (c + kPfTile - 1) / kPfTile;
  const int ic = wave_incl_scan(c), iff = wave_incl_scan(f), i64 = wave_incl_scan(n64);
  if (lane == 63) {
    wtot[0][wave] = ic;
    wtot[1][wave] = iff;
    wtot[2][wave] = i64;
  }
  __syncthreads();
  int bc = 0, bf = 0, b64 = 0, tc = 0, tf = 0, t64 = 0;
  for (int v = 0; v < 16; ++v) {
    if (v < wave) {
      bc += wtot[0][v];
      bf += wtot[1][v];
      b64 += wtot[2][v];
    }
    tc += wtot[0][v];
    tf += wtot[1][v];
    t64 += wtot[2][v];
  }
  const int xc = bc + ic - c, xf = bf + iff - f, x64 = b64 + i64 - n64;
  if (tid < E) {
    fill[tid] = xc;
    cnt[tid] = 0;
    if (f) {
      const int slot = a.table[tid];
      const bool ok = slot >= 0 && slot < a.n_slots;
      a.act_e[xf] = tid;
      a.act_off[xf] = xc;
      a.act_cnt[xf] = c;
      a.act_slot[xf] = ok ? slot : -1;
      if (!ok) set_error(a.err, EDGE0_ERANGE);
      for (int i = 0; i < n64; ++i) tiles64[x64 + i] = make_int2(xf, i);
    }
  }
  if (tid == 0) {
    a.info[0] = tf;
    a.info[1] = tc;
    a.info[3] = t64;
  }
}

// pass 3: each kept pair to a free position of its expert's run: the
// workgroup ranks its pairs per expert in LDS and reserves one block per
// expert (the order within a run is arrival order; results do not depend
// on it)
__global__ __launch_bounds__(1024) void k_pf_scatter(GrpArgs a, const int32_t* keep,
                                                     const float* keep_w, int32_t* fill) {
  __shared__ int lcnt[1024], lbase[1024];  // E <= 1024
  constexpr int PPT = kPfPairsPerWg / 1024;
  for (int e = threadIdx.x; e < a.E; e += 1024) lcnt[e] = 0;
  __syncthreads();
  int ev[PPT], rank[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = blockIdx.x * kPfPairsPerWg + threadIdx.x + 1024 * i;
    ev[i] = p < a.P ? keep[p] : -1;
    rank[i] = ev[i] >= 0 ? atomicAdd(&lcnt[ev[i]], 1) : 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += 1024)
    if (lcnt[e] != 0) lbase[e] = atomicAdd(fill + e, lcnt[e]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    if (ev[i] < 0) continue;
    const int p = blockIdx.x * kPfPairsPerWg + threadIdx.x + 1024 * i;
    const int dst = lbase[ev[i]] + rank[i];
    a.pair_tok[dst] = p / a.K;
    a.pair_src[dst] = p;
    a.pair_w[dst] = keep_w[p];
  }
}

// LoRA A x of a 64-pair tile, one workgroup per entry of the tile list: the
// tile's tokens (A operand, rows = tokens, four 16-row blocks) against the
// expert's 2r LoRA A rows (B operand; row q < r is A_gate's row q, then
// A_up's), bf16 MFMA 16x16x32 in one or two 16-row n-tiles, each step's B
// fragments loaded once for the four blocks; the 4 waves take quarters of
// d and their partials are summed in LDS in wave order.  Both operands
// carry the same 8 inputs per lane, in their natural order.
__global__ __launch_bounds__(256) void k_pf_lora_in(GrpArgs a) {
  __shared__ float part[4][kPfTile][2 * kTileRank];
  const int li = blockIdx.x;
  if (li >= a.info[3]) return;
  const int2 te = a.tiles64[li];
  const int cnt = a.act_cnt[te.x], slot = a.act_slot[te.x], q0 = a.act_off[te.x];
  if (slot < 0) return;  // reported by the scan; the GEMM kernels skip it too
  const int t0 = te.y * kPfTile, mt = min(kPfTile, cnt - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int r = a.r, d = a.d;
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const uint16_t* xr[4];  // this lane's token in each 16-row block (past the tile: its last)
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
    xr[tb] = a.x + (size_t)a.pair_tok[q0 + t0 + min(16 * tb + n, mt - 1)] * d;
  const int q1 = n, q2 = 16 + n;  // this lane's B rows in the two n-tiles
  const int e = a.lora_sep ? a.act_e[te.x] : 0;  // the expert, for adapters given apart
  const bool up1 = q1 >= r, up2 = q2 < 2 * r && q2 >= r;
  const uint16_t* w1 = reinterpret_cast<const uint16_t*>(
                           grp_lora(a, b, e, up1 ? 2 : 0, up1 ? a.lay.a_up : a.lay.a_gate)) +
                       (size_t)(q1 % r) * d;
  const uint16_t* w2 = reinterpret_cast<const uint16_t*>(
                           grp_lora(a, b, e, up2 ? 2 : 0, up2 ? a.lay.a_up : a.lay.a_gate)) +
                       (size_t)(q2 < 2 * r ? q2 % r : 0) * d;
  const bool two = 2 * r > 16;
  f32x4_t c1[4], c2[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) c1[tb] = c2[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kq = d / 4;
  for (int k0 = wave * kq; k0 < (wave + 1) * kq; k0 += 32) {
    const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(w1 + k0 + 8 * j));
    const bf16x8_t b2 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(w2 + k0 + 8 * j));
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const bf16x8_t xo =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(xr[tb] + k0 + 8 * j));
      c1[tb] = mfma16(xo, b1, c1[tb]);
      if (two) c2[tb] = mfma16(xo, b2, c2[tb]);
    }
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      part[wave][16 * tb + 4 * j + v][q1] = c1[tb][v];
      part[wave][16 * tb + 4 * j + v][q2] = two ? c2[tb][v] : 0.f;
    }
  __syncthreads();
  for (int e = tid; e < kPfTile * 2 * r; e += 256) {
    const int m = e / (2 * r), q = e % (2 * r);
    if (m < mt) {
      const float t = part[0][m][q] + part[1][m][q] + part[2][m][q] + part[3][m][q];
      const int src = a.pair_src[q0 + t0 + m];
      a.t_in[((size_t)src * 2 + q / r) * r + q % r] = t;
    }
  }
}

// ------------------------------------------------ prefill GEMM tiles
// A workgroup of the gate/up and down GEMMs covers a 64-pair tile of one
// expert (wave w: pairs 16 w .. 16 w + 15, the MFMA A rows) and a block of
// weight rows, and walks the inputs one quantisation group at a time: the
// group's activations (or h) and int4 words are staged in LDS, shared by the
// four waves, double-buffered (the next group's loads go out while the
// current one is multiplied); per group the products start from zero and
// are folded in fp32 as s * acc + (b - 128 s) * (the group's activation
// sum), as in the token tiles.  No atomics: the gate/up kernel stores h
// (bf16 hi/lo pairs, pair order) and its per-32-row sums, the down kernel
// computes A_down h itself (two more MFMAs per step against the A_down
// rows) and stores each pair's weighted output row, and the combine sums a
// token's K rows in k order.  Every output element is its own row's dot
// product whatever its tile mates, so calls are bit-reproducible.

// workgroup -> logical unit, XCD-aware: consecutive workgroups go to
// different XCDs, so unit u = (id % 8) * (n / 8) + id / 8 keeps a range of
// consecutive units (a tile's row blocks, an expert's tiles) on one XCD and
// its L2 (n a multiple of 8)
__device__ __forceinline__ int pf_unit() {
  const int id = blockIdx.x, n = gridDim.x;
  return (id % 8) * (n / 8) + id / 8;
}

// each token's activation sum per input group, fp32 in input order
__global__ __launch_bounds__(256) void k_pf_xsum(GrpArgs a, float* xsum) {
  const int ng = a.d / a.g;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.T * ng) return;
  const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)(i / ng) * a.d + (i % ng) * a.g);
  float s = 0.f;
  for (int c = 0; c < a.g / 8; ++c) {
    const uint4 v = src[c];
    s += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) +
         bf_lo(v.w) + bf_hi(v.w);
  }
  xsum[i] = s;
}

// 8 bf16 of an fp32 row as the hi and lo halves of an MFMA operand (k
// inputs in natural order; zeros where `ok` is false)
struct F8 {
  float4 a, b;
};
__device__ __forceinline__ void split_hilo8(F8 f, bool ok, bf16x8_t& hi, bf16x8_t& lo) {
  const float v[8] = {f.a.x, f.a.y, f.a.z, f.a.w, f.b.x, f.b.y, f.b.z, f.b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = ok ? v[2 * e] : 0.f, a1 = ok ? v[2 * e + 1] : 0.f;
    const uint32_t h0 = f2bf(a0), h1 = f2bf(a1);
    h[e] = h0 | (h1 << 16);
    l[e] = f2bf(a0 - bf2f(h0)) | (f2bf(a1 - bf2f(h1)) << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// 8 floats as three bf16 MFMA operands, hi + mid + lo (24 significant bits:
// the fp32 value to within its own rounding)
__device__ __forceinline__ void split3_8(F8 f, bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
  const float v[8] = {f.a.x, f.a.y, f.a.z, f.a.w, f.b.x, f.b.y, f.b.z, f.b.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t hh[2], mm[2], ll[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float x = v[2 * e + q];
      hh[q] = f2bf(x);
      const float r1 = x - bf2f(hh[q]);
      mm[q] = f2bf(r1);
      ll[q] = f2bf(r1 - bf2f(mm[q]));
    }
    h[e] = hh[0] | (hh[1] << 16);
    m[e] = mm[0] | (mm[1] << 16);
    l[e] = ll[0] | (ll[1] << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  mid = __builtin_bit_cast(bf16x8_t, make_uint4(m[0], m[1], m[2], m[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// c . x on MFMA to fp32 quality from three-way splits: the cross products
// down to 2^-16 of the leading one (hi hi, hi mid, mid hi, hi lo, lo hi, mid mid)
__device__ __forceinline__ f32x4_t mfma16_x3(const bf16x8_t (&a)[3], const bf16x8_t (&b)[3],
                                             f32x4_t c) {
  c = mfma16(a[0], b[0], c);
  c = mfma16(a[0], b[1], c);
  c = mfma16(a[1], b[0], c);
  c = mfma16(a[0], b[2], c);
  c = mfma16(a[2], b[0], c);
  c = mfma16(a[1], b[1], c);
  return c;
}

// Gate/up: unit (64-pair tile, 64 rows of gate and of up); wave w owns rows
// 16 w .. 16 w + 15 of both over the tile's four 16-pair blocks, so each
// int4 word is expanded once, straight from memory into registers, and
// SwiGLU pairs gate and up in registers.  The activations go through LDS
// (pair order, swizzled), two groups a step, double-buffered; the next
// step's weights, scales and activations are loaded while the current one
// is multiplied.  Within a group, lane quad j takes KS of its chunks, so
// an MFMA never mixes groups, and a group's products enter the
// accumulators as s * acc.  The group affine's other half,
// sum over groups of (b - 128 s) * (the pair's activation sum of the
// group), is a small product of its own: after the loop it runs on MFMA with
// both factors split three ways into bf16 (it nearly cancels the 128 s part
// of the first half, so it needs fp32's precision), added into the same
// accumulators.  Epilogue: the LoRA B t terms on MFMA (t as bf16 hi +
// lo), h as bf16 hi/lo pairs through LDS to full-width stores, and each
// wave's 16-row sums of h (hi + lo) for the down fold.
constexpr int kPfRows = 64;  // gate and up rows per k_pf_gu workgroup
template <int KS>
__global__ __launch_bounds__(256, 2) void k_pf_gu(GrpArgs a) {
  constexpr int G = 32 * KS, CPG = G / 8, NGI = 2;  // inputs, chunks per group; groups a step
  constexpr int CPB = 2 * CPG, STEP = 2 * G;         // 16-byte chunks, inputs a step
  constexpr int XU = kPfTile * CPB / 256;            // activation chunks staged per thread
  __shared__ __align__(16) uint4 xs[2][kPfTile * CPB];   // chunk c of pair m at CPB m + (c ^ m % CPB)
  __shared__ __align__(16) uint4 tlo[2][2][kPfTile][2];  // t of each pair: [gate, up][hi, lo]
  const int nblk = a.I / kPfRows;
  const int u = pf_unit();
  const int li = u / nblk, blk = u % nblk;
  if (li >= a.info[3]) return;
  const int2 te = a.tiles64[li];
  const int cnt = a.act_cnt[te.x], slot = a.act_slot[te.x], q0 = a.act_off[te.x];
  if (slot < 0) return;  // reported by the scan; the down kernel writes zeros
  const int t0 = te.y * kPfTile, mt = min(kPfTile, cnt - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, r = a.r, ng = d / G, nsteps = d / STEP;
  const int row = blk * kPfRows + 16 * wave + n;  // this lane's weight row
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const int e_lo = a.lora_sep ? a.act_e[te.x] : 0;  // the expert, for adapters given apart
  // staging duties: activation chunks (pairs past the tile repeat its last)
  const uint16_t* xrow[XU];
  int xdst[XU];
#pragma unroll
  for (int q = 0; q < XU; ++q) {
    const int c = tid + 256 * q, m = c / CPB, cc = c % CPB;
    xrow[q] = a.x + (size_t)a.pair_tok[q0 + t0 + min(m, mt - 1)] * d + 8 * cc;
    xdst[q] = m * CPB + (cc ^ (m % CPB));
  }
  // this lane's weight words: step s, k-step ks uses chunk (ks / KS) CPG + j KS + ks % KS
  const uint32_t* wgp = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q) + (size_t)row * (d / 8);
  const uint32_t* wup = reinterpret_cast<const uint32_t*>(b + a.lay.up_q) + (size_t)row * (d / 8);
  const uint16_t* sgp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s) + (size_t)row * ng;
  const uint16_t* bgp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b) + (size_t)row * ng;
  const uint16_t* sup = reinterpret_cast<const uint16_t*>(b + a.lay.up_s) + (size_t)row * ng;
  const uint16_t* bup = reinterpret_cast<const uint16_t*>(b + a.lay.up_b) + (size_t)row * ng;
  uint4 rx[XU];
  // sc: gate s, up s of the step's two groups, as loaded (bf16 pairs,
  // unpacked only where the fold uses them: work on a loaded value right
  // after its load would wait for it there)
  uint32_t wg[2 * KS], wu[2 * KS], sc[2];
  auto load_x = [&](int s) {
#pragma unroll
    for (int q = 0; q < XU; ++q) rx[q] = *reinterpret_cast<const uint4*>(xrow[q] + STEP * s);
  };
  auto load_w = [&](int s) {
#pragma unroll
    for (int ks = 0; ks < 2 * KS; ++ks) {
      const int c = s * CPB + (ks / KS) * CPG + j * KS + ks % KS;
      wg[ks] = wgp[c];
      wu[ks] = wup[c];
    }
    sc[0] = *reinterpret_cast<const uint32_t*>(sgp + s * NGI);
    sc[1] = *reinterpret_cast<const uint32_t*>(sup + s * NGI);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int q = 0; q < XU; ++q) {
      uint32_t o[4];
      pair_perm8(rx[q].x, rx[q].y, rx[q].z, rx[q].w, o);
      xs[buf][xdst[q]] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  // t of the tile's pairs (the LoRA A x launch), split hi/lo, rank-padded
  if (r > 0 && tid < 2 * kPfTile) {
    const int m = tid % kPfTile, p = tid / kPfTile;
    const float* tp = a.t_in + ((size_t)a.pair_src[q0 + t0 + min(m, mt - 1)] * 2 + p) * r;
    auto tk = [&](int k) { return k < r ? tp[k] : 0.f; };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const F8 f{make_float4(tk(8 * h), tk(8 * h + 1), tk(8 * h + 2), tk(8 * h + 3)),
                 make_float4(tk(8 * h + 4), tk(8 * h + 5), tk(8 * h + 6), tk(8 * h + 7))};
      bf16x8_t hi, lo;
      split_hilo8(f, true, hi, lo);
      tlo[p][0][m][h] = __builtin_bit_cast(uint4, hi);
      tlo[p][1][m][h] = __builtin_bit_cast(uint4, lo);
    }
  }
  load_x(0);
  load_w(0);
  store_x(0);
  __syncthreads();
  const Q4Consts kq = q4_consts();
  f32x4_t acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    uint32_t cwg[2 * KS], cwu[2 * KS], csc[2];
#pragma unroll
    for (int ks = 0; ks < 2 * KS; ++ks) {
      cwg[ks] = wg[ks];
      cwu[ks] = wu[ks];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) csc[q] = sc[q];
    if (s + 1 < nsteps) {
      load_x(s + 1);
      load_w(s + 1);
    }
    f32x4_t tmp[8];
#pragma unroll
    for (int ks = 0; ks < 2 * KS; ++ks) {
      const int gg = ks / KS;
      if (ks % KS == 0)
#pragma unroll
        for (int q = 0; q < 8; ++q) tmp[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int c = gg * CPG + j * KS + ks % KS;
      const bf16x8_t bg = q4_operand_k(cwg[ks], kq), bu = q4_operand_k(cwu[ks], kq);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int m = 16 * tb + n;
        const bf16x8_t xo = __builtin_bit_cast(bf16x8_t, xs[buf][m * CPB + (c ^ (m % CPB))]);
        tmp[tb] = mfma16(xo, bg, tmp[tb]);
        tmp[4 + tb] = mfma16(xo, bu, tmp[4 + tb]);
      }
      if (ks % KS == KS - 1) {
        const float sg = gg == 0 ? bf_lo(csc[0]) : bf_hi(csc[0]);
        const float su = gg == 0 ? bf_lo(csc[1]) : bf_hi(csc[1]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[tb][v] = fmaf(sg, tmp[tb][v], acc[tb][v]);
            acc[4 + tb][v] = fmaf(su, tmp[4 + tb][v], acc[4 + tb][v]);
          }
      }
    }
    if (s + 1 < nsteps) store_x(buf ^ 1);
    __syncthreads();
  }
  // the groups' (b - 128 s) terms: A = the pairs' activation sums (pair n of
  // block tb, groups k0 + 8 j ..), B = b - 128 s of row n over the same
  // groups; 32 groups an MFMA (groups past ng count as zeros, read at
  // clamped indices)
  const bool gvec = ng % 32 == 0;
  for (int k0 = 0; k0 < ng; k0 += 32) {
    const int g0 = k0 + 8 * j;
    float cg8[8], cu8[8];
    if (gvec) {
      const uint4 s8g = *reinterpret_cast<const uint4*>(sgp + g0);
      const uint4 b8g = *reinterpret_cast<const uint4*>(bgp + g0);
      const uint4 s8u = *reinterpret_cast<const uint4*>(sup + g0);
      const uint4 b8u = *reinterpret_cast<const uint4*>(bup + g0);
      const uint32_t sg4[4] = {s8g.x, s8g.y, s8g.z, s8g.w}, bg4[4] = {b8g.x, b8g.y, b8g.z, b8g.w};
      const uint32_t su4[4] = {s8u.x, s8u.y, s8u.z, s8u.w}, bu4[4] = {b8u.x, b8u.y, b8u.z, b8u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cg8[2 * e] = bf_lo(bg4[e]) - 128.f * bf_lo(sg4[e]);
        cg8[2 * e + 1] = bf_hi(bg4[e]) - 128.f * bf_hi(sg4[e]);
        cu8[2 * e] = bf_lo(bu4[e]) - 128.f * bf_lo(su4[e]);
        cu8[2 * e + 1] = bf_hi(bu4[e]) - 128.f * bf_hi(su4[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int gi = min(g0 + e, ng - 1);
        const bool in = g0 + e < ng;
        cg8[e] = in ? bf2f(bgp[gi]) - 128.f * bf2f(sgp[gi]) : 0.f;
        cu8[e] = in ? bf2f(bup[gi]) - 128.f * bf2f(sup[gi]) : 0.f;
      }
    }
    bf16x8_t cgs[3], cus[3];
    split3_8(F8{make_float4(cg8[0], cg8[1], cg8[2], cg8[3]),
                make_float4(cg8[4], cg8[5], cg8[6], cg8[7])}, cgs[0], cgs[1], cgs[2]);
    split3_8(F8{make_float4(cu8[0], cu8[1], cu8[2], cu8[3]),
                make_float4(cu8[4], cu8[5], cu8[6], cu8[7])}, cus[0], cus[1], cus[2]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int m = 16 * tb + n;
      const float* xp = a.xsum + (size_t)a.pair_tok[q0 + t0 + min(m, mt - 1)] * ng;
      F8 xf;
      if (gvec) {
        xf = F8{*reinterpret_cast<const float4*>(xp + g0), *reinterpret_cast<const float4*>(xp + g0 + 4)};
      } else {
        float x8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x8[e] = g0 + e < ng ? xp[min(g0 + e, ng - 1)] : 0.f;
        xf = F8{make_float4(x8[0], x8[1], x8[2], x8[3]), make_float4(x8[4], x8[5], x8[6], x8[7])};
      }
      bf16x8_t xs3[3];
      split3_8(xf, xs3[0], xs3[1], xs3[2]);
      acc[tb] = mfma16_x3(xs3, cgs, acc[tb]);
      acc[4 + tb] = mfma16_x3(xs3, cus, acc[4 + tb]);
    }
  }
  // LoRA B t: A = t of the pairs (ranks 8 j' .. as k, j' < 2), B = B rows
  if (r > 0) {
    bf16x8_t bl[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint16_t* B = reinterpret_cast<const uint16_t*>(
                              grp_lora(a, b, e_lo, p ? 3 : 1, p ? a.lay.b_up : a.lay.b_gate)) +
                          (size_t)row * r;
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 8 * j + 2 * e;
        const uint32_t lo16 = (j < 2 && k < r) ? B[k] : 0u;
        const uint32_t hi16 = (j < 2 && k + 1 < r) ? B[k + 1] : 0u;
        w4[e] = lo16 | (hi16 << 16);
      }
      bl[p] = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        f32x4_t lt = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int m = 16 * tb + n;
        uint4 t0v = tlo[p][0][m][j & 1], t1v = tlo[p][1][m][j & 1];
        if (j >= 2) t0v = t1v = make_uint4(0, 0, 0, 0);  // ranks 16..31 of the k-step
        const bf16x8_t th = __builtin_bit_cast(bf16x8_t, t0v);
        const bf16x8_t tlw = __builtin_bit_cast(bf16x8_t, t1v);
        lt = mfma16(th, bl[p], lt);
        lt = mfma16(tlw, bl[p], lt);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[4 * p + tb][v] += a.scale * lt[v];
      }
  }
  // SwiGLU; h hi/lo staged in LDS (the activation buffers are free now)
  uint16_t* hst = reinterpret_cast<uint16_t*>(&xs[0][0]);  // [hi, lo][pair][64 rows]
  const int hr = 16 * wave + n, pos = grp_pair_pos(hr);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float hv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * tb + 4 * j + v;
      const float h = grp_silu(acc[tb][v]) * acc[4 + tb][v];
      const uint32_t hi = f2bf(h), lo = f2bf(h - bf2f(hi));
      hst[m * kPfRows + pos] = (uint16_t)hi;
      hst[(kPfTile + m) * kPfRows + pos] = (uint16_t)lo;
      hv[v] = row16_sum(bf2f(hi) + bf2f(lo));
    }
    if (n == 0)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * tb + 4 * j + v;
        if (m < mt) a.hs[(size_t)(row / 16) * a.P + q0 + t0 + m] = hv[v];
      }
  }
  __syncthreads();
  // h to memory: 8 chunks of 8 per pair and half
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q, half = c >> 9, m = (c >> 3) & 63, cc = c & 7;
    if (m < mt)
      *reinterpret_cast<uint4*>((half ? a.hp_lo : a.hp_hi) + (size_t)(q0 + t0 + m) * a.I +
                                blk * kPfRows + 8 * cc) =
          *reinterpret_cast<const uint4*>(&hst[(half * kPfTile + m) * kPfRows + 8 * cc]);
  }
}

// Down: unit (64-pair tile, 128 output rows); wave w owns two 16-row blocks
// from 32 w over the four 16-pair blocks (h hi and lo, two
// MFMAs per block and step), its int4 words straight into registers, h
// through LDS (swizzled), 64 inputs a step, double-buffered; a group's
// products enter the accumulators as s * acc, and the groups' (b - 128 s)
// terms run after the loop on MFMA against each pair's h sums per group,
// kept in LDS as the steps stage them.  Wave w also forms A_down
// h for pair block w (the same two MFMAs against the A_down rows in pair
// order; no fold).  Epilogue: the LoRA-down term on MFMA (A_down h as bf16
// hi + lo against the B_down rows), then each pair's row times its routing
// weight, stored by unsorted pair.  A tile whose expert has no valid slot
// stores zeros.
// output rows per k_pf_down workgroup: 4 waves x 2 16-row blocks (four
// blocks per wave need more registers than a wave has, and the compiler
// then parks the staged h in scratch memory, behind a wait for its loads)
__host__ __device__ constexpr int pf_out(int) { return 128; }
constexpr int kPfGroupsPad = 33;  // input groups of the down projection (I / g <= 32), padded
template <int KS>
__global__ __launch_bounds__(256, 2) void k_pf_down(GrpArgs a) {
  constexpr int G = 32 * KS, NGD = 2 / KS;  // inputs per group; groups a step (64 inputs)
  constexpr int CPB = 8;                     // 16-byte chunks a step
  constexpr int HU = 2 * kPfTile * CPB / 256;
  constexpr int kPfOut = pf_out(KS), RB = kPfOut / 64;  // rows per unit, 16-row blocks per wave
  __shared__ __align__(16) uint4 hh[2][2][kPfTile * CPB];  // [buf][hi, lo], chunk c of pair m at 8 m + (c ^ m % 8)
  __shared__ __align__(16) float hsa[kPfTile][kPfGroupsPad];  // each pair's h sum per input group
  __shared__ __align__(16) uint4 ad[2][kTileRank * CPB];   // A_down rows (rank-padded), pair order
  __shared__ __align__(16) float td_s[kPfTile][kTileRank + 4];
  __shared__ int src_s[kPfTile];
  __shared__ float pw_s[kPfTile];
  const int nrb = a.d / kPfOut;
  const int u = pf_unit();
  const int li = u / nrb, rb = u % nrb;
  if (li >= a.info[3]) return;
  const int2 te = a.tiles64[li];
  const int cnt = a.act_cnt[te.x], slot = a.act_slot[te.x], q0 = a.act_off[te.x];
  const int t0 = te.y * kPfTile, mt = min(kPfTile, cnt - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, r = a.r, I = a.I, NC = I / 32, nsteps = I / 64, o0 = rb * kPfOut;
  const int o = 16 * RB * wave + n;  // this lane's output rows in the unit: o + 16 rr
  if (tid < kPfTile) {
    const int q = q0 + t0 + min(tid, mt - 1);
    src_s[tid] = a.pair_src[q];
    pw_s[tid] = a.pair_w[q];
  }
  __syncthreads();
  if (slot < 0) {
    for (int e = tid; e < mt * kPfOut; e += 256)
      a.ypair[(size_t)src_s[e / kPfOut] * d + o0 + e % kPfOut] = 0.f;
    return;
  }
  const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
  const uint16_t* hrow[HU];
  int hdst[HU], hhalf[HU];
#pragma unroll
  for (int q = 0; q < HU; ++q) {
    const int c = tid + 256 * q, half = c / (kPfTile * CPB), rem = c % (kPfTile * CPB);
    const int m = rem / CPB, cc = rem % CPB;
    hhalf[q] = half;
    hrow[q] = (half ? a.hp_lo : a.hp_hi) + (size_t)(q0 + t0 + min(m, mt - 1)) * I + 8 * cc;
    hdst[q] = m * CPB + (cc ^ (m % 8));
  }
  const int hsm = q0 + t0 + min(tid, mt - 1);  // group sums: thread < 64 (block-major sums)
  const int arr = tid / CPB, acc8 = tid % CPB; // A_down chunks: thread < 16 CPB
  const int e_lo = a.lora_sep ? a.act_e[te.x] : 0;  // the expert, for adapters given apart
  const uint16_t* adsrc = reinterpret_cast<const uint16_t*>(
      r > 0 ? grp_lora(a, b, e_lo, 4, a.lay.a_down) : b + a.lay.down_q) +
      (size_t)min(arr, max(r - 1, 0)) * I + 8 * acc8;
  // this lane's weight words: word j of row o0 + o + 16 rr in each 32-input
  // tile (64-row tile block (o0 + o) / 64, row (o0 + o) % 64 + 16 rr); its
  // rows' scales
  const uint32_t* dq = reinterpret_cast<const uint32_t*>(b + a.lay.down_q) +
                       (((size_t)((o0 + o) / 64) * NC) * 64 + (o0 + o) % 64) * 4 + j;
  const uint16_t* dsp = reinterpret_cast<const uint16_t*>(b + a.lay.down_s) + o0 + o;
  const uint16_t* dbp = reinterpret_cast<const uint16_t*>(b + a.lay.down_b) + o0 + o;
  // one step's loads, held in registers until the step before has been
  // multiplied (no arithmetic on them before then: it would wait for them)
  // (four separately named registers: as an array the compiler kept them
  // in scratch memory)
  static_assert(HU == 4, "four staged h chunks per thread");
  uint4 sh0, sh1, sh2, sh3, sad = make_uint4(0, 0, 0, 0);
  float shs[NGD][G / 16];
  uint32_t sw[RB][2], ssc[RB][NGD];  // weight words; the groups' scales s
#pragma unroll
  for (int gg = 0; gg < NGD; ++gg)
#pragma unroll
    for (int h2 = 0; h2 < G / 16; ++h2) shs[gg][h2] = 0.f;
  const uint16_t *hr0 = hrow[0], *hr1 = hrow[1], *hr2 = hrow[2], *hr3 = hrow[3];
  uint4* hd0 = &hh[0][hhalf[0]][hdst[0]];
  uint4* hd1 = &hh[0][hhalf[1]][hdst[1]];
  uint4* hd2 = &hh[0][hhalf[2]][hdst[2]];
  uint4* hd3 = &hh[0][hhalf[3]][hdst[3]];
  constexpr int kBufStride = 2 * kPfTile * CPB;  // uint4 per h buffer
#define E0_PF_DOWN_LOAD(S)                                                                  \
  {                                                                                         \
    const int s_ = (S);                                                                     \
    sh0 = *reinterpret_cast<const uint4*>(hr0 + 64 * s_);                                   \
    sh1 = *reinterpret_cast<const uint4*>(hr1 + 64 * s_);                                   \
    sh2 = *reinterpret_cast<const uint4*>(hr2 + 64 * s_);                                   \
    sh3 = *reinterpret_cast<const uint4*>(hr3 + 64 * s_);                                   \
    if (tid < kPfTile)                                                                      \
      _Pragma("unroll") for (int gg = 0; gg < NGD; ++gg)                                   \
          _Pragma("unroll") for (int h2 = 0; h2 < G / 16; ++h2) shs[gg][h2] =              \
              a.hs[(size_t)((s_ * 64 + gg * G) / 16 + h2) * a.P + hsm];                     \
    if (r > 0 && tid < kTileRank * CPB) sad = *reinterpret_cast<const uint4*>(adsrc + 64 * s_); \
    _Pragma("unroll") for (int rr = 0; rr < RB; ++rr) {                                    \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) sw[rr][ks] =                        \
          dq[(size_t)(2 * s_ + ks) * 64 * 4 + 16 * 4 * rr];                                 \
      _Pragma("unroll") for (int gg = 0; gg < NGD; ++gg)                                   \
          ssc[rr][gg] = dsp[(size_t)((s_ * 64) / G + gg) * d + 16 * rr];                    \
    }                                                                                       \
  }
#define E0_PF_DOWN_STORE(BUF, S)                                                            \
  {                                                                                         \
    const int b_ = (BUF);                                                                   \
    hd0[b_ * kBufStride] = sh0;                                                             \
    hd1[b_ * kBufStride] = sh1;                                                             \
    hd2[b_ * kBufStride] = sh2;                                                             \
    hd3[b_ * kBufStride] = sh3;                                                             \
    if (tid < kPfTile)                                                                      \
      _Pragma("unroll") for (int gg = 0; gg < NGD; ++gg) {                                 \
        float sum = 0.f;                                                                    \
        _Pragma("unroll") for (int h2 = 0; h2 < G / 16; ++h2) sum += shs[gg][h2];           \
        hsa[tid][(S) * NGD + gg] = sum;                                                     \
      }                                                                                     \
    if (r > 0 && tid < kTileRank * CPB) {                                                   \
      uint32_t w4[4];                                                                       \
      pair_perm8(sad.x, sad.y, sad.z, sad.w, w4);                                           \
      ad[b_][tid] = arr < r ? make_uint4(w4[0], w4[1], w4[2], w4[3]) : make_uint4(0, 0, 0, 0); \
    }                                                                                       \
  }
  E0_PF_DOWN_LOAD(0);
  E0_PF_DOWN_STORE(0, 0);
  __syncthreads();
  const Q4Consts kq = q4_consts();
  f32x4_t acc[4 * RB], tda = f32x4_t{0.f, 0.f, 0.f, 0.f};  // acc[4 rr + pb]
#pragma unroll
  for (int q = 0; q < 4 * RB; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    uint32_t cwv[RB][2], csc[RB][NGD];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) cwv[rr][ks] = sw[rr][ks];
#pragma unroll
      for (int gg = 0; gg < NGD; ++gg) csc[rr][gg] = ssc[rr][gg];
    }
    if (s + 1 < nsteps) E0_PF_DOWN_LOAD(s + 1);
#pragma unroll
    for (int gg = 0; gg < NGD; ++gg) {
      // the group's k-steps (32 inputs each), two row blocks at a time
#pragma unroll
      for (int half = 0; half < RB / 2; ++half) {
        f32x4_t tmp[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) tmp[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kg = 0; kg < KS; ++kg) {
          const int ks = gg * KS + kg, c = 4 * ks + j;
          const bf16x8_t w0 = q4_operand_k(cwv[2 * half][ks], kq);
          const bf16x8_t w1 = q4_operand_k(cwv[2 * half + 1][ks], kq);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) {
            const int m = 16 * pb + n, sw = m * CPB + (c ^ (m % 8));
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, hh[buf][0][sw]);
            const bf16x8_t al = __builtin_bit_cast(bf16x8_t, hh[buf][1][sw]);
            tmp[pb] = mfma16(ah, w0, tmp[pb]);
            tmp[pb] = mfma16(al, w0, tmp[pb]);
            tmp[4 + pb] = mfma16(ah, w1, tmp[4 + pb]);
            tmp[4 + pb] = mfma16(al, w1, tmp[4 + pb]);
            if (half == 0 && pb == wave && r > 0) {
              const bf16x8_t ao = __builtin_bit_cast(bf16x8_t, ad[buf][n * CPB + c]);
              tda = mfma16(ah, ao, tda);
              tda = mfma16(al, ao, tda);
            }
          }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int rr = 2 * half + h2;
          const float sd = bf2f(csc[rr][gg]);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[4 * rr + pb][v] = fmaf(sd, tmp[4 * h2 + pb][v], acc[4 * rr + pb][v]);
        }
      }
    }
    if (s + 1 < nsteps) E0_PF_DOWN_STORE(buf ^ 1, s + 1);
    __syncthreads();
  }
#undef E0_PF_DOWN_LOAD
#undef E0_PF_DOWN_STORE
  // the groups' (b - 128 s) terms, as in the gate/up kernel: A = the pairs'
  // h sums per group (from LDS), B = b - 128 s of the wave's rows, both
  // split three ways (groups past I / g count as zeros)
  {
    const int ngi = I / G;
    bf16x8_t hs3[4][3];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      float h8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h8[e] = 8 * j + e < ngi ? hsa[16 * pb + n][8 * j + e] : 0.f;
      split3_8(F8{make_float4(h8[0], h8[1], h8[2], h8[3]), make_float4(h8[4], h8[5], h8[6], h8[7])},
               hs3[pb][0], hs3[pb][1], hs3[pb][2]);
    }
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      float c8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int gi = min(8 * j + e, ngi - 1);
        const float sd = bf2f(dsp[(size_t)gi * d + 16 * rr]), bd = bf2f(dbp[(size_t)gi * d + 16 * rr]);
        c8[e] = 8 * j + e < ngi ? bd - 128.f * sd : 0.f;
      }
      bf16x8_t cs3[3];
      split3_8(F8{make_float4(c8[0], c8[1], c8[2], c8[3]), make_float4(c8[4], c8[5], c8[6], c8[7])},
               cs3[0], cs3[1], cs3[2]);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) acc[4 * rr + pb] = mfma16_x3(hs3[pb], cs3, acc[4 * rr + pb]);
    }
  }
  // LoRA-down: A = A_down h of the pairs (hi + lo), B = B_down rows
  if (r > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) td_s[16 * wave + 4 * j + v][n] = tda[v];
    __syncthreads();
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      bf16x8_t th, tl;
      const float* tdr = &td_s[16 * pb + n][8 * (j & 1)];
      split_hilo8(F8{*reinterpret_cast<const float4*>(tdr), *reinterpret_cast<const float4*>(tdr + 4)},
                  j < 2, th, tl);
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const uint16_t* B =
            reinterpret_cast<const uint16_t*>(grp_lora(a, b, e_lo, 5, a.lay.b_down)) +
            (size_t)(o0 + o + 16 * rr) * r;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 8 * j + 2 * e;
          const uint32_t lo16 = (j < 2 && k < r) ? B[k] : 0u;
          const uint32_t hi16 = (j < 2 && k + 1 < r) ? B[k + 1] : 0u;
          w4[e] = lo16 | (hi16 << 16);
        }
        const bf16x8_t bd = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
        f32x4_t lt = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lt = mfma16(th, bd, lt);
        lt = mfma16(tl, bd, lt);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[4 * rr + pb][v] += a.scale * lt[v];
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RB; ++rr)
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * pb + 4 * j + v;
        if (m < mt)
          a.ypair[(size_t)src_s[m] * d + o0 + o + 16 * rr] = pw_s[m] * acc[4 * rr + pb][v];
      }
}

// y of each token: its kept pairs' rows added in k order, rounded once
__global__ __launch_bounds__(256) void k_pf_combine(GrpArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // 4 outputs each
  const int d4 = a.d / 4;
  if (i >= a.T * d4) return;
  const int t = i / d4, o = 4 * (i % d4);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < a.K; ++k) {
    const int p = t * a.K + k;
    if (a.keep[p] < 0) continue;
    const float4 v = *reinterpret_cast<const float4*>(a.ypair + (size_t)p * a.d + o);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<uint2*>(a.y + (size_t)t * a.d + o) =
      make_uint2(f2bf(s.x) | (f2bf(s.y) << 16), f2bf(s.z) | (f2bf(s.w) << 16));
}

// ------------------------------------------------------------- host side
struct GrpWs {
  size_t err, info, act_e, act_off, act_cnt, act_slot, pair_tok, pair_src, pair_w, t_in, hp_hi,
      hp_lo, hs, tdown, acc, total;
};
static GrpWs grp_ws_layout(const edge0_moe_shape* s) {
  GrpWs L{};
  const size_t T = kGrpMaxTokens, d = s->d_model, E = s->n_experts, I = s->d_inter;
  const size_t P = T * s->top_k, r = s->lora_rank;
  const size_t A = E < P ? E : P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + (bytes ? bytes : 4) + 255) & ~(size_t)255;
    return o;
  };
  L.err = take(4);
  L.info = take(16);
  L.act_e = take(4 * A);
  L.act_off = take(4 * A);
  L.act_cnt = take(4 * A);
  L.act_slot = take(4 * A);
  L.pair_tok = take(4 * P);
  L.pair_src = take(4 * P);
  L.pair_w = take(4 * P);
  L.t_in = take(4 * P * 2 * r);
  L.hp_hi = take(2 * P * I);
  L.hp_lo = take(2 * P * I);
  L.hs = take(4 * P * (I / 16));
  L.tdown = take(8 * P * r);
  L.acc = take(8 * T * d);
  L.total = off;
  return L;
}

// The adapters of a call: in the bundles (lora NULL), or given apart, when
// the pool may hold LoRA-free bundles (the int4 arrays sit at the same
// offsets in both layouts).  Checks the pool's slot size against the layout
// it must hold.
static int grp_lora_args(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                         const edge0_lora* lora, GrpArgs& a) {
  edge0_bundle_layout lay, lay_pool;
  edge0_moe_shape s0 = *shape;
  const int r = shape->lora_rank;
  const bool sep = lora != nullptr && r > 0;
  if (sep) s0.lora_rank = 0;
  if (bundle_layout(shape, &lay) != EDGE0_OK || bundle_layout(&s0, &lay_pool) != EDGE0_OK ||
      pool->slot_bytes < lay_pool.bytes)
    return EDGE0_EINVAL;
  if (sep && (!lora->a_gate || !lora->b_gate || !lora->a_up || !lora->b_up || !lora->a_down ||
              !lora->b_down || lora->expert_stride < 0))
    return EDGE0_EINVAL;
  a.lay = lay;
  a.lora_sep = sep;
  if (sep) {
    const void* f[6] = {lora->a_gate, lora->b_gate, lora->a_up, lora->b_up, lora->a_down, lora->b_down};
    for (int i = 0; i < 6; ++i) a.lo_base[i] = static_cast<const uint8_t*>(f[i]);
    a.lo_stride = lora->expert_stride * 2;  // bf16 elements
  }
  return EDGE0_OK;
}

static bool grouped_shape_ok(const edge0_moe_shape* s) {
  const int g = s->group_size;
  return shape_ok(s) && s->d_inter / 32 <= kGrpMaxNC && s->d_model <= 4096 &&
         (g == 32 || g == 64 || g == 128);
}

// tokens per GEMV workgroup; ceil(T / kGrpSliceTokens) slices per expert
constexpr int kGrpSliceTokens = 8;
static int grp_slices(const GrpArgs& a) {
  return (a.T + kGrpSliceTokens - 1) / kGrpSliceTokens;
}

static int launch_grp_gate_up(const GrpArgs& a, int lo, int hi, hipStream_t st) {
  const int grid = grp_slices(a) * a.Amax * (a.I / 16), ts = kGrpSliceTokens;
  switch ((a.d / 32 + 63) / 64) {
    case 1:
      if (a.d == 2048) k_grp_gate_up<1, true><<<grid, 256, 0, st>>>(a, lo, hi, ts);
      else k_grp_gate_up<1, false><<<grid, 256, 0, st>>>(a, lo, hi, ts);
      break;
    case 2:
      if (a.d == 4096) k_grp_gate_up<2, true><<<grid, 256, 0, st>>>(a, lo, hi, ts);
      else k_grp_gate_up<2, false><<<grid, 256, 0, st>>>(a, lo, hi, ts);
      break;
    default: return EDGE0_EINVAL;
  }
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

static int launch_grp_down(const GrpArgs& a, int lo, int hi, hipStream_t st) {
  const int grid = grp_slices(a) * a.Amax * (a.d / 64), ts = kGrpSliceTokens;
  switch ((a.I / 32 + 3) / 4) {
    case 1: k_grp_down<1><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 2: k_grp_down<2><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 3: k_grp_down<3><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 4: k_grp_down<4><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 5: k_grp_down<5><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 6: k_grp_down<6><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 7: k_grp_down<7><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 8: k_grp_down<8><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    default: return EDGE0_EINVAL;
  }
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

// shapes of the token-tile kernels: d <= 2048, each wave quarter of d an
// even number of groups of 32 or 64, I / 32 one of the down-tile instances
// (4, 8, 12, 16, 24, 32: I up to 1024, so a tile's h fits 64 KiB of LDS),
// LoRA rank even and <= 16.  Every shape accepted here has an instance of
// both tile kernels, so a call never fails after its first launch; other
// shapes run as GEMVs.
static bool grp_tile_ok(const GrpArgs& a) {
  const int gw = a.d / (4 * a.g), nw = a.I / 32;
  return (a.g == 32 || a.g == 64) && a.d <= 2048 && a.d % (8 * a.g) == 0 &&
         (gw == 2 || gw == 4 || gw == 8 || gw == 16) && a.I % 32 == 0 &&
         (nw == 4 || nw == 8 || nw == 12 || nw == 16 || nw == 24 || nw == 32) &&
         a.r <= kTileRank && a.r % 2 == 0;
}

// experts with >= min_cnt tokens
// units = (tile, expert) units of the grid: ceil(T / tm) * Amax for the
// grouped call, the tile list's bound for prefill
static int launch_grp_tiles_gu(const GrpArgs& a, int min_cnt, int tm, int units, hipStream_t st) {
  const int wpg = a.g / 32, gw = a.d / (4 * a.g);
  const int grid_gu = units * (a.I / 16);
#define E0_GU(GW, W) \
  if (gw == GW && wpg == W) k_grp_gu_tile<GW, W><<<grid_gu, 256, 0, st>>>(a, tm, min_cnt)
  bool ok = true;
  E0_GU(2, 1); else E0_GU(4, 1); else E0_GU(8, 1); else E0_GU(16, 1);
  else E0_GU(2, 2); else E0_GU(4, 2); else E0_GU(8, 2); else E0_GU(16, 2);
  else ok = false;
#undef E0_GU
  if (!ok) return EDGE0_EINVAL;
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
static int launch_grp_tiles_down(const GrpArgs& a, int min_cnt, int tm, int units, hipStream_t st) {
  const int wpg = a.g / 32, nw = a.I / 32;
  const size_t lds_dn = (size_t)2 * tm * a.I * 2;
  const int grid_dn = units * (a.d / (64 * kDownNT));
  bool ok = true;
#define E0_DN(NW, W) \
  if (nw == NW && wpg == W) k_grp_down_tile<NW, W><<<grid_dn, 256, lds_dn, st>>>(a, tm, min_cnt)
  E0_DN(4, 1); else E0_DN(8, 1); else E0_DN(12, 1); else E0_DN(16, 1); else E0_DN(24, 1);
  else E0_DN(32, 1);
  else E0_DN(4, 2); else E0_DN(8, 2); else E0_DN(12, 2); else E0_DN(16, 2); else E0_DN(24, 2);
  else E0_DN(32, 2);
  else ok = false;
#undef E0_DN
  if (!ok) return EDGE0_EINVAL;
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

}  // namespace e0

using namespace e0;

extern "C" size_t edge0_grouped_workspace_bytes(const edge0_moe_shape* shape) {
  if (!grouped_shape_ok(shape)) return 0;
  return grp_ws_layout(shape).total;
}

static int grouped_call(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                        const edge0_lora* lora, const int32_t* slot_table, int32_t n_tokens,
                        const int32_t* ids, const float* w, const void* x, void* y,
                        void* workspace, int32_t flags, hipStream_t stream) {
  if (!shape || !grouped_shape_ok(shape) || !pool || !pool->base || !slot_table || !workspace ||
      n_tokens < 0 || n_tokens > kGrpMaxTokens || (flags & ~(EDGE0_GROUPED_NO_MFMA | 0xFF00)) != 0)
    return EDGE0_EINVAL;
  GrpArgs a{};
  if (grp_lora_args(shape, pool, lora, a) != EDGE0_OK) return EDGE0_EINVAL;
  if (n_tokens == 0) return EDGE0_OK;
  if (!ids || !w || !x || !y) return EDGE0_EINVAL;
  const GrpWs L = grp_ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  a.pool = static_cast<const uint8_t*>(pool->base);
  a.slot_bytes = pool->slot_bytes;
  a.n_slots = pool->n_slots;
  a.table = slot_table;
  a.ids = ids;
  a.w = w;
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.T = n_tokens;
  a.d = shape->d_model;
  a.E = shape->n_experts;
  a.I = shape->d_inter;
  a.K = shape->top_k;
  a.g = shape->group_size;
  a.r = shape->lora_rank;
  a.scale = a.r > 0 ? shape->lora_alpha / (float)a.r : 0.f;
  a.P = n_tokens * a.K;
  a.Amax = a.E < a.P ? a.E : a.P;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.info = reinterpret_cast<int32_t*>(ws + L.info);
  a.act_e = reinterpret_cast<int32_t*>(ws + L.act_e);
  a.act_off = reinterpret_cast<int32_t*>(ws + L.act_off);
  a.act_cnt = reinterpret_cast<int32_t*>(ws + L.act_cnt);
  a.act_slot = reinterpret_cast<int32_t*>(ws + L.act_slot);
  a.pair_tok = reinterpret_cast<int32_t*>(ws + L.pair_tok);
  a.pair_src = reinterpret_cast<int32_t*>(ws + L.pair_src);
  a.pair_w = reinterpret_cast<float*>(ws + L.pair_w);
  a.t_in = reinterpret_cast<float*>(ws + L.t_in);
  a.hp_hi = reinterpret_cast<uint16_t*>(ws + L.hp_hi);
  a.hp_lo = reinterpret_cast<uint16_t*>(ws + L.hp_lo);
  a.hs = reinterpret_cast<float*>(ws + L.hs);
  a.tdown = reinterpret_cast<unsigned long long*>(ws + L.tdown);
  a.acc = reinterpret_cast<unsigned long long*>(ws + L.acc);
  k_grp_route_lora<<<1 + (a.r > 0 ? (a.P * 2 * a.r + 15) / 16 : 0), 1024, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  // experts with >= tile_min tokens on the MFMA token tiles, the others as
  // GEMVs.  Default: every expert on the tiles from kTileMinCall tokens per
  // call on (below that the GEMVs' shorter chains win).  An expert holds at
  // most n_tokens pairs, so tile_min > n_tokens means no tiles.
  int tile_min = 0;
  if (!(flags & EDGE0_GROUPED_NO_MFMA) && grp_tile_ok(a)) {
    const int fm = (flags >> 8) & 0xFF;
    tile_min = fm ? fm : (n_tokens >= kTileMinCall ? 1 : 0);
    if (tile_min > n_tokens) tile_min = 0;
  }
  const int gemv_max = tile_min ? tile_min - 1 : 1 << 30;
  const int tm = a.T < kTileTok ? a.T : kTileTok;
  const int units = (a.T + tm - 1) / tm * a.Amax;
  int rc = gemv_max >= 1 ? launch_grp_gate_up(a, 1, gemv_max, stream) : EDGE0_OK;
  if (rc == EDGE0_OK && tile_min) rc = launch_grp_tiles_gu(a, tile_min, tm, units, stream);
  if (rc == EDGE0_OK && gemv_max >= 1) rc = launch_grp_down(a, 1, gemv_max, stream);
  if (rc == EDGE0_OK && tile_min) rc = launch_grp_tiles_down(a, tile_min, tm, units, stream);
  if (rc != EDGE0_OK) return rc;
  const int n_out = a.T * a.d;
  k_grp_out<<<(n_out + 255) / 256, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

extern "C" int edge0_moe_grouped(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                 const int32_t* slot_table, int32_t n_tokens, const int32_t* ids,
                                 const float* w, const void* x, void* y, void* workspace,
                                 int32_t flags, hipStream_t stream) {
  return grouped_call(shape, pool, nullptr, slot_table, n_tokens, ids, w, x, y, workspace, flags,
                      stream);
}

extern "C" int edge0_moe_grouped_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                      const edge0_lora* lora, const int32_t* slot_table,
                                      int32_t n_tokens, const int32_t* ids, const float* w,
                                      const void* x, void* y, void* workspace, int32_t flags,
                                      hipStream_t stream) {
  if (shape && shape->lora_rank > 0 && !lora) return EDGE0_EINVAL;
  return grouped_call(shape, pool, lora, slot_table, n_tokens, ids, w, x, y, workspace, flags,
                      stream);
}

// ------------------------------------------------------------ prefill host
namespace e0 {
struct PfWs {
  size_t err, info, cnt, fill, keep, keep_w, tiles64, act_e, act_off, act_cnt, act_slot,
      pair_tok, pair_src, pair_w, t_in, hp_hi, hp_lo, hs, xsum, ypair, total;
};
// an upper bound of the tile list: sum over experts of ceil(count / 64)
static int pf_tiles64_max(int P, int E) { return (P + kPfTile - 1) / kPfTile + (E < P ? E : P); }
static PfWs pf_ws_layout(const edge0_moe_shape* s, int max_tokens) {
  PfWs L{};
  const size_t T = max_tokens, d = s->d_model, E = s->n_experts, I = s->d_inter;
  const size_t P = T * s->top_k, r = s->lora_rank;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + (bytes ? bytes : 4) + 255) & ~(size_t)255;
    return o;
  };
  L.err = take(4);
  L.info = take(16);
  L.cnt = take(4 * E);
  L.fill = take(4 * E);
  L.keep = take(4 * P);
  L.keep_w = take(4 * P);
  L.tiles64 = take(8 * (size_t)pf_tiles64_max((int)P, (int)E));
  L.act_e = take(4 * E);
  L.act_off = take(4 * E);
  L.act_cnt = take(4 * E);
  L.act_slot = take(4 * E);
  L.pair_tok = take(4 * P);
  L.pair_src = take(4 * P);
  L.pair_w = take(4 * P);
  L.t_in = take(4 * P * 2 * r);
  L.hp_hi = take(2 * P * I);
  L.hp_lo = take(2 * P * I);
  L.hs = take(4 * P * (I / 16));
  L.xsum = take(4 * T * (d / s->group_size));
  L.ypair = take(4 * P * d);
  L.total = off;
  return L;
}
// the prefill kernels' shapes: the LoRA A x tiles (d / 4 a multiple of 32),
// the gate/up units (64 rows) and the down units (128 output rows) over
// whole groups of 32 or 64 inputs, the down kernel's groups held in LDS
static bool pf_shape_ok(const edge0_moe_shape* s) {
  if (!grouped_shape_ok(s)) return false;
  const int d = s->d_model, g = s->group_size, I = s->d_inter, r = s->lora_rank;
  return (g == 32 || g == 64) && d <= 2048 && d % 128 == 0 && d % pf_out(g / 32) == 0 &&
         I % kPfRows == 0 && I % 64 == 0 && I / g < kPfGroupsPad && r <= kTileRank;
}
}  // namespace e0

extern "C" size_t edge0_prefill_workspace_bytes(const edge0_moe_shape* shape, int32_t max_tokens) {
  if (!shape || !pf_shape_ok(shape) || max_tokens < 1 || max_tokens > kPfMaxTokens) return 0;
  return pf_ws_layout(shape, max_tokens).total;
}

static int prefill_call(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                        const edge0_lora* lora, const int32_t* slot_table, int32_t n_tokens,
                        const int32_t* ids, const float* w, const void* x, void* y,
                        void* workspace, int32_t max_tokens, hipStream_t stream) {
  if (!shape || !pf_shape_ok(shape) || !pool || !pool->base || !slot_table || !workspace ||
      max_tokens < 1 || max_tokens > kPfMaxTokens || n_tokens < 0 || n_tokens > max_tokens)
    return EDGE0_EINVAL;
  GrpArgs a{};
  if (grp_lora_args(shape, pool, lora, a) != EDGE0_OK) return EDGE0_EINVAL;
  if (n_tokens == 0) return EDGE0_OK;
  if (!ids || !w || !x || !y || x == y) return EDGE0_EINVAL;
  const PfWs L = pf_ws_layout(shape, max_tokens);
  char* ws = static_cast<char*>(workspace);
  a.pool = static_cast<const uint8_t*>(pool->base);
  a.slot_bytes = pool->slot_bytes;
  a.n_slots = pool->n_slots;
  a.table = slot_table;
  a.ids = ids;
  a.w = w;
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.T = n_tokens;
  a.d = shape->d_model;
  a.E = shape->n_experts;
  a.I = shape->d_inter;
  a.K = shape->top_k;
  a.g = shape->group_size;
  a.r = shape->lora_rank;
  a.scale = a.r > 0 ? shape->lora_alpha / (float)a.r : 0.f;
  a.P = n_tokens * a.K;
  a.Amax = a.E < a.P ? a.E : a.P;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.info = reinterpret_cast<int32_t*>(ws + L.info);
  a.act_e = reinterpret_cast<int32_t*>(ws + L.act_e);
  a.act_off = reinterpret_cast<int32_t*>(ws + L.act_off);
  a.act_cnt = reinterpret_cast<int32_t*>(ws + L.act_cnt);
  a.act_slot = reinterpret_cast<int32_t*>(ws + L.act_slot);
  a.pair_tok = reinterpret_cast<int32_t*>(ws + L.pair_tok);
  a.pair_src = reinterpret_cast<int32_t*>(ws + L.pair_src);
  a.pair_w = reinterpret_cast<float*>(ws + L.pair_w);
  a.t_in = reinterpret_cast<float*>(ws + L.t_in);
  a.hp_hi = reinterpret_cast<uint16_t*>(ws + L.hp_hi);
  a.hp_lo = reinterpret_cast<uint16_t*>(ws + L.hp_lo);
  a.hs = reinterpret_cast<float*>(ws + L.hs);
  a.tiles64 = reinterpret_cast<const int2*>(ws + L.tiles64);
  a.xsum = reinterpret_cast<const float*>(ws + L.xsum);
  a.ypair = reinterpret_cast<float*>(ws + L.ypair);
  a.keep = reinterpret_cast<const int32_t*>(ws + L.keep);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* fill = reinterpret_cast<int32_t*>(ws + L.fill);
  int32_t* keep = reinterpret_cast<int32_t*>(ws + L.keep);
  float* keep_w = reinterpret_cast<float*>(ws + L.keep_w);
  int2* tiles64 = reinterpret_cast<int2*>(ws + L.tiles64);
  const int pg = (a.P + kPfPairsPerWg - 1) / kPfPairsPerWg;
  k_pf_count<<<pg, 1024, 0, stream>>>(a, cnt, keep, keep_w);
  E0_CHECK_LAUNCH();
  k_pf_scan<<<1, 1024, 0, stream>>>(a, cnt, fill, tiles64);
  E0_CHECK_LAUNCH();
  k_pf_scatter<<<pg, 1024, 0, stream>>>(a, keep, keep_w, fill);
  E0_CHECK_LAUNCH();
  const int nxs = a.T * (a.d / a.g);
  k_pf_xsum<<<(nxs + 255) / 256, 256, 0, stream>>>(a, reinterpret_cast<float*>(ws + L.xsum));
  E0_CHECK_LAUNCH();
  if (a.r > 0) {
    k_pf_lora_in<<<pf_tiles64_max(a.P, a.E), 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
  }
  // the GEMM units: every (64-pair tile, row block), the grid a multiple of
  // 8 for the XCD-aware order (units past the tile list return)
  const int tiles_max = pf_tiles64_max(a.P, a.E);
  const int g_gu = (tiles_max * (a.I / kPfRows) + 7) / 8 * 8;
  const int g_dn = (tiles_max * (a.d / pf_out(a.g / 32)) + 7) / 8 * 8;
  if (a.g == 64) {
    k_pf_gu<2><<<g_gu, 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
    k_pf_down<2><<<g_dn, 256, 0, stream>>>(a);
  } else {
    k_pf_gu<1><<<g_gu, 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
    k_pf_down<1><<<g_dn, 256, 0, stream>>>(a);
  }
  E0_CHECK_LAUNCH();
  k_pf_combine<<<(a.T * (a.d / 4) + 255) / 256, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

extern "C" int edge0_moe_prefill(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                 const int32_t* slot_table, int32_t n_tokens, const int32_t* ids,
                                 const float* w, const void* x, void* y, void* workspace,
                                 int32_t max_tokens, hipStream_t stream) {
  return prefill_call(shape, pool, nullptr, slot_table, n_tokens, ids, w, x, y, workspace,
                      max_tokens, stream);
}

extern "C" int edge0_moe_prefill_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                      const edge0_lora* lora, const int32_t* slot_table,
                                      int32_t n_tokens, const int32_t* ids, const float* w,
                                      const void* x, void* y, void* workspace, int32_t max_tokens,
                                      hipStream_t stream) {
  if (shape && shape->lora_rank > 0 && !lora) return EDGE0_EINVAL;
  return prefill_call(shape, pool, lora, slot_table, n_tokens, ids, w, x, y, workspace,
                      max_tokens, stream);
}
