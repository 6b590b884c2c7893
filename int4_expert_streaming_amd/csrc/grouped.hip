// Several tokens through one MoE layer, grouped by expert: every routed
// expert's weights are read once per call however many tokens chose it.
//
// The result is defined token by token, exactly as the single-token layer
// ([Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction", §3.1 "Math contract", §3.3 unmerged
// LoRA, Figure 1 sum node); the grouping only reorders the work.
//
// Launches (all on the caller's stream):
//   k_grp_route   : one workgroup buckets the T*K (token, k) pairs by expert
//                   (counting sort, stable in pair order, so by token), lists
//                   the active experts with their first pair and count, and
//                   resolves each active expert's slot once.
//   k_grp_lora_in : t = A x for every pair's gate and up adapters.
//   k_grp_gate_up : one workgroup = 16 rows of one active expert's gate and
//                   up; the rows stay in registers while the expert's tokens
//                   stream through LDS in batches; SwiGLU; h stored as bf16
//                   hi/lo pairs, per-16-row sums, and A_down h accumulated in
//                   fixed point per pair.
//   k_grp_gate_up_mfma : the same for experts with >= 16 tokens, on MFMA.
//   k_grp_down    : one workgroup = 64 output rows of one active expert; the
//                   tiled down weights stay in registers while the tokens' h
//                   batches stream through LDS; the LoRA-down delta; each
//                   token's weighted row added to its fixed-point output.
//   k_grp_down_mfma : the same for experts with >= 16 tokens, on MFMA.
//   k_grp_out     : y = bf16 of each token's accumulator; clears the
//                   accumulators for the next call.
// Int4 arithmetic is the single-token path's: exact bf16 "128 + q" nibble
// pairs against pair-permuted activations, the group affine folded per
// 32-input chunk, fp32 everywhere, one bf16 rounding of y.
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
  int32_t* pair_act;  // [P] active expert of each sorted pair
  float* pair_w;      // [P] routing weight of each sorted pair
  float* t_in;        // [P][2][r]
  uint16_t* hp_hi;    // [P][I] pair-permuted
  uint16_t* hp_lo;
  float* hs;                   // [P][I/16]
  unsigned long long* tdown;   // [P][r] A_down h, fixed point
  unsigned long long* acc;     // [T][d] y, fixed point
};

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
// number of earlier pairs of the same expert (stable).
__global__ __launch_bounds__(1024) void k_grp_route(GrpArgs a) {
  __shared__ int cnt[1024];
  __shared__ int first[1024];
  __shared__ int actidx[1024];
  __shared__ int ids_s[kGrpMaxTokens * 16];
  __shared__ int wtot[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.P;
  cnt[tid] = 0;
  for (int p = tid; p < P; p += 1024) {
    int e = a.ids[p];
    if (e < 0 || e >= E) {
      set_error(a.err, EDGE0_ERANGE);
      e = -1;
    }
    ids_s[p] = e;
  }
  __syncthreads();
  for (int p = tid; p < P; p += 1024)
    if (ids_s[p] >= 0) atomicAdd(&cnt[ids_s[p]], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int f = c > 0 ? 1 : 0;
  const int ic = wave_incl_scan(c), iff = wave_incl_scan(f);
  if (lane == 63) {
    wtot[0][wave] = ic;
    wtot[1][wave] = iff;
  }
  __syncthreads();
  int bc = 0, bf = 0, tc = 0, tf = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) {
      bc += wtot[0][w];
      bf += wtot[1][w];
    }
    tc += wtot[0][w];
    tf += wtot[1][w];
  }
  const int xc = bc + ic - c, xf = bf + iff - f;  // exclusive prefixes
  if (tid < E) {
    first[tid] = xc;
    actidx[tid] = xf;
    if (f) {
      a.act_e[xf] = tid;
      a.act_off[xf] = xc;
      a.act_cnt[xf] = c;
      const int s = a.table[tid];
      const bool ok = s >= 0 && s < a.n_slots;
      a.act_slot[xf] = ok ? s : -1;
      if (!ok) set_error(a.err, EDGE0_ERANGE);
    }
  }
  if (tid == 0) {
    a.info[0] = tf;
    a.info[1] = tc;
  }
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = ids_s[p];
    if (e < 0) continue;
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += ids_s[q] == e;
    const int dst = first[e] + rank;
    a.pair_tok[dst] = p / a.K;
    a.pair_act[dst] = actidx[e];
    a.pair_w[dst] = a.w[p];
  }
}

__device__ __forceinline__ const uint8_t* grp_bundle(const GrpArgs& a, int act) {
  const int s = a.act_slot[act];
  return s < 0 ? nullptr : a.pool + (size_t)s * (size_t)a.slot_bytes;
}

// ------------------------------------------------------------ LoRA A x
// one wave per row (sorted pair q, projection p, rank row rr)
__global__ __launch_bounds__(256) void k_grp_lora_in(GrpArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = a.r;
  const int q = row / (2 * r), p = (row / r) & 1, rr = row % r;
  if (q >= a.info[1]) return;
  const uint8_t* b = grp_bundle(a, a.pair_act[q]);
  float t = 0.f;
  if (b != nullptr) {
    const uint16_t* wrow =
        reinterpret_cast<const uint16_t*>(b + (p ? a.lay.a_up : a.lay.a_gate)) + (size_t)rr * a.d;
    t = row_dot<false, false>(wrow, a.x + (size_t)a.pair_tok[q] * a.d, a.d);
  }
  if ((threadIdx.x & 63) == 0) a.t_in[row] = t;
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
template <int NJ>
__global__ __launch_bounds__(256) void k_grp_gate_up(GrpArgs a, int min_cnt, int max_cnt,
                                                     int ts) {
  __shared__ uint16_t xs[kGrpXBytes / 2];
  __shared__ float h_s[16];
  __shared__ float hrep_s[16];
  const int nblk = a.I / 16;
  const int sl = blockIdx.x / (a.Amax * nblk);
  const int act = (blockIdx.x / nblk) % a.Amax;
  const int blk = blockIdx.x % nblk;
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt || n > max_cnt) return;
  // the last slice also takes any tokens beyond the slices (only an id that
  // repeats within one token's routing can give an expert more than T pairs)
  const bool last = sl == (int)gridDim.x / (a.Amax * nblk) - 1;
  const int t_lo = sl * ts, t_hi = last ? n : min(n, t_lo + ts);
  if (t_lo >= n) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
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
      const bool on = col < cpr;
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
  float Bg[4] = {0.f, 0.f, 0.f, 0.f}, Bu[4] = {0.f, 0.f, 0.f, 0.f};
  if (has_l) {
    const uint16_t* Bgp = reinterpret_cast<const uint16_t*>(b + a.lay.b_gate);
    const uint16_t* Bup = reinterpret_cast<const uint16_t*>(b + a.lay.b_up);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      Bg[ii] = bf2f(Bgp[(size_t)(row0 + ii) * r + lane]);
      Bu[ii] = bf2f(Bup[(size_t)(row0 + ii) * r + lane]);
    }
  }
  uint4 ad0 = make_uint4(0, 0, 0, 0), ad1 = ad0;
  if ((int)threadIdx.x < r) {
    const uint4* src = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(b + a.lay.a_down) + (size_t)threadIdx.x * a.I + i0);
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
        if (col < cpr) {
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
        tg = a.t_in[((size_t)q * 2 + 0) * r + lane];
        tu = a.t_in[((size_t)q * 2 + 1) * r + lane];
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
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt || n > max_cnt) return;
  const bool last = sl == (int)gridDim.x / (a.Amax * nrb) - 1;
  const int t_lo = sl * ts, t_hi = last ? n : min(n, t_lo + ts);
  if (t_lo >= n) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
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
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(b + a.lay.b_down) + (size_t)o * (r / 2);
#pragma unroll
    for (int m = 0; m < 32; ++m) bd[m] = 2 * m < r ? src[m] : 0u;
  }
  for (int j0 = t_lo; j0 < t_hi; j0 += kGrpBT) {
    const int nb = t_hi - j0 < kGrpBT ? t_hi - j0 : kGrpBT;
    __syncthreads();  // previous batch consumed
    for (int t = threadIdx.x; t < nb * NC * 32; t += 256) {
      const int jj = t / (NC * 32), rem = t % (NC * 32);
      const int c = rem >> 5, wd = rem & 31;
      const int q = q0 + j0 + jj;
      const uint32_t* src =
          reinterpret_cast<const uint32_t*>(wd < 16 ? a.hp_hi : a.hp_lo) + (size_t)q * (I / 2);
      hp_s[jj][c][wd] = src[16 * c + (wd & 15)];
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

// ------------------------------------------------------------ MFMA paths
// v_mfma_f32_32x32x16_bf16 (lane l: A[l%32][8(l/32)+i], B[8(l/32)+i][l%32],
// accumulator 4J+i = C[8J + 4(l/32) + i][l%32]).  A = activations (rows =
// tokens of the expert, padded to 32), B = weights (columns = 32 weight
// rows), so a lane's 16 accumulators share one weight row and one scale and
// bias per group.  Per group the products start from zero and are folded in
// fp32: s * acc + (b - 128 s) * (sum of the group's activations).  Within a
// group lane half j takes SPG = g/16 consecutive packed words (8 inputs
// each); step t of the group feeds word j*SPG + t, as exact bf16 128 + q in
// the pair order (e0,e4,e1,e5,e2,e6,e3,e7), against activations in the same
// order (pair_perm8, or the pair-permuted h pairs).  The 4 waves split the
// groups; partial tiles meet in LDS.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ bf16x8_t q4_operand(uint32_t word) {
  const uint4 v = make_uint4(q4pair(word, 0), q4pair(word, 1), q4pair(word, 2), q4pair(word, 3));
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t x_operand(uint4 raw) {
  uint32_t o[4];
  pair_perm8(raw.x, raw.y, raw.z, raw.w, o);
  return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}
__device__ __forceinline__ float raw_sum8(uint4 v) {
  return bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) +
         bf_lo(v.w) + bf_hi(v.w);
}
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// SPG consecutive packed words starting at p (4-byte aligned; 16-byte
// aligned when SPG >= 4)
template <int SPG>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[SPG]) {
  if constexpr (SPG % 4 == 0) {
#pragma unroll
    for (int m = 0; m < SPG / 4; ++m) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[m];
      w[4 * m] = v.x;
      w[4 * m + 1] = v.y;
      w[4 * m + 2] = v.z;
      w[4 * m + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < SPG; ++m) w[m] = p[m];
  }
}

constexpr int kFusedRank = 16;  // LoRA rank bound of the pipelined MFMA kernels
constexpr int kGW = 8;  // groups per wave per pass (their weights held in registers)

// One workgroup = 32 rows of one active expert's gate and up, all its tokens
// in tiles of 32.
template <int SPG>
__global__ __launch_bounds__(256) void k_grp_gate_up_mfma(GrpArgs a, int min_cnt) {
  __shared__ float red[4][2][32][33];  // per wave: [G or U][weight row][token]
  __shared__ float hbuf[32][33];       // h [token][row]
  __shared__ float hrep_s[32][33];     // the value the down product sees (hi + lo)
  __shared__ float tl_s[32][2][64];    // LoRA t of the tile's tokens
  __shared__ float bl_s[2][32][64];    // B_gate / B_up rows of the block
  __shared__ float ad_s[64][32];       // A_down columns of the block
  const int nb32 = a.I / 32;
  const int act = blockIdx.x / nb32;
  const int rb = blockIdx.x % nb32;
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 31, jh = lane >> 5;
  const int d = a.d, g = a.g, ng = d / g, r = a.r, I = a.I;
  const int row0 = rb * 32, row = row0 + nn;
  if (r > 0) {
    const uint16_t* Bg = reinterpret_cast<const uint16_t*>(b + a.lay.b_gate);
    const uint16_t* Bu = reinterpret_cast<const uint16_t*>(b + a.lay.b_up);
    for (int t = tid; t < 32 * r; t += 256) {
      const int rr = t % r, rw = t / r;
      bl_s[0][rw][rr] = bf2f(Bg[(size_t)(row0 + rw) * r + rr]);
      bl_s[1][rw][rr] = bf2f(Bu[(size_t)(row0 + rw) * r + rr]);
    }
    const uint16_t* Ad = reinterpret_cast<const uint16_t*>(b + a.lay.a_down);
    for (int t = tid; t < 32 * r; t += 256) {
      const int c = t % 32, rr = t / 32;
      ad_s[rr][c] = bf2f(Ad[(size_t)rr * I + row0 + c]);
    }
  }
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q) + (size_t)row * (d / 8);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q) + (size_t)row * (d / 8);
  const uint16_t* gsp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s) + (size_t)row * ng;
  const uint16_t* gbp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b) + (size_t)row * ng;
  const uint16_t* usp = reinterpret_cast<const uint16_t*>(b + a.lay.up_s) + (size_t)row * ng;
  const uint16_t* ubp = reinterpret_cast<const uint16_t*>(b + a.lay.up_b) + (size_t)row * ng;
  for (int t0 = 0; t0 < n; t0 += 32) {
    const int mt = n - t0 < 32 ? n - t0 : 32;
    __syncthreads();  // LDS of the previous tile consumed; staging above done
    for (int t = tid; t < mt * 2 * r; t += 256) {
      const int m = t / (2 * r), rem = t % (2 * r);
      tl_s[m][rem / r][rem % r] = a.t_in[(size_t)(q0 + t0 + m) * 2 * r + rem];
    }
    const bool tok_ok = nn < mt;
    const uint16_t* xrow = a.x + (size_t)a.pair_tok[q0 + t0 + (tok_ok ? nn : 0)] * d;
    f32x16_t accG, accU;
#pragma unroll
    for (int v = 0; v < 16; ++v) accG[v] = accU[v] = 0.f;
    // passes of up to kGW groups per wave: every weight load of the pass is
    // issued first, the activations of group i+1 while group i computes
    for (int G0 = wave; G0 < ng; G0 += 4 * kGW) {
      uint32_t wg[kGW][SPG], wu[kGW][SPG];
      uint32_t sc[kGW][4];  // raw bf16 s, b of gate and up
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        const int G = G0 + 4 * i;
        if (G < ng) {
          load_words<SPG>(gq + (size_t)G * (g / 8) + jh * SPG, wg[i]);
          load_words<SPG>(uq + (size_t)G * (g / 8) + jh * SPG, wu[i]);
          sc[i][0] = gsp[G];
          sc[i][1] = gbp[G];
          sc[i][2] = usp[G];
          sc[i][3] = ubp[G];
        }
      }
      uint4 xr[2][SPG];
      auto load_x = [&](int i, uint4 (&dst)[SPG]) {
        const int G = G0 + 4 * i;
#pragma unroll
        for (int t = 0; t < SPG; ++t)
          dst[t] = (tok_ok && G < ng)
                       ? reinterpret_cast<const uint4*>(xrow + G * g + jh * (g / 2))[t]
                       : make_uint4(0, 0, 0, 0);
      };
      load_x(0, xr[0]);
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        const int G = G0 + 4 * i;
        if (i + 1 < kGW) load_x(i + 1, xr[(i + 1) & 1]);
        if (G < ng) {
          const uint4* xv = xr[i & 1];
          const float sg = bf2f(sc[i][0]), cbg = bf2f(sc[i][1]) - 128.f * sg;
          const float su = bf2f(sc[i][2]), cbu = bf2f(sc[i][3]) - 128.f * su;
          float sx = 0.f;
#pragma unroll
          for (int t = 0; t < SPG; ++t) sx += raw_sum8(xv[t]);
          sx += __shfl_xor(sx, 32, kWave);  // the group's sum for token nn
          f32x16_t cg, cu;
#pragma unroll
          for (int v = 0; v < 16; ++v) cg[v] = cu[v] = 0.f;
#pragma unroll
          for (int t = 0; t < SPG; ++t) {
            const bf16x8_t xo = x_operand(xv[t]);
            cg = mfma32(xo, q4_operand(wg[i][t]), cg);
            cu = mfma32(xo, q4_operand(wu[i][t]), cu);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
            const float sxm = __shfl(sx, m, kWave);
            accG[v] += sg * cg[v] + cbg * sxm;
            accU[v] += su * cu[v] + cbu * sxm;
          }
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
      red[wave][0][nn][m] = accG[v];
      red[wave][1][nn][m] = accU[v];
    }
    __syncthreads();
    for (int t = tid; t < mt * 32; t += 256) {
      const int m = t / 32, rw = t % 32;
      float Gv = red[0][0][rw][m] + red[1][0][rw][m] + red[2][0][rw][m] + red[3][0][rw][m];
      float Uv = red[0][1][rw][m] + red[1][1][rw][m] + red[2][1][rw][m] + red[3][1][rw][m];
      if (r > 0) {
        float dg = 0.f, du = 0.f;
        for (int rr = 0; rr < r; ++rr) {
          dg += bl_s[0][rw][rr] * tl_s[m][0][rr];
          du += bl_s[1][rw][rr] * tl_s[m][1][rr];
        }
        Gv += a.scale * dg;
        Uv += a.scale * du;
      }
      const float h = grp_silu(Gv) * Uv;
      hbuf[m][rw] = h;
      hrep_s[m][rw] = grp_store_h(a, q0 + t0 + m, row0 + rw, h);
    }
    __syncthreads();
    for (int t = tid; t < mt * 2; t += 256) {
      const int m = t / 2, half = t % 2;
      float sm = 0.f;
      for (int k = 0; k < 16; ++k) sm += hrep_s[m][16 * half + k];
      a.hs[(size_t)(q0 + t0 + m) * (I / 16) + rb * 2 + half] = sm;
    }
    for (int t = tid; t < mt * r; t += 256) {
      const int m = t / r, rr = t % r;
      float sm = 0.f;
      for (int k = 0; k < 32; ++k) sm += ad_s[rr][k] * hbuf[m][k];
      atomicAdd(a.tdown + (size_t)(q0 + t0 + m) * r + rr, to_fix(sm));
    }
  }
}

// One workgroup = 32 output rows of one active expert's down projection,
// all its tokens in tiles of 32; h enters as its bf16 hi and lo parts.
template <int SPG>
__global__ __launch_bounds__(256) void k_grp_down_mfma(GrpArgs a, int min_cnt) {
  __shared__ float red[4][32][33];  // per wave: [output row][token]
  __shared__ float bd_s[32][64];    // B_down rows of the block
  __shared__ float td_s[32][64];    // t_down of the tile's tokens
  const int nb32 = a.d / 32;
  const int act = blockIdx.x / nb32;
  const int ob = blockIdx.x % nb32;
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 31, jh = lane >> 5;
  const int d = a.d, g = a.g, I = a.I, r = a.r, NC = I / 32, ngI = I / g;
  const int o0 = ob * 32, o = o0 + nn;
  const int trb = o / 64, within = o % 64;
  if (r > 0) {
    const uint16_t* Bd = reinterpret_cast<const uint16_t*>(b + a.lay.b_down);
    for (int t = tid; t < 32 * r; t += 256) bd_s[t / r][t % r] = bf2f(Bd[(size_t)(o0 + t / r) * r + t % r]);
  }
  const uint32_t* dq = reinterpret_cast<const uint32_t*>(b + a.lay.down_q);
  const uint16_t* dsp = reinterpret_cast<const uint16_t*>(b + a.lay.down_s);
  const uint16_t* dbp = reinterpret_cast<const uint16_t*>(b + a.lay.down_b);
  for (int t0 = 0; t0 < n; t0 += 32) {
    const int mt = n - t0 < 32 ? n - t0 : 32;
    __syncthreads();
    for (int t = tid; t < mt * r; t += 256)
      td_s[t / r][t % r] = from_fix(a.tdown[(size_t)(q0 + t0 + t / r) * r + t % r]);
    const bool tok_ok = nn < mt;
    const int q = q0 + t0 + (tok_ok ? nn : 0);
    const uint16_t* hhi = a.hp_hi + (size_t)q * I;
    const uint16_t* hlo = a.hp_lo + (size_t)q * I;
    const float* hsq = a.hs + (size_t)q * (I / 16);
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    for (int G0 = wave; G0 < ngI; G0 += 4 * kGW) {
      // the pass's weights first: words j*SPG .. of each group (input
      // i0 = G*g + j*g/2; tiled layout: chunk i0/32, word (i0%32)/8 of row
      // o's 16 bytes), then the h pairs of group i+1 while group i computes
      uint32_t wd[kGW][SPG];
      uint32_t sc[kGW][2];
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        const int G = G0 + 4 * i;
        if (G < ngI) {
          const int i0 = G * g + jh * (g / 2);
#pragma unroll
          for (int t = 0; t < SPG; ++t) {
            const int ii = i0 + 8 * t;
            wd[i][t] = dq[(((size_t)trb * NC + ii / 32) * 64 + within) * 4 + (ii % 32) / 8];
          }
          sc[i][0] = dsp[(size_t)G * d + o];
          sc[i][1] = dbp[(size_t)G * d + o];
        }
      }
      uint4 hh[2][SPG], hl[2][SPG];
      auto load_h = [&](int i, uint4 (&dh)[SPG], uint4 (&dl)[SPG]) {
        const int G = G0 + 4 * i;
        const int i0 = G * g + jh * (g / 2);
        const bool on = tok_ok && G < ngI;
#pragma unroll
        for (int t = 0; t < SPG; ++t) {
          dh[t] = on ? reinterpret_cast<const uint4*>(hhi + i0)[t] : make_uint4(0, 0, 0, 0);
          dl[t] = on ? reinterpret_cast<const uint4*>(hlo + i0)[t] : make_uint4(0, 0, 0, 0);
        }
      };
      load_h(0, hh[0], hl[0]);
#pragma unroll
      for (int i = 0; i < kGW; ++i) {
        const int G = G0 + 4 * i;
        if (i + 1 < kGW) load_h(i + 1, hh[(i + 1) & 1], hl[(i + 1) & 1]);
        if (G < ngI) {
          const float sd = bf2f(sc[i][0]);
          const float cbd = bf2f(sc[i][1]) - 128.f * sd;
          float sh = 0.f;
          if (tok_ok)
            for (int k = 0; k < g / 16; ++k) sh += hsq[G * (g / 16) + k];
          f32x16_t c;
#pragma unroll
          for (int v = 0; v < 16; ++v) c[v] = 0.f;
#pragma unroll
          for (int t = 0; t < SPG; ++t) {
            const bf16x8_t wo = q4_operand(wd[i][t]);
            c = mfma32(__builtin_bit_cast(bf16x8_t, hh[i & 1][t]), wo, c);
            c = mfma32(__builtin_bit_cast(bf16x8_t, hl[i & 1][t]), wo, c);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
            acc[v] += sd * c[v] + cbd * __shfl(sh, m, kWave);
          }
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave][nn][8 * (v >> 2) + 4 * jh + (v & 3)] = acc[v];
    __syncthreads();
    for (int t = tid; t < mt * 32; t += 256) {
      const int m = t / 32, rw = t % 32;
      float tot = red[0][rw][m] + red[1][rw][m] + red[2][rw][m] + red[3][rw][m];
      if (r > 0) {
        float dl = 0.f;
        for (int rr = 0; rr < r; ++rr) dl += bd_s[rw][rr] * td_s[m][rr];
        tot += a.scale * dl;
      }
      const int qq = q0 + t0 + m;
      atomicAdd(a.acc + (size_t)a.pair_tok[qq] * d + o0 + rw, to_fix(a.pair_w[qq] * tot));
    }
  }
}

// ------------------------------------------------- MFMA, pipelined (v2)
// GEMM-shaped variants for I % 128 == 0, d % 128 == 0 and lora_rank <= 16:
// a workgroup covers 128 weight rows (4 waves x 32, each wave the full
// reduction) for up to 32 tokens of one expert; the activation tile is
// staged in LDS in chunks of kKC inputs (double-buffered, shared by the 4
// waves, with each group's activation sum), and each wave's weight words of
// the next chunk are in flight while the current chunk computes.  Operand
// order and the per-group fold are those of the kernels above.
constexpr int kKC = 128;  // inputs per staged chunk

// Stage the activations of chunk c (tokens m < mt of the tile): thread t ->
// token t / 8, 16 inputs (16 p .. 16 p + 15), p = t % 8; each group's sum
// from the threads of its parts (neighbouring lanes of the same token).
template <int SPG>
__device__ __forceinline__ void grp_stage_x(const GrpArgs& a, int q0, int t0, int mt, int c,
                                            uint16_t (*xs)[kKC], float (*gs)[8]) {
  constexpr int G = 16 * SPG;     // group size
  constexpr int PPG = G / 16;     // parts per group (2, 4, 8)
  const int t = threadIdx.x, m = t >> 3, p = t & 7;
  uint4 v[2];
  float sum = 0.f;
  if (m < mt) {
    const uint16_t* src = a.x + (size_t)a.pair_tok[q0 + t0 + m] * a.d + c * kKC + 16 * p;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      v[u] = reinterpret_cast<const uint4*>(src)[u];
      sum += raw_sum8(v[u]);
    }
  } else {
    v[0] = v[1] = make_uint4(0, 0, 0, 0);
  }
  reinterpret_cast<uint4*>(&xs[m][16 * p])[0] = v[0];
  reinterpret_cast<uint4*>(&xs[m][16 * p])[1] = v[1];
  sum += __shfl_xor(sum, 1, kWave);
  if constexpr (PPG >= 4) sum += __shfl_xor(sum, 2, kWave);
  if constexpr (PPG >= 8) sum += __shfl_xor(sum, 4, kWave);
  if (p % PPG == 0) gs[m][p / PPG] = sum;
}

template <int SPG>
__global__ __launch_bounds__(256, 2) void k_grp_gate_up_mfma2(GrpArgs a, int min_cnt) {
  constexpr int G = 16 * SPG, CG = kKC / G;  // group size, groups per chunk
  __shared__ uint16_t xs[2][32][kKC];
  __shared__ float gsx[2][32][8];
  __shared__ float tl_s[32][2][kFusedRank];
  __shared__ float bl_s[2][128][kFusedRank];
  const int nb = a.I / 128;
  const int act = blockIdx.x / nb;
  const int rb = blockIdx.x % nb;
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 31, jh = lane >> 5;
  const int d = a.d, ng = d / G, r = a.r, I = a.I;
  const int row = rb * 128 + 32 * wave + nn;
  const int nch = d / kKC;
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q) + (size_t)row * (d / 8);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q) + (size_t)row * (d / 8);
  const uint16_t* gsp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s) + (size_t)row * ng;
  const uint16_t* gbp = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b) + (size_t)row * ng;
  const uint16_t* usp = reinterpret_cast<const uint16_t*>(b + a.lay.up_s) + (size_t)row * ng;
  const uint16_t* ubp = reinterpret_cast<const uint16_t*>(b + a.lay.up_b) + (size_t)row * ng;
  if (r > 0) {
    const uint16_t* Bg = reinterpret_cast<const uint16_t*>(b + a.lay.b_gate);
    const uint16_t* Bu = reinterpret_cast<const uint16_t*>(b + a.lay.b_up);
    for (int t = tid; t < 128 * r; t += 256) {
      const int rw = t / r, rr = t % r;
      bl_s[0][rw][rr] = bf2f(Bg[(size_t)(rb * 128 + rw) * r + rr]);
      bl_s[1][rw][rr] = bf2f(Bu[(size_t)(rb * 128 + rw) * r + rr]);
    }
  }
  uint32_t wg[2][CG][SPG], wu[2][CG][SPG], sc[2][CG][4];
  auto load_w = [&](int c, int bi) {
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      const int Gi = c * CG + i;
      load_words<SPG>(gq + (size_t)Gi * (G / 8) + jh * SPG, wg[bi][i]);
      load_words<SPG>(uq + (size_t)Gi * (G / 8) + jh * SPG, wu[bi][i]);
      sc[bi][i][0] = gsp[Gi];
      sc[bi][i][1] = gbp[Gi];
      sc[bi][i][2] = usp[Gi];
      sc[bi][i][3] = ubp[Gi];
    }
  };
  for (int t0 = 0; t0 < n; t0 += 32) {
    const int mt = n - t0 < 32 ? n - t0 : 32;
    __syncthreads();  // previous tile's LDS consumed
    for (int t = tid; t < mt * 2 * r; t += 256) {
      const int m = t / (2 * r), rem = t % (2 * r);
      tl_s[m][rem / r][rem % r] = a.t_in[(size_t)(q0 + t0 + m) * 2 * r + rem];
    }
    f32x16_t accG, accU;
#pragma unroll
    for (int v = 0; v < 16; ++v) accG[v] = accU[v] = 0.f;
    load_w(0, 0);
    grp_stage_x<SPG>(a, q0, t0, mt, 0, xs[0], gsx[0]);
    for (int c = 0; c < nch; ++c) {
      const int buf = c & 1;
      __syncthreads();  // chunk c staged; the other buffer free
      if (c + 1 < nch) {
        if (buf) load_w(c + 1, 0); else load_w(c + 1, 1);
        grp_stage_x<SPG>(a, q0, t0, mt, c + 1, xs[buf ^ 1], gsx[buf ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < CG; ++i) {
        f32x16_t cg, cu;
#pragma unroll
        for (int v = 0; v < 16; ++v) cg[v] = cu[v] = 0.f;
        uint32_t w_g[SPG], w_u[SPG], s_[4];
#pragma unroll
        for (int st = 0; st < SPG; ++st) {
          w_g[st] = buf ? wg[1][i][st] : wg[0][i][st];
          w_u[st] = buf ? wu[1][i][st] : wu[0][i][st];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) s_[q] = buf ? sc[1][i][q] : sc[0][i][q];
#pragma unroll
        for (int st = 0; st < SPG; ++st) {
          const uint4 xr = *reinterpret_cast<const uint4*>(&xs[buf][nn][i * G + jh * (G / 2) + 8 * st]);
          const bf16x8_t xo = x_operand(xr);
          cg = mfma32(xo, q4_operand(w_g[st]), cg);
          cu = mfma32(xo, q4_operand(w_u[st]), cu);
        }
        const float sg = bf2f(s_[0]), cbg = bf2f(s_[1]) - 128.f * sg;
        const float su = bf2f(s_[2]), cbu = bf2f(s_[3]) - 128.f * su;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
          const float sxm = gsx[buf][m][i];
          accG[v] += sg * cg[v] + cbg * sxm;
          accU[v] += su * cu[v] + cbu * sxm;
        }
      }
    }
    // epilogue: LoRA B t, SwiGLU, h pairs and the 16-row sums of this wave
    const int rl = 32 * wave + nn;  // row within the workgroup
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
      float Gv = accG[v], Uv = accU[v];
      if (r > 0) {
        float dg = 0.f, du = 0.f;
        for (int rr = 0; rr < r; ++rr) {
          dg += bl_s[0][rl][rr] * tl_s[m][0][rr];
          du += bl_s[1][rl][rr] * tl_s[m][1][rr];
        }
        Gv += a.scale * dg;
        Uv += a.scale * du;
      }
      const float h = grp_silu(Gv) * Uv;
      const float hr = m < mt ? grp_store_h(a, q0 + t0 + m, row, h) : 0.f;
      const float s16 = row16_sum(hr);  // rows of the same 16-row block
      if ((nn & 15) == 0 && m < mt) a.hs[(size_t)(q0 + t0 + m) * (I / 16) + (row >> 4)] = s16;
    }
  }
}

template <int SPG>
__global__ __launch_bounds__(256, 2) void k_grp_down_mfma2(GrpArgs a, int min_cnt) {
  constexpr int G = 16 * SPG, CG = kKC / G;
  __shared__ uint16_t hs_hi[2][32][kKC];
  __shared__ uint16_t hs_lo[2][32][kKC];
  __shared__ uint16_t ad_s[2][kFusedRank][kKC];   // A_down rows of the chunk
  __shared__ float gsh[2][32][kKC / 16];          // 16-row sums of h per chunk
  __shared__ float td_s[32][kFusedRank + 1];      // t_down [token][rank]
  __shared__ float bd_s[128][kFusedRank];
  const int nb = a.d / 128;
  const int act = blockIdx.x / nb;
  const int ob = blockIdx.x % nb;
  if (act >= a.info[0]) return;
  const int n = a.act_cnt[act];
  if (n < min_cnt) return;
  const uint8_t* b = grp_bundle(a, act);
  if (b == nullptr) return;
  const int q0 = a.act_off[act];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 31, jh = lane >> 5;
  const int d = a.d, I = a.I, r = a.r, NC = I / 32;
  const int o = ob * 128 + 32 * wave + nn;
  const int trb = o / 64, within = o % 64;
  const int nch = I / kKC;
  const uint32_t* dq = reinterpret_cast<const uint32_t*>(b + a.lay.down_q);
  const uint16_t* dsp = reinterpret_cast<const uint16_t*>(b + a.lay.down_s);
  const uint16_t* dbp = reinterpret_cast<const uint16_t*>(b + a.lay.down_b);
  const uint16_t* adp = reinterpret_cast<const uint16_t*>(b + (r > 0 ? a.lay.a_down : 0));
  if (r > 0) {
    const uint16_t* Bd = reinterpret_cast<const uint16_t*>(b + a.lay.b_down);
    for (int t = tid; t < 128 * r; t += 256)
      bd_s[t / r][t % r] = bf2f(Bd[(size_t)(ob * 128 + t / r) * r + t % r]);
  }
  uint32_t wd[2][CG][SPG], sc[2][CG][2];
  auto load_w = [&](int c, int bi) {
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      const int Gi = c * CG + i;
      const int i0 = Gi * G + jh * (G / 2);
#pragma unroll
      for (int st = 0; st < SPG; ++st) {
        const int ii = i0 + 8 * st;
        wd[bi][i][st] = dq[(((size_t)trb * NC + ii / 32) * 64 + within) * 4 + (ii % 32) / 8];
      }
      sc[bi][i][0] = dsp[(size_t)Gi * d + o];
      sc[bi][i][1] = dbp[(size_t)Gi * d + o];
    }
  };
  auto stage_h = [&](int t0, int mt, int c, int buf) {
    // thread t -> token t / 8, 16 inputs of the chunk; h pairs as stored
    const int t = tid, m = t >> 3, p = t & 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 hv = make_uint4(0, 0, 0, 0), lv = hv;
      if (m < mt) {
        const size_t off = (size_t)(q0 + t0 + m) * I + c * kKC + 16 * p + 8 * u;
        hv = *reinterpret_cast<const uint4*>(a.hp_hi + off);
        lv = *reinterpret_cast<const uint4*>(a.hp_lo + off);
      }
      reinterpret_cast<uint4*>(&hs_hi[buf][m][16 * p])[u] = hv;
      reinterpret_cast<uint4*>(&hs_lo[buf][m][16 * p])[u] = lv;
    }
    gsh[buf][m][p] = m < mt ? a.hs[(size_t)(q0 + t0 + m) * (I / 16) + c * (kKC / 16) + p] : 0.f;
    // A_down rows of the chunk (ranks >= r are zero)
    for (int e = t; e < kFusedRank * (kKC / 8); e += 256) {
      const int rr = e / (kKC / 8), k8 = e % (kKC / 8);
      uint4 av = make_uint4(0, 0, 0, 0);
      if (rr < r) av = *reinterpret_cast<const uint4*>(adp + (size_t)rr * I + c * kKC + 8 * k8);
      reinterpret_cast<uint4*>(&ad_s[buf][rr][0])[k8] = av;
    }
  };
  for (int t0 = 0; t0 < n; t0 += 32) {
    const int mt = n - t0 < 32 ? n - t0 : 32;
    __syncthreads();
    f32x16_t acc, tdv;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = tdv[v] = 0.f;
    load_w(0, 0);
    stage_h(t0, mt, 0, 0);
    for (int c = 0; c < nch; ++c) {
      const int buf = c & 1;
      __syncthreads();
      if (c + 1 < nch) {
        if (buf) load_w(c + 1, 0); else load_w(c + 1, 1);
        stage_h(t0, mt, c + 1, buf ^ 1);
      }
#pragma unroll
      for (int i = 0; i < CG; ++i) {
        f32x16_t cc;
#pragma unroll
        for (int v = 0; v < 16; ++v) cc[v] = 0.f;
#pragma unroll
        for (int st = 0; st < SPG; ++st) {
          const int col = i * G + jh * (G / 2) + 8 * st;
          const bf16x8_t hh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&hs_hi[buf][nn][col]));
          const bf16x8_t hl = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&hs_lo[buf][nn][col]));
          const bf16x8_t wo = q4_operand(buf ? wd[1][i][st] : wd[0][i][st]);
          cc = mfma32(hh, wo, cc);
          cc = mfma32(hl, wo, cc);
          if (wave == 0 && r > 0) {
            // t_down += h A_down^T (lane nn = rank; A_down in the pair order of h)
            const uint4 araw = nn < kFusedRank ? *reinterpret_cast<const uint4*>(&ad_s[buf][nn][col])
                                               : make_uint4(0, 0, 0, 0);
            const bf16x8_t ao = x_operand(araw);
            tdv = mfma32(hh, ao, tdv);
            tdv = mfma32(hl, ao, tdv);
          }
        }
        const uint32_t s0 = buf ? sc[1][i][0] : sc[0][i][0];
        const uint32_t s1 = buf ? sc[1][i][1] : sc[0][i][1];
        const float sd = bf2f(s0), cbd = bf2f(s1) - 128.f * sd;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
          float sh = 0.f;
#pragma unroll
          for (int k = 0; k < G / 16; ++k) sh += gsh[buf][m][i * (G / 16) + k];
          acc[v] += sd * cc[v] + cbd * sh;
        }
      }
    }
    if (wave == 0 && nn < kFusedRank) {
#pragma unroll
      for (int v = 0; v < 16; ++v) td_s[8 * (v >> 2) + 4 * jh + (v & 3)][nn] = tdv[v];
    }
    __syncthreads();
    const int rl = 32 * wave + nn;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * jh + (v & 3);
      if (m < mt) {
        float tot = acc[v];
        if (r > 0) {
          float dl = 0.f;
          for (int rr = 0; rr < r; ++rr) dl += bd_s[rl][rr] * td_s[m][rr];
          tot += a.scale * dl;
        }
        const int qq = q0 + t0 + m;
        atomicAdd(a.acc + (size_t)a.pair_tok[qq] * d + o, to_fix(a.pair_w[qq] * tot));
      }
    }
  }
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

// ------------------------------------------------------------- host side
struct GrpWs {
  size_t err, info, act_e, act_off, act_cnt, act_slot, pair_tok, pair_act, pair_w, t_in, hp_hi,
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
  L.pair_act = take(4 * P);
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
    case 1: k_grp_gate_up<1><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
    case 2: k_grp_gate_up<2><<<grid, 256, 0, st>>>(a, lo, hi, ts); break;
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

static bool grp_mfma2_ok(const GrpArgs& a) {
  return a.I % 128 == 0 && a.d % 128 == 0 && a.r <= kFusedRank && a.g <= kKC;
}

// which = 0 gate/up, 1 down
static int launch_grp_mfma(const GrpArgs& a, int which, int min_cnt, hipStream_t st) {
  const int spg = a.g / 16;
  if (grp_mfma2_ok(a)) {
    const int grid2 = a.Amax * ((which ? a.d : a.I) / 128);
#define E0_GRP_MFMA2(S)                                                     \
  if (which) k_grp_down_mfma2<S><<<grid2, 256, 0, st>>>(a, min_cnt);        \
  else k_grp_gate_up_mfma2<S><<<grid2, 256, 0, st>>>(a, min_cnt)
    switch (spg) {
      case 2: E0_GRP_MFMA2(2); break;
      case 4: E0_GRP_MFMA2(4); break;
      case 8: E0_GRP_MFMA2(8); break;
      default: return EDGE0_EINVAL;
    }
#undef E0_GRP_MFMA2
    E0_CHECK_LAUNCH();
    return EDGE0_OK;
  }
  const int grid = a.Amax * ((which ? a.d : a.I) / 32);
#define E0_GRP_MFMA(S)                                            \
  if (which) k_grp_down_mfma<S><<<grid, 256, 0, st>>>(a, min_cnt); \
  else k_grp_gate_up_mfma<S><<<grid, 256, 0, st>>>(a, min_cnt)
  switch (spg) {
    case 2: E0_GRP_MFMA(2); break;
    case 4: E0_GRP_MFMA(4); break;
    case 8: E0_GRP_MFMA(8); break;
    default: return EDGE0_EINVAL;
  }
#undef E0_GRP_MFMA
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

}  // namespace e0

using namespace e0;

extern "C" size_t edge0_grouped_workspace_bytes(const edge0_moe_shape* shape) {
  if (!grouped_shape_ok(shape)) return 0;
  return grp_ws_layout(shape).total;
}

extern "C" int edge0_moe_grouped(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                 const int32_t* slot_table, int32_t n_tokens, const int32_t* ids,
                                 const float* w, const void* x, void* y, void* workspace,
                                 int32_t flags, hipStream_t stream) {
  if (!shape || !grouped_shape_ok(shape) || !pool || !pool->base || !slot_table || !workspace ||
      n_tokens < 0 || n_tokens > kGrpMaxTokens || (flags & ~(EDGE0_GROUPED_NO_MFMA | 0xFF00)) != 0)
    return EDGE0_EINVAL;
  if (n_tokens == 0) return EDGE0_OK;
  if (!ids || !w || !x || !y) return EDGE0_EINVAL;
  edge0_bundle_layout lay;
  if (bundle_layout(shape, &lay) != EDGE0_OK || pool->slot_bytes < lay.bytes) return EDGE0_EINVAL;
  const GrpWs L = grp_ws_layout(shape);
  char* ws = static_cast<char*>(workspace);
  GrpArgs a{};
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
  a.lay = lay;
  a.P = n_tokens * a.K;
  a.Amax = a.E < a.P ? a.E : a.P;
  a.err = reinterpret_cast<uint32_t*>(ws + L.err);
  a.info = reinterpret_cast<int32_t*>(ws + L.info);
  a.act_e = reinterpret_cast<int32_t*>(ws + L.act_e);
  a.act_off = reinterpret_cast<int32_t*>(ws + L.act_off);
  a.act_cnt = reinterpret_cast<int32_t*>(ws + L.act_cnt);
  a.act_slot = reinterpret_cast<int32_t*>(ws + L.act_slot);
  a.pair_tok = reinterpret_cast<int32_t*>(ws + L.pair_tok);
  a.pair_act = reinterpret_cast<int32_t*>(ws + L.pair_act);
  a.pair_w = reinterpret_cast<float*>(ws + L.pair_w);
  a.t_in = reinterpret_cast<float*>(ws + L.t_in);
  a.hp_hi = reinterpret_cast<uint16_t*>(ws + L.hp_hi);
  a.hp_lo = reinterpret_cast<uint16_t*>(ws + L.hp_lo);
  a.hs = reinterpret_cast<float*>(ws + L.hs);
  a.tdown = reinterpret_cast<unsigned long long*>(ws + L.tdown);
  a.acc = reinterpret_cast<unsigned long long*>(ws + L.acc);
  k_grp_route<<<1, 1024, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  if (a.r > 0) {
    k_grp_lora_in<<<(a.P * 2 * a.r + 3) / 4, 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
  }
  // GEMVs for every expert unless the caller asks for MFMA from min_mfma
  // tokens per expert on
  const int min_mfma = (flags >> 8) & 0xFF;
  const bool mfma = !(flags & EDGE0_GROUPED_NO_MFMA) && min_mfma > 0 && n_tokens >= min_mfma;
  const int gemv_max = mfma ? min_mfma - 1 : 1 << 30;
  int rc = gemv_max >= 1 ? launch_grp_gate_up(a, 1, gemv_max, stream) : EDGE0_OK;
  if (rc == EDGE0_OK && mfma) rc = launch_grp_mfma(a, 0, min_mfma, stream);
  if (rc == EDGE0_OK && gemv_max >= 1) rc = launch_grp_down(a, 1, gemv_max, stream);
  if (rc == EDGE0_OK && mfma) rc = launch_grp_mfma(a, 1, min_mfma, stream);
  if (rc != EDGE0_OK) return rc;
  const int n_out = a.T * a.d;
  k_grp_out<<<(n_out + 255) / 256, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
