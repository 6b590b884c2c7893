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
__global__ __launch_bounds__(256) void k_lora_in(MoeArgs a) {
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  const int nrows = a.K * 2 * a.r;
  if (row >= nrows) return;
  const int k = row / (2 * a.r);
  const int p = (row / a.r) & 1;
  const int rr = row % a.r;
  const uint8_t* b = slot_of(a, k);
  float t = 0.f;
  if (b != nullptr) {
    const uint16_t* A = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.a_up : a.lay.a_gate)) +
                        (size_t)rr * a.d;
    t = row_dot<false, false>(A, a.x, a.d);
  } else if ((threadIdx.x & 63) == 0) {
    set_error(a.err, EDGE0_ERANGE);
  }
  if ((threadIdx.x & 63) == 0) a.t_in[row] = t;
}

// -------------------------------------------------------------- k_gate_up
// Activation chunk `col` (32 bf16 of x) as the 16 pairs chunk_dot128 expects,
// and its fp32 sum.
__device__ __forceinline__ float load_x_pairs(const uint16_t* __restrict__ x, int col,
                                              uint32_t xp[16]) {
  const uint4* src = reinterpret_cast<const uint4*>(x + 32 * col);
  float sum = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 v = src[m];
    pair_perm8(v.x, v.y, v.z, v.w, xp + 4 * m);
    sum += bf_lo(v.x) + bf_hi(v.x) + bf_lo(v.y) + bf_hi(v.y) + bf_lo(v.z) + bf_hi(v.z) +
           bf_lo(v.w) + bf_hi(v.w);
  }
  return sum;
}

// position of element i of h in the pair-permuted order of its 8-group
__device__ __forceinline__ int pair_pos(int i) {
  const int s = i & 7;
  return (i & ~7) + (s < 4 ? 2 * s : 2 * (s - 4) + 1);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

// store one row of h: fp32, the bf16 hi/lo split (hi = bf16(h), lo = bf16(h - hi))
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
// the gate and the up row; one row pair per step, 4 steps per wave.
template <int NJ>
__device__ __forceinline__ void gate_up_wide(const MoeArgs& a, const uint8_t* b, int k, int i0,
                                             float* h_s, float* hrep_s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = a.d, g = a.g, ng = d / g;
  uint32_t xp[NJ][16];
  float X[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) X[j] = load_x_pairs(a.x, lane + 64 * j, xp[j]);
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s);
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(b + a.lay.up_s);
  const uint16_t* ub = reinterpret_cast<const uint16_t*>(b + a.lay.up_b);
  constexpr int R = 4;
  uint4 qg[R][NJ], qu[R][NJ];
  uint32_t sg[R][NJ], bg[R][NJ], su[R][NJ], bu[R][NJ];
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    const int row = i0 + 4 * wave + ii;
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
#pragma unroll
  for (int ii = 0; ii < R; ++ii) {
    const int row = i0 + 4 * wave + ii;
    float G = 0.f, U = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float s1 = bf2f(sg[ii][j]), b1 = bf2f(bg[ii][j]);
      const float s2 = bf2f(su[ii][j]), b2 = bf2f(bu[ii][j]);
      G += s1 * chunk_dot128(qg[ii][j], xp[j]) + (b1 - 128.f * s1) * X[j];
      U += s2 * chunk_dot128(qu[ii][j], xp[j]) + (b2 - 128.f * s2) * X[j];
    }
    if (a.r > 0) {
      const uint16_t* Bg = reinterpret_cast<const uint16_t*>(b + a.lay.b_gate) + (size_t)row * a.r;
      const uint16_t* Bu = reinterpret_cast<const uint16_t*>(b + a.lay.b_up) + (size_t)row * a.r;
      const float* tg = a.t_in + (size_t)(k * 2 + 0) * a.r;
      const float* tu = a.t_in + (size_t)(k * 2 + 1) * a.r;
      float dg = 0.f, du = 0.f;
      for (int rr = lane; rr < a.r; rr += 64) {
        dg += bf2f(Bg[rr]) * tg[rr];
        du += bf2f(Bu[rr]) * tu[rr];
      }
      G += a.scale * dg;
      U += a.scale * du;
    }
    G = wave_sum(G);
    U = wave_sum(U);
    const float h = silu_f(G) * U;
    if (lane == 0) {
      h_s[4 * wave + ii] = h;
      hrep_s[4 * wave + ii] = store_h(a, k, row, h);
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rloc = lane / (2 * CPR);
  const int p = (lane / CPR) & 1;
  const int col = lane % CPR;
  const int d = a.d, g = a.g, ng = d / g;
  uint32_t xp[16];
  const float X = load_x_pairs(a.x, col, xp);
  const uint32_t* q = reinterpret_cast<const uint32_t*>(b + (p ? a.lay.up_q : a.lay.gate_q));
  const uint16_t* sp = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.up_s : a.lay.gate_s));
  const uint16_t* bp = reinterpret_cast<const uint16_t*>(b + (p ? a.lay.up_b : a.lay.gate_b));
  uint4 qq[STEPS];
  uint32_t ss[STEPS], bb[STEPS];
  const int grp = (32 * col) / g;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int row = i0 + 4 * wave + st * R + rloc;
    qq[st] = reinterpret_cast<const uint4*>(q + (size_t)row * (d / 8))[col];
    ss[st] = sp[row * ng + grp];
    bb[st] = bp[row * ng + grp];
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int row = i0 + 4 * wave + st * R + rloc;
    const float s = bf2f(ss[st]), bv = bf2f(bb[st]);
    float v = s * chunk_dot128(qq[st], xp) + (bv - 128.f * s) * X;
    if (a.r > 0) {
      const uint16_t* B =
          reinterpret_cast<const uint16_t*>(b + (p ? a.lay.b_up : a.lay.b_gate)) + (size_t)row * a.r;
      const float* t = a.t_in + (size_t)(k * 2 + p) * a.r;
      float dl = 0.f;
      for (int rr = col; rr < a.r; rr += CPR) dl += bf2f(B[rr]) * t[rr];
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

template <int CPR>
__global__ __launch_bounds__(256) void k_gate_up(MoeArgs a) {
  __shared__ float h_s[16];
  __shared__ float hrep_s[16];
  const int nblk = a.I / 16;
  const int k = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int i0 = blk * 16;
  const uint8_t* b = slot_of(a, k);
  if (b == nullptr) {
    // unresolvable expert: zero activations, flag the error
    for (int t = threadIdx.x; t < 16; t += blockDim.x) {
      store_h(a, k, i0 + t, 0.f);
    }
    if (threadIdx.x < a.r) a.tdpart[((size_t)k * nblk + blk) * a.r + threadIdx.x] = 0.f;
    if (threadIdx.x == 0) {
      a.hs[(size_t)k * nblk + blk] = 0.f;
      set_error(a.err, EDGE0_ERANGE);
    }
    return;
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
  if (threadIdx.x < a.r) {
    const int rr = threadIdx.x;
    const uint16_t* Ad = reinterpret_cast<const uint16_t*>(b + a.lay.a_down) + (size_t)rr * a.I + i0;
    float s = 0.f;
    for (int t = 0; t < 16; ++t) s += bf2f(Ad[t]) * h_s[t];
    a.tdpart[((size_t)k * nblk + blk) * a.r + rr] = s;
  }
}

// ------------------------------------------------------------------ k_down
__global__ __launch_bounds__(256) void k_down(MoeArgs a) {
  __shared__ float red[4][64];
  __shared__ float td[16 * 64];  // K * r <= 1024
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K, S = a.S, I = a.I, d = a.d;
  const int NC = I / 32;
  const int u = blockIdx.x;
  const int rb = u / (K * S);
  const int k = (u / S) % K;
  const int sl = u % S;
  const int cps = (NC + S - 1) / S;
  const int c0 = sl * cps;
  const int c1 = min(NC, c0 + cps);
  const uint8_t* b = slot_of(a, k);
  float part = 0.f;
  if (b != nullptr) {
    const uint4* dq = reinterpret_cast<const uint4*>(b + a.lay.down_q);
    const uint16_t* ds = reinterpret_cast<const uint16_t*>(b + a.lay.down_s);
    const uint16_t* db = reinterpret_cast<const uint16_t*>(b + a.lay.down_b);
    const uint32_t* hph = reinterpret_cast<const uint32_t*>(a.hp_hi + (size_t)k * I);
    const uint32_t* hpl = reinterpret_cast<const uint32_t*>(a.hp_lo + (size_t)k * I);
    const float* hs = a.hs + (size_t)k * (I / 16);
    const int o = rb * 64 + lane;
    for (int c = c0 + wave; c < c1; c += 4) {
      const uint4 q = dq[((size_t)rb * NC + c) * 64 + lane];
      const int grp = (32 * c) / a.g;
      const float s = bf2f(ds[(size_t)grp * d + o]);
      const float bv = bf2f(db[(size_t)grp * d + o]);
      const float acc = chunk_dot128(q, hph + 16 * c) + chunk_dot128(q, hpl + 16 * c);
      const float H = hs[2 * c] + hs[2 * c + 1];
      part += s * acc + (bv - 128.f * s) * H;
    }
  } else if (threadIdx.x == 0) {
    set_error(a.err, EDGE0_ERANGE);
  }
  red[wave][lane] = part;
  __syncthreads();
  if (wave == 0) {
    const float t = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    a.dpart[(((size_t)rb * K + k) * S + sl) * 64 + lane] = t;
  }
  if (!last_arrival(a.cnt_down + rb, (uint32_t)(K * S))) return;
  // fixup: this workgroup finishes rows rb*64 .. rb*64+63
  const int r = a.r;
  const int nblk = I / 16;
  for (int t = threadIdx.x; t < K * r; t += blockDim.x) {
    const int kk = t / r, rr = t % r;
    float s = 0.f;
    for (int blk = 0; blk < nblk; ++blk) s += a.tdpart[((size_t)kk * nblk + blk) * r + rr];
    td[t] = s;
  }
  __syncthreads();
  if (wave == 0) {
    const int o = rb * 64 + lane;
    float yv = 0.f;
    for (int kk = 0; kk < K; ++kk) {
      float D = 0.f;
      for (int s2 = 0; s2 < S; ++s2) D += a.dpart[(((size_t)rb * K + kk) * S + s2) * 64 + lane];
      const uint8_t* bk = slot_of(a, kk);
      if (r > 0 && bk != nullptr) {
        const uint16_t* Bd = reinterpret_cast<const uint16_t*>(bk + a.lay.b_down) + (size_t)o * r;
        float dl = 0.f;
        for (int rr = 0; rr < r; ++rr) dl += bf2f(Bd[rr]) * td[kk * r + rr];
        D += a.scale * dl;
      }
      yv += a.w[kk] * D;
    }
    const uint32_t yb = f2bf(yv);
    a.y[o] = (uint16_t)yb;
    if (a.h_out != nullptr) a.h_out[o] = (uint16_t)f2bf(bf2f(a.h_res[o]) + bf2f(yb));
  }
  if (threadIdx.x == 0) atomicExch(a.cnt_down + rb, 0u);
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
  a->dpart = reinterpret_cast<float*>(ws + L.dpart);
  const int RB = a->d / 64, NC = a->I / 32;
  int S = (512 + RB * a->K - 1) / (RB * a->K);
  a->S = S < 1 ? 1 : (S > NC ? NC : S);
  return EDGE0_OK;
}

int launch_moe(const MoeArgs& a, hipStream_t stream) {
  if (a.r > 0) {
    const int rows = a.K * 2 * a.r;
    k_lora_in<<<(rows + 3) / 4, 256, 0, stream>>>(a);
    E0_CHECK_LAUNCH();
  }
  const int cpr = a.d / 32;
  const int grid2 = a.K * (a.I / 16);
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
  const int grid3 = (a.d / 64) * a.K * a.S;
  k_down<<<grid3, 256, 0, stream>>>(a);
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
