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
// A layer is a short chain of launches, each one dependent round trip to
// memory (a kernel boundary inside a HIP graph costs less than any
// in-kernel hand-off between workgroups on this chip):
//   k_layer_in : the previous layer's combine and residual, RMSNorm, and
//                then either the router rows or (routing known) the LoRA A x
//                rows; resolves the K slots through the slot table once.
//                Router layers run it twice (router rows; then top-K, which
//                every workgroup computes, and the A x rows).
//   k_gate_up  : gate and up rows of the K experts, one wave per row pair
//                (row-major weights; each lane owns 32-input chunks and keeps
//                its activation chunk in registers), LoRA B t, SwiGLU.  Writes
//                h as bf16 hi/lo pairs, per-16-row sums of h, and per-16-row
//                partials of A_down h.
//   k_down     : tiled down weights (1 KiB tile = 64 rows x 32 inputs; lane =
//                output row, the tile's activation chunk is wave-uniform and
//                staged in LDS); a unit = 64 rows x one input slice over all
//                K experts, weighted by w_k, plus (slice 0) the LoRA-down
//                delta.  Writes S partial rows.
//   k_combine  : y = bf16(sum of the S partials) for the single-layer call
//                and the stack's last layer (otherwise the next layer's
//                k_layer_in does it).
//
// Int4 arithmetic: each 32-input chunk accumulates sum (128 + q) x with
// v_dot2_f32_bf16 on exact bf16 "128 + q" nibble pairs, and the group affine
// is applied per chunk as s * acc + (b - 128 s) * sum(x), which equals
// sum (s q + b) x.  Everything after the loads is fp32, rounded once to bf16.

#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>

#include "gemv_dev.h"
#include "heads_dev.h"
#include "moe_internal.h"

namespace e0 {

// routed expert k -> its bundle, from the slots resolved by k_layer_in
__device__ __forceinline__ const uint8_t* slot_ptr(const MoeArgs& a, int k) {
  const int s = a.slots[k];
  if (s < 0 || s >= a.n_slots) return nullptr;
  return a.pool + (size_t)s * (size_t)a.slot_bytes;
}
// id -> slot through the table (-1 when the id or its slot is invalid)
__device__ __forceinline__ int resolve_slot(const MoeArgs& a, int e) {
  if (e < 0 || e >= a.E) return -1;
  const int s = a.table[e];
  return (s < 0 || s >= a.n_slots) ? -1 : s;
}

// ------------------------------------------------------------ k_layer_in

// PER = d / 256 elements of the hidden state per thread
template <int PER>
__global__ __launch_bounds__(256) void k_layer_in(MoeArgs a, LayerIn li) {
  constexpr int kMaxPerThread = PER;
  __shared__ uint16_t xs[kMaxD];
  __shared__ int32_t ids_s[16];
  __shared__ float w_s[16];
  __shared__ float red[4];
  const int d = a.d, K = a.K, r = a.r, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x * 4 + wave;
  const bool router = li.flags & IN_ROUTER, lora = li.flags & IN_LORA;
  const int nrows = router ? a.E : (lora ? K * 2 * r : 0);
  const bool active = row < nrows;
  // Load order matters (loads complete in issue order): first the
  // prologue's h_prev and fixed-point y, then the chain that locates this
  // wave's weight row (ids, slot table) and the row itself, which lands
  // while the prologue computes.
  const bool has_pro = li.flags & (IN_COMBINE | IN_NORM);
  const bool comb = li.flags & IN_COMBINE;
  uint32_t hb[kMaxPerThread];
  unsigned long long av[kMaxPerThread];
  if (has_pro) {
#pragma unroll
    for (int m = 0; m < kMaxPerThread; ++m) {
      const int j = tid + 256 * m;
      hb[m] = li.h_prev[j];
      av[m] = comb ? a.acc_prev[j] : 0ull;
    }
  }
  // weight row of this wave, in flight during the prologue (when its address
  // does not depend on the top-K computed here)
  RowPref pf;
  const uint16_t* wrow = nullptr;
  if (active && router) wrow = li.w_router + (size_t)row * d;
  if (active && lora && !(li.flags & IN_TOPK)) {
    const int kk = row / (2 * r), up = (row / r) & 1;
    const int s = resolve_slot(a, a.ids[kk]);
    if (s >= 0)
      wrow = reinterpret_cast<const uint16_t*>(E0_LORA(a, a.pool + (size_t)s * a.slot_bytes, kk,
                                                       up ? 2 : 0, up ? a.lay.a_up : a.lay.a_gate)) +
             (size_t)(row % r) * d;
  }
  const bool pref = wrow != nullptr && d <= 64 * kPrefChunks * 8;
  if (pref) row_prefetch(wrow, d, pf);
  // prologue: combine, residual, RMSNorm
  const uint16_t* x = a.x;
  if (has_pro) {
    constexpr int per = PER;
    // this layer's accumulator starts from zero (its down units add into it)
    if (blockIdx.x == 0)
      for (int j = tid; j < d; j += 256) a.acc[j] = 0ull;
    float hv[kMaxPerThread];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < kMaxPerThread; ++m) {
      const int j = tid + 256 * m;
      hv[m] = bf2f(hb[m]);
      if (comb) {
        const uint32_t yb = f2bf(from_fix(av[m]));
        hv[m] = bf2f(f2bf(hv[m] + bf2f(yb)));
        if (blockIdx.x == 0) {
          li.y_prev_out[j] = (uint16_t)yb;
          li.h_out[j] = (uint16_t)f2bf(hv[m]);
        }
      }
      ss = fmaf(hv[m], hv[m], ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float inv = 1.f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + li.eps);
#pragma unroll
    for (int m = 0; m < kMaxPerThread; ++m) {
      const int j = tid + 256 * m;
      if (m < per) {
        const uint16_t xb = (uint16_t)f2bf(hv[m] * inv);
        xs[j] = xb;
        if (blockIdx.x == 0) li.x_out[j] = xb;
      }
    }
    __syncthreads();
    x = xs;
  }
  if (!(li.flags & (IN_COMBINE | IN_NORM)) && blockIdx.x == 0 && (li.flags & IN_LORA))
    for (int j = tid; j < d; j += 256) a.acc[j] = 0ull;
  // routing known to this launch: given, or top-K of the router logits
  const int32_t* ids = a.ids;
  if (li.flags & IN_TOPK) {
    if (wave == 0) wave_topk<false>(li.logits, a.E, K, ids_s, w_s);
    __syncthreads();
    if (blockIdx.x == 0 && tid < K) {
      li.ids_out[tid] = ids_s[tid];
      li.w_out[tid] = w_s[tid];
    }
    ids = ids_s;
  }
  if ((li.flags & IN_GATHER) && blockIdx.x == 0 && wave == 0)
    wave_softmax_at(li.logits, a.ids, a.E, K, li.w_out, a.err);
  if (lora && blockIdx.x == 0 && tid < K) a.slots[tid] = resolve_slot(a, ids[tid]);
  if (!lora && !router && blockIdx.x == 0 && tid < K) a.slots[tid] = resolve_slot(a, ids[tid]);
  if (!active) return;
  if (router) {
    const float s = pref ? row_dot_pref(pf, x, d) : row_dot<false, false>(wrow, x, d);
    if (lane == 0) li.logits[row] = s;
    return;
  }
  // LoRA A x rows
  const int k = row / (2 * r), p = (row / r) & 1, rr = row % r;
  if (li.flags & IN_TOPK) {
    const int s = resolve_slot(a, ids[k]);
    wrow = s < 0 ? nullptr
                 : reinterpret_cast<const uint16_t*>(E0_LORA_E(a, a.pool + (size_t)s * a.slot_bytes,
                                                               ids[k], p ? 2 : 0,
                                                               p ? a.lay.a_up : a.lay.a_gate)) +
                       (size_t)rr * d;
  }
  float t = 0.f;
  if (wrow != nullptr) {
    t = pref ? row_dot_pref(pf, x, d) : row_dot<false, false>(wrow, x, d);
  } else if (lane == 0) {
    set_error(a.err, EDGE0_ERANGE);
  }
  if (lane == 0) a.t_in[row] = t;
}

// -------------------------------------------------------------- k_gate_up

template <int NJ>
__device__ __forceinline__ void gate_up_wide(const MoeArgs& a, const uint8_t* b, int k, int i0,
                                             float* h_s, float* hrep_s) {
  GuW<NJ> w;
  gu_load<NJ>(a, b, i0, w, tid_here() >> 6, k);
  const int lane = threadIdx.x & 63, r = a.r;
  float tg = 0.f, tu = 0.f;
  if (r > 0 && lane < r) {
    tg = a.t_in[(size_t)(k * 2 + 0) * r + lane];
    tu = a.t_in[(size_t)(k * 2 + 1) * r + lane];
  }
  gu_finish<NJ>(a, w, k, i0, a.x, tg, tu, h_s, hrep_s);
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
    const uint16_t* B =
        reinterpret_cast<const uint16_t*>(E0_LORA(a, b, k, p ? 3 : 1, p ? a.lay.b_up : a.lay.b_gate));
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
__global__ __launch_bounds__(gate_up_threads(CPR)) void k_gate_up(MoeArgs a) {
  __shared__ float h_s[16];
  __shared__ float hrep_s[16];
  const int nblk = a.I / 16;
  const int k = blockIdx.x / nblk;
  const int blk = blockIdx.x % nblk;
  const int i0 = blk * 16;
  const int r = a.r;
  const uint8_t* b = slot_ptr(a, k);
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
        reinterpret_cast<const uint16_t*>(E0_LORA(a, b, k, 4, a.lay.a_down)) + (size_t)threadIdx.x * a.I +
        i0);
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

// ------------------------------------------------------------- k_layer_fused
// A layer's input and gate/up in one launch (wide rows, lora_rank <= 16).
// Two kinds of workgroup:
//  - a.n_prod producers, the first workgroups of the grid (dispatched before
//    any workgroup that waits for them).  Each loads a.prod_rows of the
//    routed experts' LoRA A rows, forms the layer input x like every other
//    workgroup and stores t = A x for its rows into t_hand;
//  - K * d_inter / 16 gate/up workgroups (16 rows of one routed expert):
//    each loads its int4 rows, forms x redundantly from L2-resident data
//    (previous layer's fixed-point y, h, RMSNorm; without IN_NORM x is
//    li.h_prev as given, the single-layer call) into LDS, computes the rows'
//    dot products and stores them, without the LoRA term, to gu_pre.
// The LoRA B t terms and the SwiGLU are the down launch's (down_unit_defer):
// t crosses the kernel boundary, so no workgroup of this launch waits for
// another's stores.
// ROUTE (a router layer): the producers first compute a.route_rows router
// logits each from x and publish them through lg_hand (parity a.par; the
// down kernel that follows empties them again); every workgroup then commits the
// top-K of the published logits itself (wave 0, bounded wait) before it
// loads its expert's rows, and gate/up workgroup 0 stores the committed
// ids/w.  Otherwise the routing (a.ids, a.w) is given and the rows are
// loaded before x is formed.
// Gate/up workgroup 0 clears this layer's accumulator and, in the stack
// (li.x_out given), stores h, y_prev and x; the first workgroup of each
// expert publishes its slot for the down kernel.  One launch replaces the router / layer-input launch and the
// gate/up GEMV, and A x is computed once per expert instead of once per
// workgroup.
constexpr int kFusedMaxRank = 16;
constexpr int kFusedRowsPerWave = 2;  // 8 waves: 16 rows of gate and up per workgroup
constexpr int kFusedMaxExperts = 256;  // slot-table row held in 4 registers per lane
constexpr int kFusedMaxProdRows = 8;   // A rows per producer: 2, 4 or 8
constexpr int kFusedMaxRouteRows = 4;  // router rows per producer
constexpr int kFusedThreads = 512;     // 8 waves

// slot of a (wave-uniform) expert id from the layer's table row held as
// entries l + 64 j in word j of lane l; -1 when the id or the slot is out of
// range
__device__ __forceinline__ int table_slot(int t0, int t1, int t2, int t3, int expert, int E,
                                          int n_slots) {
  const int ec = min(max(expert, 0), E - 1);
  const int hi = ec >> 6;
  const int v = hi == 0 ? t0 : hi == 1 ? t1 : hi == 2 ? t2 : t3;
  const int slot = __builtin_amdgcn_readlane(v, ec & 63);
  return (expert < 0 || expert >= E || slot < 0 || slot >= n_slots) ? -1 : slot;
}

template <int NJ, bool ROUTE>
__global__ __launch_bounds__(kFusedThreads) void k_layer_fused(MoeArgs a, LayerIn li) {
  constexpr int PER = 4 * NJ;  // hidden elements per thread (d = 2048 NJ, 512 threads)
  constexpr int RW = kFusedRowsPerWave, ROWS = 8 * RW;  // rows per workgroup
  constexpr int MU = kFusedMaxProdRows * NJ / 2;        // producer: A pieces per thread (max)
  constexpr int MR = (kFusedMaxRouteRows * NJ + 1) / 2;  // producer: router pieces per thread
  __shared__ uint16_t xs[2048 * NJ];
  __shared__ float red[8];
  __shared__ float redp[MU][8];
  __shared__ int32_t ids_w[16];
  __shared__ float w_w[16];
  __shared__ float lg_s[ROUTE ? kFusedMaxExperts : 1];
  // The arguments the start depends on, in one batch of scalar loads: left
  // to itself the compiler loads them group by group behind the branches
  // that need them, a dependent round trip each before the first memory
  // load of the workgroup goes out.
  asm volatile("" ::"s"(a.d), "s"(a.r), "s"(a.I), "s"(a.K), "s"(a.E), "s"(a.n_prod),
               "s"(a.prod_rows), "s"(a.n_slots), "s"(li.flags), "s"(a.route_rows),
               "s"((int)a.lora_sep));
  asm volatile("" ::"s"(a.table), "s"(a.pool), "s"(a.slot_bytes), "s"(a.ids), "s"(a.acc_prev),
               "s"(li.h_prev), "s"(a.lay.gate_q), "s"(a.lay.up_q), "s"(a.lay.gate_s),
               "s"(a.lay.gate_b), "s"(a.lay.up_s), "s"(a.lay.up_b));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = a.d, r = a.r;
  const int nwg = a.I / ROWS;
  const int P = a.n_prod;
  const bool prod = (int)blockIdx.x < P;
  const bool comb = (li.flags & IN_COMBINE) != 0;
  // XCD-aware order of the gate/up workgroups: consecutive workgroups go to
  // different XCDs (round-robin over 8; P is a multiple of 8), so logical
  // block L = (id % 8) * (n / 8) + id / 8 gives each XCD a contiguous range
  // of an expert's blocks
  int k, lb = 0;
  if (prod) {
    k = r > 0 ? (int)blockIdx.x * a.prod_rows / (2 * r) : a.K;  // K: no LoRA rows
    const bool routes = ROUTE && (int)blockIdx.x * a.route_rows < a.E;
    if (k >= a.K && !routes) return;  // padding producer
  } else {
    const int id = blockIdx.x - P, gsz = gridDim.x - P;
    lb = (gsz % 8 == 0) ? (id % 8) * (gsz / 8) + id / 8 : id;
    k = lb / nwg;
  }
  const int i0 = (lb % nwg) * ROWS;
  const int nblk = a.I / 16;
  const int blk = i0 / 16;  // first 16-row block of the workgroup
  // 0. the layer's slot-table row (E <= 256), lane l holding entries
  // l + 64 j: issued first, so resolving the routed expert's slot below is
  // a register read rather than one more dependent memory round trip
  int32_t tbl[kFusedMaxExperts / 64];
#pragma unroll
  for (int j = 0; j < kFusedMaxExperts / 64; ++j) tbl[j] = a.table[min(lane + 64 * j, a.E - 1)];
  // 1. the prologue's loads: h_prev and the previous layer's fixed-point y,
  // written by other workgroups (other XCDs) just before; few wide requests.
  // Thread tid owns elements j = 4 (tid + 512 c) + e, c < NJ, e < 4.
  uint2 hq[NJ];  // h_prev words (bf16 pairs)
  unsigned long long av[PER];
#pragma unroll
  for (int c = 0; c < NJ; ++c) {
    const int j0 = 4 * (tid + 512 * c);
    hq[c] = *reinterpret_cast<const uint2*>(li.h_prev + j0);
    const ulonglong2 a0 = *reinterpret_cast<const ulonglong2*>(a.acc_prev + j0);
    const ulonglong2 a1 = *reinterpret_cast<const ulonglong2*>(a.acc_prev + j0 + 2);
    av[4 * c + 0] = a0.x;
    av[4 * c + 1] = a0.y;
    av[4 * c + 2] = a1.x;
    av[4 * c + 3] = a1.y;
  }
  // 2. the routed expert's bundle; an invalid slot reads slot 0 and its
  // results are discarded
  // (the table words are passed by value: an array captured by a lambda is
  // placed in LDS by the compiler)
  int slot = -1, eid = 0;  // eid: the routed expert (for adapters given apart)
  bool ok = false;
  const uint8_t* b = a.pool;
  const int t0 = tbl[0], t1 = tbl[1], t2 = tbl[2], t3 = tbl[3];
  static_assert(kFusedMaxExperts == 256, "four table words per lane");
  auto resolve = [&](int expert) {
    eid = expert;
    slot = table_slot(t0, t1, t2, t3, expert, a.E, a.n_slots);
    ok = slot >= 0;
    b = a.pool + (size_t)(ok ? slot : 0) * (size_t)a.slot_bytes;
  };
  if constexpr (!ROUTE) resolve(a.ids[min(k, a.K - 1)]);

  // 3. combine, residual, RMSNorm -> x in LDS; `lead` stores h, y_prev, x
  // and clears the accumulator
  auto form_x = [&](bool lead) {
    // the prologue's loaded values enter through an empty asm, so the
    // compiler cannot hoist their first use (and its wait) above the weight
    // loads issued in between
#pragma unroll
    for (int c = 0; c < NJ; ++c) asm volatile("" : "+v"(hq[c].x), "+v"(hq[c].y));
#pragma unroll
    for (int m = 0; m < PER; ++m) asm volatile("" : "+v"(av[m]));
    float hv[PER];
    float ss = 0.f;
    uint32_t hb[PER];
#pragma unroll
    for (int c = 0; c < NJ; ++c) {
      hb[4 * c + 0] = hq[c].x & 0xFFFFu;
      hb[4 * c + 1] = hq[c].x >> 16;
      hb[4 * c + 2] = hq[c].y & 0xFFFFu;
      hb[4 * c + 3] = hq[c].y >> 16;
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const uint32_t yb = comb ? f2bf(from_fix(av[m])) : 0u;
      hv[m] = bf2f(f2bf(bf2f(hb[m]) + bf2f(yb)));
      ss = fmaf(hv[m], hv[m], ss);
      av[m] = yb;  // keep y_prev's bits for the stores below
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w8 = 0; w8 < 8; ++w8) tot += red[w8];
    // without IN_NORM x is h itself (the single-layer call's given input)
    const float inv = (li.flags & IN_NORM) ? 1.f / sqrtf(tot / (float)d + li.eps) : 1.f;
    uint32_t xw[2 * NJ];
#pragma unroll
    for (int c = 0; c < NJ; ++c) {
      xw[2 * c] = f2bf(hv[4 * c] * inv) | (f2bf(hv[4 * c + 1] * inv) << 16);
      xw[2 * c + 1] = f2bf(hv[4 * c + 2] * inv) | (f2bf(hv[4 * c + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(xs + 4 * (tid + 512 * c)) = make_uint2(xw[2 * c], xw[2 * c + 1]);
    }
    __syncthreads();
    if (lead) {
      if (li.x_out != nullptr) {  // the stack's copies of x, y_prev and h
#pragma unroll
        for (int c = 0; c < NJ; ++c) {
          const int j0 = 4 * (tid + 512 * c);
          *reinterpret_cast<uint2*>(li.x_out + j0) = make_uint2(xw[2 * c], xw[2 * c + 1]);
          if (comb)
            *reinterpret_cast<uint2*>(li.y_prev_out + j0) =
                make_uint2((uint32_t)av[4 * c] | ((uint32_t)av[4 * c + 1] << 16),
                           (uint32_t)av[4 * c + 2] | ((uint32_t)av[4 * c + 3] << 16));
          *reinterpret_cast<uint2*>(li.h_out + j0) =
              make_uint2(f2bf(hv[4 * c]) | (f2bf(hv[4 * c + 1]) << 16),
                         f2bf(hv[4 * c + 2]) | (f2bf(hv[4 * c + 3]) << 16));
        }
      }
      for (int j = tid; j < d; j += 512) a.acc[j] = 0ull;
    }
  };

  // ROUTE: the top-K of the producers' published logits (wave 0 polls them
  // into LDS, bounded), committed by every workgroup itself
  auto route = [&]() {
    if (wave == 0) {
      const float* src = a.lg_hand + (size_t)a.par * a.E;
      constexpr int NL = kFusedMaxExperts / 64;
      uint32_t v[NL];
      int64_t n = 0;
      for (;;) {
#pragma unroll
        for (int j = 0; j < NL; ++j)
          v[j] = lane + 64 * j < a.E ? __float_as_uint(ld_dev(src + lane + 64 * j)) : 0u;
        bool miss = false;
#pragma unroll
        for (int j = 0; j < NL; ++j) miss |= v[j] == kTHandEmpty;
        if (!__any(miss)) break;
        if (++n >= a.spin) {
          set_error(a.err, EDGE0_EHIP);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int j = 0; j < NL; ++j)
        if (lane + 64 * j < a.E) lg_s[lane + 64 * j] = __uint_as_float(v[j]);
      __builtin_amdgcn_wave_barrier();
      if (a.E <= 128)
        wave_topk_n<2, false>(lg_s, a.E, a.K, ids_w, w_w);
      else
        wave_topk_n<kFusedMaxExperts / 64, false>(lg_s, a.E, a.K, ids_w, w_w);  // E <= 256
    }
    __syncthreads();
  };

  if (prod) {
    if constexpr (ROUTE) {
      // router rows e0 .. e0 + RR - 1: piece u = tid + 512 m of the
      // concatenated rows is 8 bf16 (row u / (d / 8)); a wave's 64 pieces
      // lie in one row
      const int RR = a.route_rows, e0 = (int)blockIdx.x * RR;
      const int nr = max(0, min(RR, a.E - e0)), nu = nr * d / 8;
      uint4 rp[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int u = min(tid + 512 * m, max(nu - 1, 0));
        rp[m] = reinterpret_cast<const uint4*>(li.w_router + (size_t)min(e0, a.E - 1) * d)[u];
      }
      form_x(false);
      const uint4* xv = reinterpret_cast<const uint4*>(xs);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int u = tid + 512 * m;
        if (512 * m < nu) {  // uniform over each wave
          const uint4 xq4 = xv[u % (d / 8)];
          float p = u < nu ? dot2bf(rp[m].x, xq4.x, 0.f) : 0.f;
          if (u < nu) {
            p = dot2bf(rp[m].y, xq4.y, p);
            p = dot2bf(rp[m].z, xq4.z, p);
            p = dot2bf(rp[m].w, xq4.w, p);
          }
          p = wave_sum(p);
          if (lane == 0) redp[m][wave] = p;
        }
      }
      __syncthreads();
      if (tid < nr) {
        float l = 0.f;
        for (int m = 0; 512 * m < nu; ++m)
          for (int w8 = 0; w8 < 8; ++w8)
            if ((512 * m + 64 * w8) / (d / 8) == tid) l += redp[m][w8];
        if (__float_as_uint(l) == kTHandEmpty) l = __uint_as_float(0x7FC00000u);
        st_dev(a.lg_hand + (size_t)a.par * a.E + e0 + tid, l);
        st_dev(a.lg_hand + (size_t)(1 - a.par) * a.E + e0 + tid, __uint_as_float(kTHandEmpty));
      }
      if (k >= a.K) return;  // router rows only
      route();
      resolve(ids_w[k]);
    }
    // LoRA producer: rows tr0 .. tr0 + RP - 1 of the expert's 2r A rows
    // (gate rows, then up rows).  Piece u = tid + 512 m of the concatenated
    // rows is 8 bf16: row u / (d / 8), position u % (d / 8); a wave's 64
    // pieces lie in one row.
    const int RP = a.prod_rows, nu = RP * d / 8;
    const int tr0 = ((int)blockIdx.x * RP) % (2 * r);
    uint4 ap[MU];
#pragma unroll
    for (int m = 0; m < MU; ++m) {
      const int u = min(tid + 512 * m, nu - 1);  // past nu: repeats of the last piece
      const int tr = tr0 + u / (d / 8);
      const uint4* row = reinterpret_cast<const uint4*>(
                             E0_LORA_E(a, b, eid, tr < r ? 0 : 2,
                                       tr < r ? a.lay.a_gate : a.lay.a_up)) +
                         (size_t)(tr % r) * (d / 8);
      ap[m] = row[u % (d / 8)];
    }
    if constexpr (!ROUTE) form_x(false);
    const uint4* xv = reinterpret_cast<const uint4*>(xs);
#pragma unroll
    for (int m = 0; m < MU; ++m) {
      const int u = tid + 512 * m;
      if (512 * m < nu) {  // uniform over each wave
        const uint4 xq4 = xv[u % (d / 8)];
        float p = dot2bf(ap[m].x, xq4.x, 0.f);
        p = dot2bf(ap[m].y, xq4.y, p);
        p = dot2bf(ap[m].z, xq4.z, p);
        p = dot2bf(ap[m].w, xq4.w, p);
        p = wave_sum(p);
        if (lane == 0) redp[m][wave] = p;
      }
    }
    __syncthreads();
    if (tid < RP) {
      float t = 0.f;
      for (int m = 0; 512 * m < nu; ++m)
        for (int w8 = 0; w8 < 8; ++w8)
          if ((512 * m + 64 * w8) / (d / 8) == tid) t += redp[m][w8];
      a.t_hand[(size_t)k * 2 * r + tr0 + tid] = ok ? t : 0.f;
    }
    return;
  }

  // gate/up workgroup: every weight load (HBM) and x; a routed layer loads
  // the rows once its top-K is committed
  GuW<NJ, RW> gw;
  if constexpr (ROUTE) {
    form_x(lb == 0);
    route();
    resolve(ids_w[k]);
    if (lb == 0 && tid < a.K) {
      li.ids_out[tid] = ids_w[tid];
      li.w_out[tid] = w_w[tid];
    }
    gu_load<NJ, RW>(a, b, i0, gw, wave, 0, eid);
  } else {
    gu_load<NJ, RW>(a, b, i0, gw, wave, 0, eid);
    form_x(lb == 0);
  }
  if (blk == 0 && tid == 0) {
    a.slots[k] = ok ? slot : -1;
    if (!ok) set_error(a.err, EDGE0_ERANGE);
  }
  // 4. the rows' dot products on x from LDS; lane (64 / 2RW) ii of the wave
  // holds gate row ii, lane 32 + (64 / 2RW) ii its up row.  An invalid slot
  // stores zeros (its producers store t = 0, so its h is 0).
  float v[2 * RW];
  gu_base<NJ, RW>(gw, xs, v);
  const float s1 = wave_sums_2r<RW>(v);
  constexpr int kSpan = 64 / (2 * RW);
  if ((lane & 31) % kSpan == 0) {
    const int ii = (lane & 31) / kSpan, half = lane >> 5;
    a.gu_pre[((size_t)k * 2 + half) * a.I + i0 + RW * wave + ii] = ok ? s1 : 0.f;
  }
}

// ------------------------------------------------------------------ k_down
// Unit (rb, sl): rows 64 rb .. 64 rb + 63 over input chunks of slice sl, for
// all K experts, each tile's contribution weighted by w_k.  The LoRA-down
// delta is linear in t_down = A_down h = sum over chunks of the chunk's part,
// so each tile (k, c) also adds (alpha/r) w_k B_down[o] . (A_down h)_c: every
// unit carries an equal share of it.  The partial row is added to the layer's
// fixed-point accumulator (exact, order-independent).
// The unit's nt = K * ncs tiles (expert-major) are split into contiguous runs
// of TPW tiles per wave; every address is wave-uniform scalar arithmetic so
// all of a wave's tile loads are in flight together.  An expert whose slot is
// invalid reads slot 0 with weight 0 (never an out-of-range address).
constexpr int kMaxSliceChunks = 64;  // expert-chunks per unit staged in LDS
constexpr int kMaxDeferT = 16 * 2 * kFusedMaxRank;  // t of up to 16 routed experts

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One down unit: workgroup `bid` of the (d / 64) * S units.
template <int TPW>
__device__ __forceinline__ void down_unit(const MoeArgs& a, const unsigned bid) {
  __shared__ float red[4][64];
  __shared__ uint32_t hp_s[kMaxSliceChunks][32];  // hi pairs then lo pairs of each chunk
  __shared__ float hsum_s[kMaxSliceChunks];
  __shared__ float tdc_s[kMaxSliceChunks][64];    // per tile: the chunk's part of A_down h
  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int K = a.K, S = a.S, I = a.I, r = a.r, d = a.d;
  const int NC = I / 32;
  const int rb = bid / S;
  const int sl = bid % S;
  const int cps = (NC + S - 1) / S;
  const int c0 = sl * cps;
  const int ncs = min(NC, c0 + cps) - c0;
  const int nt = K * ncs;
  const int o = rb * 64 + lane;
  // this wave's tiles: t = wave * TPW + m
  uint4 q[TPW];
  uint32_t sv[TPW], bv[TPW];
  float wt[TPW];
  constexpr int kBd = 2;  // B_down pieces (8 ranks each) held per tile; more are read in the loop
  uint4 bdq[TPW][kBd];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int t = wave * TPW + m;
    const bool valid = t < nt;
    const int tc = valid ? t : 0;
    const int kk = tc / ncs, c = c0 + tc % ncs;
    int slot = a.slots[kk];
    const bool ok = slot >= 0 && slot < a.n_slots;
    wt[m] = (valid && ok) ? a.w[kk] : 0.f;
    slot = ok ? slot : 0;
    const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
    q[m] = reinterpret_cast<const uint4*>(b + a.lay.down_q)[((size_t)rb * NC + c) * 64 + lane];
    const int grp = (32 * c) / a.g;
    sv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_s)[(size_t)grp * d + o];
    bv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_b)[(size_t)grp * d + o];
    // B_down row o of the tile's expert (r bf16; an in-bundle word when r = 0)
    const uint4* Bdp = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(r > 0 ? E0_LORA(a, b, kk, 5, a.lay.b_down) : b) +
        (size_t)o * r);
#pragma unroll
    for (int j = 0; j < kBd; ++j) bdq[m][j] = (8 * j < r) ? Bdp[j] : make_uint4(0, 0, 0, 0);
  }
  // stage the unit's activation pairs and chunk sums (all K experts) in LDS
  {
    constexpr int kStage = kMaxSliceChunks * 32 / 256;  // words per thread
    uint32_t st[kStage];
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int t = threadIdx.x + 256 * m;
      if (t < nt * 32) {
        const int tt = t >> 5, j = t & 31;
        const int kk = tt / ncs, c = c0 + tt % ncs;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(j < 16 ? a.hp_hi : a.hp_lo) +
                              (size_t)kk * (I / 2);
        st[m] = src[16 * c + (j & 15)];
      }
    }
    float h0v = 0.f, h1v = 0.f;
    const int tt = threadIdx.x;
    if (tt < nt) {
      const int kk = tt / ncs, c = c0 + tt % ncs;
      const float* hs = a.hs + (size_t)kk * (I / 16);
      h0v = hs[2 * c];
      h1v = hs[2 * c + 1];
    }
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int t = threadIdx.x + 256 * m;
      if (t < nt * 32) hp_s[t >> 5][t & 31] = st[m];
    }
    if (tt < nt) hsum_s[tt] = h0v + h1v;
    // each tile's chunk part of A_down h: its two 16-row partials
    for (int e = threadIdx.x; e < nt * r; e += 256) {
      const int te = e / r, rr = e % r;
      const int kk = te / ncs, c = c0 + te % ncs;
      const float* tp = a.tdpart + ((size_t)kk * (I / 16) + 2 * c) * r;
      tdc_s[te][rr] = tp[rr] + tp[r + rr];
    }
  }
  if (bid == 0) {
    if (threadIdx.x < (unsigned)K) {
      const int slot = a.slots[threadIdx.x];
      if (slot < 0 || slot >= a.n_slots) set_error(a.err, EDGE0_ERANGE);
    }
    // the router logits the layer kernel before this one read, if it was a
    // router layer: empty them for the next
    if (a.lg_consumed != nullptr)
      for (int i = threadIdx.x; i < a.E; i += 256) a.lg_consumed[i] = __uint_as_float(kTHandEmpty);
  }
  __syncthreads();  // every thread, unconditionally
  float part = 0.f;
  const Q4Consts kq = q4_consts();
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int t = wave * TPW + m;
    if (t < nt) {
      const float s = bf2f(sv[m]), bb = bf2f(bv[m]);
      const uint32_t* hp = hp_s[t];
      const float acc = chunk_dot128(q[m], hp, kq) + chunk_dot128(q[m], hp + 16, kq);
      float dl = 0.f;  // B_down[o] . (A_down h)_c
      for (int j = 0; 8 * j < r; ++j) {
        uint4 bw4;
        if (j < kBd) {
          bw4 = bdq[m][j];
        } else {
          const int kk = t / ncs;
          int slot = a.slots[kk];
          slot = (slot >= 0 && slot < a.n_slots) ? slot : 0;
          bw4 = reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(
                  E0_LORA(a, a.pool + (size_t)slot * a.slot_bytes, kk, 5, a.lay.b_down)) +
              (size_t)o * r)[j];
        }
        const uint32_t bw[4] = {bw4.x, bw4.y, bw4.z, bw4.w};
        const float4 t0 = *reinterpret_cast<const float4*>(&tdc_s[t][8 * j]);
        const float4 t1 = *reinterpret_cast<const float4*>(&tdc_s[t][8 * j + 4]);
        const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          dl += bf_lo(bw[q2]) * tv[2 * q2];
          dl += bf_hi(bw[q2]) * tv[2 * q2 + 1];
        }
      }
      part += wt[m] * (s * acc + (bb - 128.f * s) * hsum_s[t] + a.scale * dl);
    }
  }
  red[wave][lane] = part;
  __syncthreads();
  if (wave == 0)
    atomicAdd(a.acc + o, to_fix(red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane]));
}

// One down unit after the fused layer kernel, whose gate/up rows (gu_pre)
// still lack their LoRA terms.  Same unit and tiles as down_unit; before its
// tiles the unit finishes its chunks' rows of h: each wave takes its own
// tiles, lane j < 32 row j of the chunk's gate and lane 32 + j its up row,
// adds scale * B[row] . t (t = A x of the expert, from t_hand), and lane j
// forms h = SiLU(gate) * up, its hi/lo split and the chunk sum; then lane
// (qq, rr) forms A_down[rr][8 qq ..] . h, the chunk's part of A_down h.
// Order of the loads: the arguments in one batch, then what needs no slot
// (gu_pre, t), then the slot-dependent rows; the LoRA rows are read at
// clamped in-row addresses and zeroed past the rank instead of behind
// branches (r = 0, 8 or 16).
template <int TPW>
__device__ __forceinline__ void down_unit_defer(const MoeArgs& a, const unsigned bid) {
  __shared__ float red[4][64];
  __shared__ uint32_t hp_s[4 * TPW][32];  // hi pairs then lo pairs of each chunk
  __shared__ float hf_s[4 * TPW][32];     // each chunk's h rows (fp32)
  __shared__ float hsum_s[4 * TPW];
  __shared__ float tdc_s[4 * TPW][kFusedMaxRank];  // per tile: the chunk's part of A_down h
  __shared__ float tt_s[kMaxDeferT];                // t of the K experts, zero past K * 2r
  asm volatile("" ::"s"(a.K), "s"(a.S), "s"(a.I), "s"(a.r), "s"(a.d), "s"(a.g), "s"(a.n_slots),
               "s"(a.E), "s"((int)a.lora_sep));
  asm volatile("" ::"s"(a.slots), "s"(a.w), "s"(a.pool), "s"(a.slot_bytes), "s"(a.gu_pre),
               "s"(a.t_hand), "s"(a.ids));
  asm volatile("" ::"s"(a.lay.down_q), "s"(a.lay.down_s), "s"(a.lay.down_b), "s"(a.lay.b_down),
               "s"(a.lay.b_gate), "s"(a.lay.b_up), "s"(a.lay.a_down));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int K = a.K, S = a.S, I = a.I, r = a.r, d = a.d;
  const int NC = I / 32;
  const int rb = bid / S;
  const int sl = bid % S;
  const int cps = (NC + S - 1) / S;
  const int c0 = sl * cps;
  const int ncs = min(NC, c0 + cps) - c0;
  const int nt = K * ncs;
  const int o = rb * 64 + lane;
  const int half = lane >> 5, j32 = lane & 31;  // gate (0) or up (1) row j32 of a chunk
  const int rr = lane & 15, qq = lane >> 4;     // A_down rank rr, rows 8 qq .. 8 qq + 7
  const int p1 = r > 8 ? 1 : 0;                 // second 8-rank piece of a LoRA row, if any
  const int rrc = min(rr, max(r - 1, 0));
  // 1. what the previous launch wrote and needs no slot: the tiles' gate/up
  // rows and t (two entries per thread cover kMaxDeferT)
  int kk_m[TPW], c_m[TPW];
  float gu[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int t = wave * TPW + m;
    const int tc = t < nt ? t : 0;
    kk_m[m] = tc / ncs;
    c_m[m] = c0 + tc % ncs;
    gu[m] = a.gu_pre[((size_t)kk_m[m] * 2 + half) * I + 32 * c_m[m] + j32];
  }
  const int nT = K * 2 * r;
  const float tv0 = a.t_hand[min(tid, max(nT - 1, 0))];
  const float tv1 = a.t_hand[min(tid + 256, max(nT - 1, 0))];
  // 2. each tile's slot, then its rows
  uint4 q[TPW], bg[TPW][2], ad[TPW], bd[TPW][2];
  uint32_t sv[TPW], bv[TPW];
  float wt[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int t = wave * TPW + m;
    const int kk = kk_m[m], c = c_m[m];
    int slot = a.slots[kk];
    const int eid = a.ids[kk];  // the expert, for adapters given apart
    const float wk = a.w[kk];
    const bool ok = slot >= 0 && slot < a.n_slots;
    wt[m] = (t < nt && ok) ? wk : 0.f;
    slot = ok ? slot : 0;
    const uint8_t* b = a.pool + (size_t)slot * (size_t)a.slot_bytes;
    const uint8_t* bgp =
        r > 0 ? E0_LORA_E(a, b, eid, half ? 3 : 1, half ? a.lay.b_up : a.lay.b_gate) : b;
    const uint8_t* adp = r > 0 ? E0_LORA_E(a, b, eid, 4, a.lay.a_down) : b;
    const uint8_t* bdp = r > 0 ? E0_LORA_E(a, b, eid, 5, a.lay.b_down) : b;
    const uint4* Bg = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(bgp) + (size_t)(32 * c + j32) * r);
    bg[m][0] = Bg[0];
    bg[m][1] = Bg[p1];
    ad[m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(adp) +
                                            (r > 0 ? (size_t)rrc * I + 32 * c + 8 * qq : 0));
    const uint4* Bd =
        reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(bdp) + (size_t)o * r);
    bd[m][0] = Bd[0];
    bd[m][1] = Bd[p1];
    q[m] = reinterpret_cast<const uint4*>(b + a.lay.down_q)[((size_t)rb * NC + c) * 64 + lane];
    const int grp = (32 * c) / a.g;
    sv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_s)[(size_t)grp * d + o];
    bv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_b)[(size_t)grp * d + o];
  }
  // the pieces past the rank count as zeros (masked where they are used, so
  // no branch waits for the loads here)
  const uint32_t mk0 = r > 0 ? ~0u : 0u, mk1 = r > 8 ? ~0u : 0u, mka = rr < r ? ~0u : 0u;
  tt_s[tid] = tid < nT ? tv0 : 0.f;
  tt_s[tid + 256] = tid + 256 < nT ? tv1 : 0.f;
  __syncthreads();
  // 3. the tiles' rows of h
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int tl = wave * TPW + m;
    const float* tv = tt_s + (size_t)kk_m[m] * 2 * r + half * r;
    const uint32_t bw[8] = {bg[m][0].x & mk0, bg[m][0].y & mk0, bg[m][0].z & mk0,
                            bg[m][0].w & mk0, bg[m][1].x & mk1, bg[m][1].y & mk1,
                            bg[m][1].z & mk1, bg[m][1].w & mk1};
    float dl = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2) {
      dl += bf_lo(bw[q2]) * tv[2 * q2];
      dl += bf_hi(bw[q2]) * tv[2 * q2 + 1];
    }
    const float pre = gu[m] + a.scale * dl;
    const float up = __shfl_xor(pre, 32, kWave);
    const float h = silu_f(pre) * up;  // lanes j < 32
    const uint32_t hi = f2bf(h);
    const uint32_t lo = f2bf(h - bf2f(hi));
    float hr = half == 0 ? bf2f(hi) + bf2f(lo) : 0.f;
    if (half == 0) {
      const int pos = pair_pos(j32);
      uint16_t* hp16 = reinterpret_cast<uint16_t*>(hp_s[tl]);
      hp16[pos] = (uint16_t)hi;
      hp16[32 + pos] = (uint16_t)lo;
      hf_s[tl][j32] = h;
    }
    hr = wave_sum(hr);
    if (lane == 0) hsum_s[tl] = hr;
  }
  __syncthreads();
  // 4. each tile's chunk part of A_down h (zero for ranks past r)
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int tl = wave * TPW + m;
    const float* hq = hf_s[tl] + 8 * qq;
    const uint32_t aw[4] = {ad[m].x & mka, ad[m].y & mka, ad[m].z & mka, ad[m].w & mka};
    float sm = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) sm += bf_lo(aw[q2]) * hq[2 * q2] + bf_hi(aw[q2]) * hq[2 * q2 + 1];
    sm += __shfl_xor(sm, 16, kWave);
    sm += __shfl_xor(sm, 32, kWave);
    if (qq == 0) tdc_s[tl][rr] = sm;
  }
  if (bid == 0) {
    if (tid < K) {
      const int slot = a.slots[tid];
      if (slot < 0 || slot >= a.n_slots) set_error(a.err, EDGE0_ERANGE);
    }
    // the router logits the layer kernel before this one read, if it was a
    // router layer: empty them for the next
    if (a.lg_consumed != nullptr)
      for (int i = tid; i < a.E; i += 256) a.lg_consumed[i] = __uint_as_float(kTHandEmpty);
  }
  __syncthreads();
  // 5. the tiles: each adds w_k (s acc + (b - 128 s) sum h + scale B_down[o] . (A_down h)_c)
  float part = 0.f;
  const Q4Consts kq = q4_consts();
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int tl = wave * TPW + m;
    if (tl < nt) {
      const float s = bf2f(sv[m]), bb = bf2f(bv[m]);
      const uint32_t* hp = hp_s[tl];
      const float acc = chunk_dot128(q[m], hp, kq) + chunk_dot128(q[m], hp + 16, kq);
      const uint32_t bw[8] = {bd[m][0].x & mk0, bd[m][0].y & mk0, bd[m][0].z & mk0,
                              bd[m][0].w & mk0, bd[m][1].x & mk1, bd[m][1].y & mk1,
                              bd[m][1].z & mk1, bd[m][1].w & mk1};
      float dl = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < 8; ++q2) {
        dl += bf_lo(bw[q2]) * tdc_s[tl][2 * q2];
        dl += bf_hi(bw[q2]) * tdc_s[tl][2 * q2 + 1];
      }
      part += wt[m] * (s * acc + (bb - 128.f * s) * hsum_s[tl] + a.scale * dl);
    }
  }
  red[wave][lane] = part;
  __syncthreads();
  if (wave == 0)
    atomicAdd(a.acc + o, to_fix(red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane]));
}

template <int TPW, bool DEFER>
__global__ __launch_bounds__(256) void k_down(MoeArgs a) {
  if constexpr (DEFER)
    down_unit_defer<TPW>(a, blockIdx.x);
  else
    down_unit<TPW>(a, blockIdx.x);
}

// The same launch with one prerouter head's fc1 rows beside it (the stack's
// folded head schedule): row y = 0 of the grid runs the head's workgroups
// (dispatched first, so their loads go out before the units'), row y = 1 the
// down units.  The role comes from the workgroup id alone, so no argument
// load stands between a unit's start and its weight loads.
template <int TPW, bool DEFER>
__global__ __launch_bounds__(256) void k_down_fc1(MoeArgs a, HeadPart h) {
  if (blockIdx.y == 0) {
    if ((int)blockIdx.x < h.n_wg) head_fc1_row(h, blockIdx.x * kHeadFc1Rows + (threadIdx.x >> 6));
    return;
  }
  if ((int)blockIdx.x >= (a.d / 64) * a.S) return;
  if constexpr (DEFER)
    down_unit_defer<TPW>(a, blockIdx.x);
  else
    down_unit<TPW>(a, blockIdx.x);
}

// y = bf16 of the layer's fixed-point accumulator; optional residual
// h_out = bf16(h_res + y).  (In the stack the next layer's k_layer_in does it.)
__global__ __launch_bounds__(256) void k_combine(MoeArgs a) { combine_unit(a, blockIdx.x); }

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
// The single-layer call's launches.  Wide rows (layer_fused_ok): the fused
// layer kernel with x as given (no residual, no RMSNorm) and the down launch
// that finishes its gate/up rows; otherwise the LoRA A x launch, the gate/up
// and down GEMVs.  Then the combine (y, and the error word for err_out).
static int launch_layer_call(const MoeArgs& a, hipStream_t stream) {
  int rc;
  if (layer_fused_ok(a)) {
    LayerIn li{};
    li.flags = IN_LORA;
    li.h_prev = a.x;
    if ((rc = launch_layer_fused(a, li, stream)) != EDGE0_OK ||
        (rc = launch_down(a, stream, nullptr, nullptr, true)) != EDGE0_OK)
      return rc;
  } else {
    LayerIn li{};
    li.flags = IN_LORA;  // with r = 0 it only resolves the slots
    if ((rc = launch_layer_in(a, li, stream)) != EDGE0_OK) return rc;
    if ((rc = launch_expert_gemvs(a, stream)) != EDGE0_OK) return rc;
  }
  return launch_combine(a, stream);
}

int fill_moe_args(const edge0_moe_shape* sh, const edge0_slot_pool* pool, const int32_t* table,
                  const int32_t* ids, const float* w, const void* x, void* y, void* workspace,
                  MoeArgs* a, bool lora_in_bundle) {
  edge0_bundle_layout lay, lay_pool;
  edge0_moe_shape s0 = *sh;
  if (!lora_in_bundle) s0.lora_rank = 0;  // the bundles hold the int4 arrays only
  if (bundle_layout(sh, &lay) != EDGE0_OK || bundle_layout(&s0, &lay_pool) != EDGE0_OK)
    return EDGE0_EINVAL;
  if (!pool || !pool->base || pool->n_slots <= 0 || pool->slot_bytes < lay_pool.bytes ||
      pool->slot_bytes % 256 != 0 || !table || !ids || !w || !workspace)
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
  a->t_hand = reinterpret_cast<float*>(ws + L.t_hand);
  a->n_prod = 0;
  a->prod_rows = 0;
  a->lg_hand = reinterpret_cast<float*>(ws + L.lg_hand);
  a->route_rows = 0;
  a->par = 0;
  a->lg_consumed = nullptr;
  a->lora_sep = false;
  a->lo_stride = 0;
  for (auto& p : a->lo_base) p = nullptr;
  a->err_out = nullptr;
  a->spin = kFusedDefaultSpin;
  a->gu_pre = reinterpret_cast<float*>(ws + L.gu_pre);
  a->hp_hi = reinterpret_cast<uint16_t*>(ws + L.hp_hi);
  a->hp_lo = reinterpret_cast<uint16_t*>(ws + L.hp_lo);
  a->hs = reinterpret_cast<float*>(ws + L.hs);
  a->tdpart = reinterpret_cast<float*>(ws + L.tdpart);
  a->slots = reinterpret_cast<int32_t*>(ws + L.slots);
  a->acc = reinterpret_cast<unsigned long long*>(ws + L.acc);
  a->acc_prev = a->acc + a->d;
  // down units: 64-row blocks x input slices, about 256 of them, and a
  // unit's expert-chunks fit the LDS stage
  const int RB = a->d / 64, NC = a->I / 32;
  int S = (768 + RB - 1) / RB;
  S = S < 1 ? 1 : (S > NC ? NC : S);
  while ((a->K * ((NC + S - 1) / S)) > kMaxSliceChunks && S < NC) ++S;
  a->S = S;
  if ((a->K * ((NC + S - 1) / S) + 3) / 4 > 16) return EDGE0_EINVAL;
  return EDGE0_OK;
}

#define E0_MARK(kind, is_start)                                                 \
  do {                                                                         \
    if (timing && timing->which == (kind))                                     \
      (void)hipEventRecord((is_start) ? timing->start : timing->stop, stream); \
  } while (0)

int launch_layer_in(const MoeArgs& a, const LayerIn& li, hipStream_t stream,
                    const LaunchTiming* timing) {
  const int rows = (li.flags & IN_ROUTER) ? a.E : ((li.flags & IN_LORA) ? a.K * 2 * a.r : 0);
  E0_MARK(3, true);
  const int grid = rows > 0 ? (rows + 3) / 4 : 1;
  switch (a.d / 256) {
    case 1: k_layer_in<1><<<grid, 256, 0, stream>>>(a, li); break;
    case 2: k_layer_in<2><<<grid, 256, 0, stream>>>(a, li); break;
    case 4: k_layer_in<4><<<grid, 256, 0, stream>>>(a, li); break;
    case 8: k_layer_in<8><<<grid, 256, 0, stream>>>(a, li); break;
    case 16: k_layer_in<16><<<grid, 256, 0, stream>>>(a, li); break;
    case 24: k_layer_in<24><<<grid, 256, 0, stream>>>(a, li); break;
    case 32: k_layer_in<32><<<grid, 256, 0, stream>>>(a, li); break;
    default: return EDGE0_EINVAL;
  }
  E0_CHECK_LAUNCH();
  E0_MARK(3, false);
  return EDGE0_OK;
}

int launch_expert_gemvs(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing,
                        const HeadPart* fc1) {
  const int cpr = a.d / 32;
  const int grid2 = a.K * (a.I / 16);
  if (timing && timing->which == 1 && cpr == 64) {
    // measured launch: the dispatch itself records the events at the
    // kernel's start and end
    hipExtLaunchKernelGGL(k_gate_up<64>, dim3(grid2), dim3(gate_up_threads(64)), 0, stream,
                          timing->start,
                          timing->stop, 0, a);
    E0_CHECK_LAUNCH();
  } else {
  E0_MARK(1, true);
  switch (cpr) {
    case 8: k_gate_up<8><<<grid2, gate_up_threads(8), 0, stream>>>(a); break;
    case 16: k_gate_up<16><<<grid2, gate_up_threads(16), 0, stream>>>(a); break;
    case 32: k_gate_up<32><<<grid2, gate_up_threads(32), 0, stream>>>(a); break;
    case 64: k_gate_up<64><<<grid2, gate_up_threads(64), 0, stream>>>(a); break;
    case 128: k_gate_up<128><<<grid2, gate_up_threads(128), 0, stream>>>(a); break;
    case 192: k_gate_up<192><<<grid2, gate_up_threads(192), 0, stream>>>(a); break;
    case 256: k_gate_up<256><<<grid2, gate_up_threads(256), 0, stream>>>(a); break;
    default: return EDGE0_EINVAL;
  }
  E0_CHECK_LAUNCH();
  E0_MARK(1, false);
  }
  return launch_down(a, stream, timing, fc1);
}

template <int TPW, bool DEFER>
static void launch_down_t(const MoeArgs& a, int units, const HeadPart* fc1, hipStream_t stream) {
  if (fc1 == nullptr) {
    k_down<TPW, DEFER><<<units, 256, 0, stream>>>(a);
  } else {
    k_down_fc1<TPW, DEFER><<<dim3(std::max(units, fc1->n_wg), 2), 256, 0, stream>>>(a, *fc1);
  }
}

template <bool DEFER>
static int launch_down_tpw(const MoeArgs& a, int tpw, int units, const HeadPart* fc1,
                           hipStream_t stream) {
  if (tpw <= 1) launch_down_t<1, DEFER>(a, units, fc1, stream);
  else if (tpw <= 2) launch_down_t<2, DEFER>(a, units, fc1, stream);
  else if (tpw <= 3) launch_down_t<3, DEFER>(a, units, fc1, stream);
  else if (tpw <= 4) launch_down_t<4, DEFER>(a, units, fc1, stream);
  else if (tpw <= 6) launch_down_t<6, DEFER>(a, units, fc1, stream);
  else if (tpw <= 8) launch_down_t<8, DEFER>(a, units, fc1, stream);
  else if (tpw <= 12) launch_down_t<12, DEFER>(a, units, fc1, stream);
  else if (tpw <= 16) launch_down_t<16, DEFER>(a, units, fc1, stream);
  else return EDGE0_EINVAL;
  return EDGE0_OK;
}

int launch_down(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing,
                const HeadPart* fc1, bool defer) {
  if (fc1 != nullptr && fc1->n_wg < 1) return EDGE0_EINVAL;
  // DEFER finishes the fused layer kernel's rows: at most 16 ranks and 16 experts
  if (defer && (a.r > kFusedMaxRank || a.r % 8 != 0 || a.K > 16)) return EDGE0_EINVAL;
  E0_MARK(2, true);
  {
    const int NC = a.I / 32, cps = (NC + a.S - 1) / a.S;
    const int tpw = (a.K * cps + 3) / 4;
    const int units = (a.d / 64) * a.S;
    const int rc = defer ? launch_down_tpw<true>(a, tpw, units, fc1, stream)
                         : launch_down_tpw<false>(a, tpw, units, fc1, stream);
    if (rc != EDGE0_OK) return rc;
  }
  E0_CHECK_LAUNCH();
  E0_MARK(2, false);
  return EDGE0_OK;
}

bool layer_fused_ok(const MoeArgs& a) {
  return (a.d == 2048 || a.d == 4096) && a.r <= kFusedMaxRank && a.r % 8 == 0 &&
         a.I % (8 * kFusedRowsPerWave) == 0 && a.E <= kFusedMaxExperts;
}

// LoRA producers of the fused layer kernel: 2, 4 or 8 A rows each (a divisor
// of 2r), at most 64 producers where possible, their count a multiple of 8
static void fused_producers(const MoeArgs& a, int* n_prod, int* rows) {
  *n_prod = 0;
  *rows = 0;
  if (a.r == 0) return;
  const int nr = a.K * 2 * a.r;
  int rp = 2;
  while (nr / rp > 64 && rp < kFusedMaxProdRows) rp *= 2;
  *rows = rp;
  *n_prod = ((nr + rp - 1) / rp + 7) / 8 * 8;
}

int launch_layer_fused(const MoeArgs& a, const LayerIn& li, hipStream_t stream,
                       const LaunchTiming* timing) {
  if (!layer_fused_ok(a)) return EDGE0_EINVAL;
  MoeArgs b = a;
  fused_producers(a, &b.n_prod, &b.prod_rows);
  const bool route = li.flags & IN_ROUTER;
  if (route) {
    // router rows: at most 64 producers, kFusedMaxRouteRows rows each
    b.route_rows = (a.E + 63) / 64;
    const int pr = ((a.E + b.route_rows - 1) / b.route_rows + 7) / 8 * 8;
    b.n_prod = std::max(b.n_prod, pr);
  }
  const int grid = b.n_prod + a.K * (a.I / (8 * kFusedRowsPerWave));
  auto kern = a.d == 2048 ? (route ? k_layer_fused<1, true> : k_layer_fused<1, false>)
                          : (route ? k_layer_fused<2, true> : k_layer_fused<2, false>);
  if (timing && timing->which == 1) {
    // measured launch: events recorded by the dispatch at its start and end
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(kFusedThreads), 0, stream, timing->start,
                          timing->stop, 0, b, li);
  } else {
    kern<<<grid, kFusedThreads, 0, stream>>>(b, li);
  }
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

int launch_combine(const MoeArgs& a, hipStream_t stream) {
  k_combine<<<(a.d + 255) / 256, 256, 0, stream>>>(a);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

}  // namespace e0

using namespace e0;

extern "C" int edge0_moe_layer(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                               const int32_t* slot_table, const int32_t* ids, const float* w,
                               const void* x, void* y, void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !x || !y || x == y) return EDGE0_EINVAL;
  MoeArgs a;
  const int rc = fill_moe_args(shape, pool, slot_table, ids, w, x, y, workspace, &a);
  if (rc != EDGE0_OK) return rc;
  return launch_layer_call(a, stream);
}

extern "C" int edge0_moe_layer_lora(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                    const edge0_lora* lora, const int32_t* slot_table,
                                    const int32_t* ids, const float* w, const void* x, void* y,
                                    void* workspace, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !x || !y || x == y) return EDGE0_EINVAL;
  const int r = shape->lora_rank;
  if (r > 0 && (!lora || !lora->a_gate || !lora->b_gate || !lora->a_up || !lora->b_up ||
                !lora->a_down || !lora->b_down || lora->expert_stride < 0))
    return EDGE0_EINVAL;
  // the bundles need not hold adapters: the pool is checked against the
  // LoRA-free layout (the int4 arrays sit at the same offsets in both)
  MoeArgs a;
  int rc = fill_moe_args(shape, pool, slot_table, ids, w, x, y, workspace, &a, false);
  if (rc != EDGE0_OK) return rc;
  if (r > 0) {
    a.lora_sep = true;
    const void* f[6] = {lora->a_gate, lora->b_gate, lora->a_up, lora->b_up, lora->a_down, lora->b_down};
    for (int i = 0; i < 6; ++i) a.lo_base[i] = static_cast<const uint8_t*>(f[i]);
    a.lo_stride = lora->expert_stride * 2;  // bf16 elements
  }
  return launch_layer_call(a, stream);
}

// ------------------------------------------------- no-allocation variant
// The single-layer call on a workspace the library holds itself: a file-scope
// device array (one copy per GPU, alive until the process ends), for callers
// that cannot allocate (code under graph capture, tight serving loops).  Its
// device address is looked up once per device, with that device current,
// and only that address is handed to kernels.
namespace e0 {
constexpr size_t kStaticScratchBytes = EDGE0_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace e0

static __device__ __align__(256) uint8_t scratch[e0::kStaticScratchBytes];

namespace e0 {
__global__ void k_zero_words(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];
static bool g_scratch_zeroed[kMaxDevices];

// the calling thread's current device's copy of `scratch`, zero-filled by a
// kernel on `stream` the first time (the calls leave it ready for the next)
static int static_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EDGE0_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return EDGE0_EHIP;
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_zeroed[dev]) {
    k_zero_words<<<64, 256, 0, stream>>>(static_cast<uint32_t*>(g_scratch_ptr[dev]),
                                         kStaticScratchBytes / 4);
    E0_CHECK_LAUNCH();
    g_scratch_zeroed[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return EDGE0_OK;
}
}  // namespace e0

extern "C" int edge0_moe_layer_noalloc(const edge0_moe_shape* shape, const edge0_slot_pool* pool,
                                       const int32_t* slot_table, const int32_t* ids,
                                       const float* w, const void* x, void* y,
                                       int32_t* error_out, hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !x || !y || x == y || !pool || !slot_table || !ids || !w)
    return EDGE0_EINVAL;
  if (ws_layout(shape).total > kStaticScratchBytes) return EDGE0_ESCRATCH;
  void* ws = nullptr;
  int rc = static_scratch(&ws, stream);
  if (rc != EDGE0_OK) return rc;
  MoeArgs a;
  if ((rc = fill_moe_args(shape, pool, slot_table, ids, w, x, y, ws, &a)) != EDGE0_OK) return rc;
  a.err_out = error_out;
  return launch_layer_call(a, stream);
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
