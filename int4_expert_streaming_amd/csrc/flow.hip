// The resident decode step as one persistent cooperative launch.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction": §3.1 "Math contract" and "Executor
// paths" (the routed experts' int4 rows gathered through the slot table,
// SwiGLU, weighted sum), §3.3 (unmerged LoRA as a parallel delta), §3.2
// "Prediction-as-routing" (consumer layers route by the prediction their
// owner's head committed one token earlier, so their experts are known
// before the step starts); App. A "Softmax-topk" for the router layers.
//
// Why: at batch 1 a layer moves ~14 MB, 1.8 us at 8 TB/s, but as a chain of
// dependent launches each kernel pays its launch, the latency of reading
// what the previous kernel wrote, and the HBM latency of its own weights.
// Here the workgroups stay resident for the whole step and hand data to each
// other through device-coherent memory: at every phase boundary each
// workgroup has already issued the loads of its next phase (registers, and
// LoRA A rows into LDS), so weight latency overlaps the hand-off.
//
// Work of layer L (G workgroups, G = K * d_inter / 16):
//   prologue  every workgroup: y_{L-1} = bf16(fixed-point sum), h_L =
//             bf16(h_{L-1} + y_{L-1}) (each keeps its own copy of h),
//             x_L = bf16(RMSNorm(h_L)) into LDS; workgroup 0 stores x, y, h
//             and clears layer L's accumulator.
//   R phase   (router layers) workgroup e < E: logit e = W_r[e] . x; then
//             every workgroup commits the top-K itself (control wave).
//   A phase   unit = 16 rows of one routed expert: t = A x for the expert's
//             gate/up adapters, gate/up int4 rows + (alpha/r) B t, SwiGLU;
//             publishes h as bf16 hi/lo pair words, 16-row sums of h and
//             16-row partials of A_down h.
//   D phase   unit = 64 output rows x 4 input chunks x all K experts (tiled
//             int4 down weights), weighted by w_k, plus (first slice) the
//             LoRA-down delta; added into layer L's fixed-point accumulator.
// Each phase ends at a grid-wide boundary: every thread's device-coherent
// stores and atomics complete, the workgroup synchronises, the control wave
// (a ninth wave that issues no weight loads, so its polls never queue behind
// them) counts the arrival and polls until all G workgroups have arrived.
// Every wait is bounded: after `spin` polls the workgroup records EDGE0_EHIP,
// raises the abort word and exits, and every other wait exits on seeing it.
// Arithmetic is the fused single-layer path's (same helpers, same orders).
#include <hip/hip_ext.h>

#include "gemv_dev.h"
#include "moe_internal.h"

namespace e0 {

constexpr int kFlowWaves = 8;                          // compute waves
constexpr int kFlowCompute = 64 * kFlowWaves;
constexpr int kFlowThreads = kFlowCompute + 64;        // + the control wave
constexpr int kFlowD = 2048;                           // d_model of this path
constexpr int kFlowPer = kFlowD / kFlowCompute;        // hidden elements per thread
constexpr int kFlowRW = 2;                             // gate/up row pairs per wave
constexpr int kFlowRows = kFlowWaves * kFlowRW;        // 16 rows per A unit
constexpr int kFlowMaxRank = 16;
constexpr int kFlowMaxExperts = 256;
constexpr int kFlowTPW = 2;                            // down tiles per compute wave
constexpr int kFlowMaxTiles = kFlowWaves * kFlowTPW;   // 16 per D unit
constexpr int kFlowMaxK = 16;
constexpr int kFlowAR = 2 * kFlowMaxRank / kFlowWaves; // LoRA A rows per wave (4)

__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev_u64(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shared state of one workgroup.
struct FlowLds {
  uint16_t xs[kFlowD];
  uint32_t hp_s[kFlowMaxTiles][32];       // D unit: hi then lo pair words per tile
  float hsum_s[kFlowMaxTiles];
  float td_s[kFlowWaves][64];
  float red[kFlowWaves][64];
  float t_s[2][kFlowMaxRank];
  float h_s[kFlowRows];
  float hrep_s[kFlowRows];
  int32_t ids_s[kFlowMaxK];               // routing of the current layer
  float w_s[kFlowMaxK];
  int32_t slot_s[kFlowMaxK];
  int32_t nslot_s[kFlowMaxK];             // next layer's (prediction-routed) routing
  float nw_s[kFlowMaxK];
  float lg[kFlowWaves];
  int go;
};

// Grid-wide end of phase p.  All threads call it after their stores and
// atomics of the phase; `issue` runs in the compute waves (loads of later
// phases) while the control wave, which issues no weight loads and so never
// waits behind them, counts the arrival and polls.  Returns false when the
// launch aborts.
template <class F>
__device__ __forceinline__ bool flow_phase_end(const FlowArgs& a, FlowLds& s, int p, F&& issue) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores and atomics have completed
  __syncthreads();
  if (tid_here() >= kFlowCompute) {
    if (tid_here() == kFlowCompute) {
      // arrivals spread over kFlowCounters counters (256 bytes apart), so the
      // atomic increments of the G workgroups do not all serialise on one
      // address; every counter is polled
      uint32_t* base = a.cnt + (size_t)p * kFlowCounters * 64;
      __hip_atomic_fetch_add(base + (blockIdx.x % kFlowCounters) * 64, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t tgt = a.target[p];
      int go = 1;
      int64_t it = 0;
      for (;;) {
        uint32_t v[kFlowCounters];
#pragma unroll
        for (int c = 0; c < kFlowCounters; ++c) v[c] = ld_dev_u32(base + c * 64);
        bool done = true;
#pragma unroll
        for (int c = 0; c < kFlowCounters; ++c) done &= (int32_t)(v[c] - tgt) >= 0;
        if (done) break;
        __builtin_amdgcn_s_sleep(1);
        ++it;
        if ((it & 15) == 0 && ld_dev_u32(a.abort_word) != 0) {
          go = 0;
          break;
        }
        if (it >= a.spin) {
          set_error(a.err, EDGE0_EHIP);
          st_dev_u32(a.abort_word, 1u);
          go = 0;
          break;
        }
      }
      s.go = go;
    }
  } else {
    issue();
  }
  __syncthreads();
  return s.go != 0;
}

__device__ __forceinline__ bool flow_is_router(const FlowArgs& a, int L) {
  return !(L >= a.consumer_first && L <= a.consumer_last && a.step > 0);
}

// a MoeArgs carrying the fields the shared gate/up helpers read
__device__ __forceinline__ MoeArgs flow_moe(const FlowArgs& a) {
  MoeArgs m{};
  m.d = a.d;
  m.E = a.E;
  m.I = a.I;
  m.K = a.K;
  m.g = a.g;
  m.r = a.r;
  m.scale = a.scale;
  m.lay = a.lay;
  return m;
}

// Register weights of one layer's A unit and D unit.
struct FlowPreA {
  uint2 arow;                  // T unit: 4 elements of one LoRA A row
  GuW<1, kFlowRW> gw;          // 2 gate + 2 up rows of the wave
  uint4 ad0, ad1;              // A_down columns of the A unit (wave 0, lanes < r)
  int slotA;                   // slot of the A unit's expert (-1 invalid)
};
struct FlowPreD {
  uint4 q[kFlowTPW];           // down tiles of the wave
  uint32_t sv[kFlowTPW], bv[kFlowTPW];
  float wt[kFlowTPW];
  uint4 bdr[2];                // B_down row o (r <= 16), LoRA unit waves < K
};

__device__ __forceinline__ const uint8_t* flow_bundle(const FlowArgs& a, int slot) {
  return a.pool + (size_t)(slot >= 0 ? slot : 0) * (size_t)a.slot_bytes;
}

// Slot of expert e of layer L from the lane-distributed table row tv0..tv3
// (wave-uniform e), -1 when e or its slot is out of range.
__device__ __forceinline__ int flow_slot_of(const FlowArgs& a, int e, int tv0, int tv1, int tv2,
                                            int tv3) {
  const int ec = min(max(e, 0), a.E - 1);
  const int j = ec >> 6;
  const int v = j == 0 ? tv0 : j == 1 ? tv1 : j == 2 ? tv2 : tv3;
  int slot = __builtin_amdgcn_readlane(v, ec & 63);
  if (e < 0 || e >= a.E || slot < 0 || slot >= a.n_slots) slot = -1;
  return slot;
}

// Compute waves: the slots of routing ids[0..K) of layer L; wave 0 stores
// them (lane kk) to slot_out.  Waits for the table row only.
__device__ __forceinline__ void flow_resolve(const FlowArgs& a, int L, const int32_t* ids,
                                             int32_t* slot_out) {
  const int tid = tid_here(), lane = tid & 63, wave = tid >> 6;
  const int32_t* trow = a.tables + (size_t)L * a.E;
  const int tv0 = trow[min(lane, a.E - 1)];
  const int tv1 = trow[min(lane + 64, a.E - 1)];
  const int tv2 = trow[min(lane + 128, a.E - 1)];
  const int tv3 = trow[min(lane + 192, a.E - 1)];
  int myslot = -1;
  for (int kk = 0; kk < a.K; ++kk) {
    const int slot = flow_slot_of(a, ids[kk], tv0, tv1, tv2, tv3);
    if (lane == kk) myslot = slot;
  }
  if (wave == 0 && lane < a.K) slot_out[lane] = myslot;
}

// Compute waves: the loads of one layer's T unit (LoRA A row tr of routed
// expert kT, slot slotT: 4 elements per thread) and A unit (expert slot
// slotA, rows i0..i0+15: gate/up rows and A_down columns).  Nothing waits on
// them here.
__device__ __forceinline__ void flow_issue_a(const FlowArgs& a, int slotT, int tr, int slotA,
                                             int i0, FlowPreA& pre) {
  const int tid = tid_here(), lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  pre.arow = make_uint2(0, 0);
  if (r > 0) {
    const uint8_t* bT = flow_bundle(a, slotT);
    const int trc = min(max(tr, 0), 2 * r - 1);
    const uint16_t* arow =
        reinterpret_cast<const uint16_t*>(bT + (trc >= r ? a.lay.a_up : a.lay.a_gate)) +
        (size_t)(trc % r) * a.d;
    pre.arow = reinterpret_cast<const uint2*>(arow)[tid];
  }
  pre.slotA = slotA;
  const uint8_t* bA = flow_bundle(a, slotA);
  MoeArgs m = flow_moe(a);
  gu_load<1, kFlowRW>(m, bA, i0, pre.gw);
  pre.ad0 = pre.ad1 = make_uint4(0, 0, 0, 0);
  if (wave == 0 && lane < r) {
    const uint4* src = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(bA + a.lay.a_down) + (size_t)lane * a.I + i0);
    pre.ad0 = src[0];
    pre.ad1 = src[1];
  }
}

// Compute waves: the D unit's loads (row block rb, chunks c0 .. c0+ncs-1 of
// all K experts) from the current layer's slots and weights in LDS.
__device__ __forceinline__ void flow_issue_d(const FlowArgs& a, const FlowLds& s, int rb, int sl,
                                             int c0, int ncs, FlowPreD& pre) {
  const int tid = tid_here(), lane = tid & 63, wave = tid >> 6;
  const int d = a.d, r = a.r, K = a.K, NC = a.I / 32;
  const int nt = K * ncs;
  const int o = rb * 64 + lane;
#pragma unroll
  for (int mm = 0; mm < kFlowTPW; ++mm) {
    const int t = wave * kFlowTPW + mm;
    const bool valid = t < nt;
    const int tc = valid ? t : 0;
    const int kk = ncs > 0 ? tc / ncs : 0, c = c0 + (ncs > 0 ? tc % ncs : 0);
    const int slot = s.slot_s[kk];
    pre.wt[mm] = (valid && slot >= 0) ? s.w_s[kk] : 0.f;
    const uint8_t* b = flow_bundle(a, slot);
    const int cc = min(c, NC - 1);
    pre.q[mm] = reinterpret_cast<const uint4*>(b + a.lay.down_q)[((size_t)rb * NC + cc) * 64 + lane];
    const int grp = (32 * cc) / a.g;
    pre.sv[mm] = reinterpret_cast<const uint16_t*>(b + a.lay.down_s)[(size_t)grp * d + o];
    pre.bv[mm] = reinterpret_cast<const uint16_t*>(b + a.lay.down_b)[(size_t)grp * d + o];
  }
  pre.bdr[0] = pre.bdr[1] = make_uint4(0, 0, 0, 0);
  if (r > 0 && sl == 0 && wave < K) {
    const uint8_t* b = flow_bundle(a, s.slot_s[wave]);
    const uint4* Bdp = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(b + a.lay.b_down) + (size_t)o * r);
    pre.bdr[0] = Bdp[0];
    if (r > 8) pre.bdr[1] = Bdp[1];
  }
}

// Router row e = w of layer L (compute wave v covers elements [256 v, 256 v
// + 256), lane 4 elements)
__device__ __forceinline__ uint2 flow_router_row(const FlowArgs& a, int L, int w) {
  const int tid = tid_here();
  const int e = min(w, a.E - 1);
  const uint16_t* row = a.routers[L] + (size_t)e * a.d;
  return reinterpret_cast<const uint2*>(row)[tid];
}

__global__ __launch_bounds__(kFlowThreads) void k_flow_step(FlowArgs a) {
  __shared__ FlowLds s;
  const int d = a.d, r = a.r, K = a.K, I = a.I, NC = I / 32;
  const int w = blockIdx.x, G = gridDim.x;
  // A units in XCD-aware order: consecutive workgroups sit on different XCDs
  // (round-robin over 8), so logical unit lb = (w % 8) * (G / 8) + w / 8 gives
  // each XCD a contiguous range of an expert's row blocks
  const int lb = (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
  const int nwg = I / kFlowRows;
  const int kA = lb / nwg, i0 = (lb % nwg) * kFlowRows, blk = i0 / 16;
  // T unit: LoRA A row trT (gate rows 0..r-1, up rows r..2r-1) of expert kT
  const int nT = r > 0 ? K * 2 * r : 0;
  const bool has_t = w < nT;
  const int kT = has_t ? w / (2 * r) : 0, trT = has_t ? w % (2 * r) : 0;
  const int rb = w % (d / 64), sl = w / (d / 64);
  const int c0 = sl * a.cps;
  const int ncs = max(0, min(NC, c0 + a.cps) - c0);
  const int nt = K * ncs;
  const bool compute = tid_here() < kFlowCompute;
  const int nOut = min(G, kFlowCompute);
  MoeArgs m = flow_moe(a);
  // running hidden state, compute thread tid owns elements 4 tid .. 4 tid + 3
  float hc[kFlowPer] = {0.f, 0.f, 0.f, 0.f};
  if (compute) {
    const uint2 hq = reinterpret_cast<const uint2*>(a.h)[tid_here()];
    hc[0] = bf_lo(hq.x);
    hc[1] = bf_hi(hq.x);
    hc[2] = bf_lo(hq.y);
    hc[3] = bf_hi(hq.y);
  }
  FlowPreA pa;
  FlowPreD pd;
  uint2 rrow = make_uint2(0, 0);
  int p = 0;
  // layer 0's first loads: its router row (layer 0 is never prediction-routed)
  if (compute) rrow = flow_router_row(a, 0, w);
  for (int L = 0; L < a.n_layers; ++L) {
    // thread indices re-derived per layer (see tid_here)
    const int tid = tid_here(), lane = tid & 63, wave = tid >> 6;
    const int o = rb * 64 + lane;
    const bool router = flow_is_router(a, L);
    // a prediction-routed layer's routing was resolved during the previous
    // layer (s.nslot_s, s.nw_s) and its loads issued at the last boundary
    if (!router && tid < K) {
      s.slot_s[tid] = s.nslot_s[tid];
      s.w_s[tid] = s.nw_s[tid];
    }
    // ---- prologue: h_L, x_L (every workgroup the same values)
    uint32_t yb[kFlowPer] = {0u, 0u, 0u, 0u};
    if (compute) {
      if (L > 0) {
        const unsigned long long* src = a.acc + (size_t)((L - 1) & 1) * d;
        unsigned long long av[kFlowPer];
#pragma unroll
        for (int e = 0; e < kFlowPer; ++e) av[e] = ld_dev_u64(src + kFlowPer * tid + e);
#pragma unroll
        for (int e = 0; e < kFlowPer; ++e) {
          yb[e] = f2bf(from_fix(av[e]));
          hc[e] = bf2f(f2bf(hc[e] + bf2f(yb[e])));
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < kFlowPer; ++e) ss = fmaf(hc[e], hc[e], ss);
      ss = wave_sum(ss);
      if (lane == 0) s.lg[wave] = ss;
    }
    __syncthreads();
    uint2 xq = make_uint2(0, 0);  // this thread's 4 elements of x
    if (compute) {
      float tot = 0.f;
#pragma unroll
      for (int v = 0; v < kFlowWaves; ++v) tot += s.lg[v];
      const float inv = 1.f / sqrtf(tot / (float)d + a.eps);
      xq.x = f2bf(hc[0] * inv) | (f2bf(hc[1] * inv) << 16);
      xq.y = f2bf(hc[2] * inv) | (f2bf(hc[3] * inv) << 16);
      reinterpret_cast<uint2*>(s.xs)[tid] = xq;
      // outputs and the cleared accumulator, spread over the workgroups
      // (workgroup w < nOut takes the threads tid = w mod nOut)
      if (w < nOut && tid % nOut == w) {
        reinterpret_cast<uint2*>(a.x + (size_t)L * d)[tid] = xq;
        reinterpret_cast<uint2*>(a.h + (size_t)L * d)[tid] =
            make_uint2(f2bf(hc[0]) | (f2bf(hc[1]) << 16), f2bf(hc[2]) | (f2bf(hc[3]) << 16));
        if (L > 0)
          reinterpret_cast<uint2*>(a.y + (size_t)(L - 1) * d)[tid] =
              make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
        unsigned long long* acc = a.acc + (size_t)(L & 1) * d;
#pragma unroll
        for (int e = 0; e < kFlowPer; ++e) st_dev_u64(acc + kFlowPer * tid + e, 0ull);
      }
      // this layer's A_down h sums start from zero (last read in the previous
      // layer's D phase; first added to after the T boundary)
      if (w == G - 1 && tid < K * r) st_dev_u64(a.tdown + tid, 0ull);
    }
    __syncthreads();  // xs complete
    // ---- R phase: router logits, then every workgroup's own top-K
    if (router) {
      if (compute && w < a.E) {
        float acc = 0.f;
        acc = dot2bf(rrow.x, xq.x, acc);
        acc = dot2bf(rrow.y, xq.y, acc);
        acc = wave_sum(acc);
        if (lane == 0) s.red[wave][0] = acc;
      }
      __syncthreads();
      if (tid == 0 && w < a.E) {
        float l = 0.f;
        for (int v = 0; v < kFlowWaves; ++v) l += s.red[v][0];
        st_dev(a.logits + w, l);
      }
      if (!flow_phase_end(a, s, p++, [] {})) return;
      if (!compute) {
        if (a.E <= 128)  // E <= 256 in this mode
          wave_topk_n<2, true>(a.logits, a.E, K, s.ids_s, s.w_s);
        else
          wave_topk_n<4, true>(a.logits, a.E, K, s.ids_s, s.w_s);
        if (w == 0 && lane < K) {
          a.exec_ids[(size_t)L * K + lane] = s.ids_s[lane];
          a.exec_w[(size_t)L * K + lane] = s.w_s[lane];
        }
      }
      __syncthreads();
      if (compute) flow_resolve(a, L, s.ids_s, s.slot_s);
      __syncthreads();
      if (compute) flow_issue_a(a, s.slot_s[kT], trT, s.slot_s[kA], i0, pa);
    }
    // ---- T phase: one LoRA A row of one routed expert per workgroup
    if (nT > 0) {
      if (compute && has_t) {
        float acc = 0.f;
        acc = dot2bf(pa.arow.x, xq.x, acc);
        acc = dot2bf(pa.arow.y, xq.y, acc);
        acc = wave_sum(acc);
        if (lane == 0) s.red[wave][0] = acc;
      }
      __syncthreads();
      if (tid == 0 && has_t) {
        float t = 0.f;
        for (int v = 0; v < kFlowWaves; ++v) t += s.red[v][0];
        st_dev(a.t_in + w, s.slot_s[kT] >= 0 ? t : 0.f);
      }
      if (!flow_phase_end(a, s, p++, [&] { flow_issue_d(a, s, rb, sl, c0, ncs, pd); })) return;
    }
    // ---- A phase
    const int slotA = s.slot_s[kA];
    const bool okA = slotA >= 0;
    if (compute) {
      float tg = 0.f, tu = 0.f;
      if (r > 0 && lane < r) {
        tg = ld_dev(a.t_in + kA * 2 * r + lane);
        tu = ld_dev(a.t_in + kA * 2 * r + r + lane);
      }
      gu_finish<1, kFlowRW, false>(m, pa.gw, kA, i0, s.xs, tg, tu, s.h_s, s.hrep_s);
    }
    __syncthreads();
    // publish: pair words of the 16 rows (threads 0-7 hi, 8-15 lo), the 16-row
    // sum, and the 16-row partials of A_down h added into the expert's
    // fixed-point sums (wave 0, lanes < r)
    if (tid < 16) {
      const int gi = (tid & 7) >> 2, mm = tid & 3;
      const float e0 = okA ? s.h_s[8 * gi + mm] : 0.f, e4 = okA ? s.h_s[8 * gi + mm + 4] : 0.f;
      const uint32_t h0 = f2bf(e0), h4 = f2bf(e4);
      uint32_t word;
      if (tid < 8) word = h0 | (h4 << 16);
      else word = f2bf(e0 - bf2f(h0)) | (f2bf(e4 - bf2f(h4)) << 16);
      uint32_t* dst = (tid < 8 ? a.hp_hi : a.hp_lo) + (size_t)kA * (I / 2) + i0 / 2 + 4 * gi + mm;
      st_dev_u32(dst, word);
    }
    if (tid == 16) {
      float sm = 0.f;
      for (int t = 0; t < 16; ++t) sm += s.hrep_s[t];
      st_dev(a.hs + (size_t)kA * (I / 16) + blk, okA ? sm : 0.f);
    }
    if (wave == 0 && lane < r) {
      const uint32_t wd[8] = {pa.ad0.x, pa.ad0.y, pa.ad0.z, pa.ad0.w,
                              pa.ad1.x, pa.ad1.y, pa.ad1.z, pa.ad1.w};
      float sm = 0.f;
#pragma unroll
      for (int mm = 0; mm < 8; ++mm)
        sm += bf_lo(wd[mm]) * s.h_s[2 * mm] + bf_hi(wd[mm]) * s.h_s[2 * mm + 1];
      if (okA) atomicAdd(a.tdown + kA * r + lane, to_fix(sm));
    }
    if (!okA && tid == 0 && (lb % nwg) == 0) set_error(a.err, EDGE0_ERANGE);
    // A boundary; meanwhile the D unit's weights (when no T phase issued them)
    // and the next layer's committed prediction and slots
    const int Ln = L + 1;
    const bool last = Ln >= a.n_layers;
    const bool next_pred = !last && !flow_is_router(a, Ln);
    if (!flow_phase_end(a, s, p++, [&] {
          int32_t nid = 0;
          float nw = 0.f;
          int tv0 = 0, tv1 = 0, tv2 = 0, tv3 = 0;
          if (next_pred) {
            if (lane < K) {
              nid = a.pred_ids[(size_t)Ln * K + lane];
              nw = a.pred_w[(size_t)Ln * K + lane];
            }
            const int32_t* trow = a.tables + (size_t)Ln * a.E;
            tv0 = trow[min(lane, a.E - 1)];
            tv1 = trow[min(lane + 64, a.E - 1)];
            tv2 = trow[min(lane + 128, a.E - 1)];
            tv3 = trow[min(lane + 192, a.E - 1)];
          }
          if (nT == 0) flow_issue_d(a, s, rb, sl, c0, ncs, pd);
          if (next_pred) {
            int myslot = -1;
            for (int kk = 0; kk < K; ++kk) {
              const int e = __shfl(nid, kk, kWave);
              const int slot = flow_slot_of(a, e, tv0, tv1, tv2, tv3);
              if (lane == kk) myslot = slot;
            }
            if (wave == 0 && lane < K) {
              s.nslot_s[lane] = myslot;
              s.nw_s[lane] = nw;
            }
          }
        }))
      return;
    // ---- D phase: h pairs, 16-row sums and A_down h partials of the layer
    if (compute) {
      const int t = tid >> 5, j = tid & 31;  // 16 tiles x 32 words
      uint32_t v = 0;
      if (t < nt) {
        const int kk = t / ncs, c = c0 + t % ncs;
        const uint32_t* src = (j < 16 ? a.hp_hi : a.hp_lo) + (size_t)kk * (I / 2);
        v = ld_dev_u32(src + 16 * c + (j & 15));
      }
      float hv = 0.f;
      if (tid < nt) {
        const int kk = tid / ncs, c = c0 + tid % ncs;
        const float* hsp = a.hs + (size_t)kk * (I / 16);
        hv = ld_dev(hsp + 2 * c) + ld_dev(hsp + 2 * c + 1);
      }
      const bool lora_unit = r > 0 && sl == 0 && wave < K;
      unsigned long long tdq = 0;
      if (lora_unit && lane < r) tdq = ld_dev_u64(a.tdown + wave * r + lane);
      s.hp_s[t][j] = v;
      if (tid < kFlowMaxTiles) s.hsum_s[tid] = hv;
      if (lora_unit) s.td_s[wave][lane] = from_fix(tdq);  // lane rr (< r): t_down[rr]
    }
    __syncthreads();
    if (compute) {
      float part = 0.f;
      const Q4Consts kq = q4_consts();
#pragma unroll
      for (int mm = 0; mm < kFlowTPW; ++mm) {
        const int t = wave * kFlowTPW + mm;
        if (t < nt) {
          const float sc = bf2f(pd.sv[mm]), bb = bf2f(pd.bv[mm]);
          const uint32_t* hp = s.hp_s[t];
          const float acc = chunk_dot128(pd.q[mm], hp, kq) + chunk_dot128(pd.q[mm], hp + 16, kq);
          part += pd.wt[mm] * (sc * acc + (bb - 128.f * sc) * s.hsum_s[t]);
        }
      }
      if (r > 0 && sl == 0 && wave < K && s.slot_s[wave] >= 0) {
        float dl = 0.f;
        const uint32_t bw[8] = {pd.bdr[0].x, pd.bdr[0].y, pd.bdr[0].z, pd.bdr[0].w,
                                pd.bdr[1].x, pd.bdr[1].y, pd.bdr[1].z, pd.bdr[1].w};
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          if (2 * q2 < r) {
            dl += bf_lo(bw[q2]) * s.td_s[wave][2 * q2];
            dl += bf_hi(bw[q2]) * s.td_s[wave][2 * q2 + 1];
          }
        }
        part += s.w_s[wave] * (a.scale * dl);
      }
      s.red[wave][lane] = part;
    }
    __syncthreads();
    if (wave == 0) {
      float tot = 0.f;
#pragma unroll
      for (int v = 0; v < kFlowWaves; ++v) tot += s.red[v][lane];
      atomicAdd(a.acc + (size_t)(L & 1) * d + o, to_fix(tot));
    }
    // D boundary; meanwhile the next layer's first loads
    if (!flow_phase_end(a, s, p++, [&] {
          if (last) return;
          if (next_pred) flow_issue_a(a, s.nslot_s[kT], trT, s.nslot_s[kA], i0, pa);
          else rrow = flow_router_row(a, Ln, w);
        }))
      return;
  }
  // final combine: y of the last layer, h_out
  if (w == 0 && compute) {
    const int tid = tid_here();
    const int L = a.n_layers - 1;
    const unsigned long long* src = a.acc + (size_t)(L & 1) * d;
    uint32_t yb[kFlowPer];
#pragma unroll
    for (int e = 0; e < kFlowPer; ++e) {
      yb[e] = f2bf(from_fix(ld_dev_u64(src + kFlowPer * tid + e)));
      hc[e] = bf2f(f2bf(hc[e] + bf2f(yb[e])));
    }
    reinterpret_cast<uint2*>(a.y + (size_t)L * d)[tid] =
        make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
    reinterpret_cast<uint2*>(a.h + (size_t)(L + 1) * d)[tid] =
        make_uint2(f2bf(hc[0]) | (f2bf(hc[1]) << 16), f2bf(hc[2]) | (f2bf(hc[3]) << 16));
  }
}

// ------------------------------------------------------------------ host
int flow_grid(const edge0_moe_shape& sh) { return sh.top_k * (sh.d_inter / kFlowRows); }

bool flow_shape_ok(const edge0_moe_shape& sh, int n_layers) {
  if (sh.d_model != kFlowD || sh.n_experts < 1 || sh.n_experts > kFlowMaxExperts) return false;
  if (sh.lora_rank < 0 || sh.lora_rank > kFlowMaxRank || sh.lora_rank % 8 != 0) return false;
  if (sh.top_k < 1 || sh.top_k > kFlowMaxK || sh.d_inter % 32 != 0) return false;
  if (n_layers < 1 || 4 * n_layers > kFlowMaxPhases) return false;
  const int G = flow_grid(sh), rbs = sh.d_model / 64;
  if (G < rbs || G % rbs != 0 || G < sh.n_experts || G % kFlowCounters != 0) return false;
  if (G < sh.top_k * 2 * sh.lora_rank) return false;
  const int S = G / rbs, NC = sh.d_inter / 32;
  const int cps = (NC + S - 1) / S;
  return sh.top_k * cps <= kFlowMaxTiles;
}

int flow_coresident(int G) {
  int dev = 0, cus = 0, per = 0, coop = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EDGE0_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
    return EDGE0_EHIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_flow_step, kFlowThreads, 0) !=
      hipSuccess)
    return EDGE0_EHIP;
  return (coop && per * cus >= G) ? EDGE0_OK : EDGE0_EINVAL;
}

int launch_flow_step(const FlowArgs& a, int G, hipStream_t stream) {
  void* args[] = {const_cast<FlowArgs*>(&a)};
  if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_flow_step), dim3(G),
                                 dim3(kFlowThreads), args, 0, stream) != hipSuccess)
    return EDGE0_EHIP;
  return EDGE0_OK;
}

}  // namespace e0
