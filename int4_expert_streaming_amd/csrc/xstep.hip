// The resident decode step as one persistent launch, work split by XCD.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction": §3.1 "Math contract" and "Executor
// paths" (the routed experts' int4 rows gathered through the slot table,
// SwiGLU, weighted sum), §3.3 (unmerged LoRA as a parallel delta), §3.2
// "Prediction-as-routing" (consumer layers route by the prediction their
// owner's head committed one token earlier, so their experts are known
// before the step starts); App. A "Softmax-topk" for the router layers.
//
// Why: a layer moves ~14 MB (1.8 us at 8 TB/s) but is a chain of hand-offs:
// x needs all of the previous layer's y, the SwiGLU activations h of an
// expert need all of x, and the down projection of an output row needs all
// of that expert's h.  Here each layer has three hand-offs, none of them a
// barrier:
//
//   256 workgroups, 32 per XCD (workgroup w runs on XCD w % 8).  With K
//   routed experts, XCD X works on expert k = X / P of the routing, P = 8/K,
//   over its slice of the intermediate rows [part * Ix, (part+1) * Ix),
//   part = X % P, Ix = I / P.  Workgroup j (= w / 8) of the XCD:
//     - gate/up rows i0 .. i0 + RW - 1 of the slice (RW = Ix / 32), with the
//       expert's whole LoRA A x computed by the workgroup itself from A rows
//       held in registers (no hand-off for it);
//     - publishes its RW values of h (bf16 hi + lo) to its XCD, and reads
//       the slice's Ix values back (hand-off 1, within the XCD);
//     - down output rows 64 j .. 64 j + 63 over the slice's input columns,
//       plus the LoRA-down term on the slice's part of A_down h (the delta
//       is linear in h, so the slices' terms add up to the expert's),
//       weighted by w_k: an fp32 partial of y rows 64 j .. 64 j + 63;
//     - sums the 8 XCDs' partials of those 64 rows in XCD order (hand-off 2)
//       and publishes bf16 y for them to its XCD's copy of y; every
//       workgroup reads its XCD's copy (hand-off 3), so each line of y has
//       32 readers rather than 256.
//   Every workgroup keeps its own copy of the residual h in registers and
//   forms x = bf16(RMSNorm(h)) itself.
//
// Hand-offs carry their own completion: every exchanged value is one 64-bit
// word (tag << 32 | payload) stored with one device-coherent atomic store,
// the tag being a running layer number, and a reader polls the words until
// every tag matches.  There are no arrival counters and no wait for a
// store to complete.  A writer can only overwrite a word once every reader
// of its previous value has gone on to a later hand-off that needed the
// writer's new data (the y partials alternate between two buffers for this).
//
// Weights are loaded one layer ahead: a prediction-routed layer's experts
// are known when the step starts, so once a layer's down tiles are done the
// next layer's LoRA A rows, gate/up rows and down tiles are loaded into
// registers, and their latency overlaps the hand-offs.  A router layer
// computes its logits (each XCD all E rows, shared within the XCD), takes
// the top-K, and only then loads its experts.
//
// A control wave issues no weight loads: it performs every store that other
// workgroups read and every poll of what they wrote, so its waits never
// queue behind the weight stream of the compute waves.  Every poll is
// bounded: after `spin` polls the workgroup records EDGE0_EHIP, raises the
// abort word, and every workgroup leaves at its next hand-off.
#include <hip/hip_ext.h>

#include "gemv_dev.h"
#include "moe_internal.h"

namespace e0 {

constexpr int kXWaves = 7;                    // compute waves; wave 7 is the control wave
constexpr int kXThreads = 64 * (kXWaves + 1);
constexpr int kXD = 2048;
constexpr int kXPerXcd = 32;
constexpr int kXG = 8 * kXPerXcd;
constexpr int kXMaxNPW = 4;                   // gate/up row pairs (and down tiles) per wave
constexpr int kXMaxRW = 24;                   // rows per workgroup = chunks per XCD slice
constexpr int kXMaxIx = 32 * kXMaxRW;         // 768
constexpr int kXMaxRank = 16;
constexpr int kXMaxE = 256;
constexpr int kXTdRows = (kXMaxRank + kXWaves - 1) / kXWaves;  // A_down ranks per wave (3)

__device__ __forceinline__ uint32_t x_ld32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void x_st32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long x_ld64(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void x_st64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef __attribute__((address_space(3))) void x_lds_void;
typedef const __attribute__((address_space(1))) void x_glb_void;

struct XLds {
  uint4 arow[2 * kXMaxRank][kXD / 8];  // LoRA A rows (gate, then up) or router rows, bf16
  uint16_t xs[kXD];                    // x of the layer
  uint32_t yw[kXD / 2];                // the previous layer's y (bf16 pairs)
  uint32_t hw[kXMaxIx];                // the XCD slice's h words (hi | lo << 16)
  uint32_t hp[kXMaxRW][32];            // per chunk: 16 hi pair words, 16 lo pair words
  float hsp[kXMaxRW][4];               // per chunk: sums of hi + lo over its four 8-groups
  float red[kXWaves][64];
  float t_s[2 * kXMaxRank];            // LoRA A x of the expert (gate rows, then up rows)
  float td_s[kXMaxRank];               // A_down h over the XCD slice
  float ss[kXWaves + 1];
  uint32_t hrow[kXMaxRW];              // this workgroup's h words
  float lg[kXMaxE];                    // router logits (router layers)
  float lgp[8];                        // this workgroup's router rows
  int32_t tbl[kXMaxE];                 // slot-table row (router layers)
  int32_t ids[16];
  float wts[16];
  int32_t slot_of[kXMaxLayers];        // slot of this workgroup's expert per layer (-1 invalid)
  float w_of[kXMaxLayers];             // its routing weight
  float ypart[64];
  int go;
};

__device__ __forceinline__ bool x_is_pred(const XArgs& a, int L) {
  return L >= a.consumer_first && L <= a.consumer_last && a.step > 0;
}
__device__ __forceinline__ const uint8_t* x_bundle(const XArgs& a, int slot) {
  return a.pool + (size_t)(slot >= 0 ? slot : 0) * (size_t)a.slot_bytes;
}
__device__ __forceinline__ unsigned long long x_word(uint32_t tag, uint32_t payload) {
  return ((unsigned long long)tag << 32) | payload;
}

// Control wave: the poll budget.  Called once per unsuccessful poll; false
// (give up) on the abort word or after `spin` polls, recording EDGE0_EHIP.
__device__ __forceinline__ bool x_again(const XArgs& a, int64_t& n) {
  __builtin_amdgcn_s_sleep(1);
  ++n;
  if ((n & 15) == 0 && x_ld32(a.abort_word) != 0) return false;
  if (n >= a.spin) {
    if ((threadIdx.x & 63) == 0) {
      set_error(a.err, EDGE0_EHIP);
      x_st32(a.abort_word, 1u);
    }
    return false;
  }
  return true;
}

// Control wave: read n <= 64 NW tagged words of src into dst (payloads)
// once every tag equals `tag`.  First lane l < nprobe waits for word
// l * stride alone (one word of each writer), then the whole range is read
// (all of a lane's loads in flight together) and checked, and read again
// while any tag differs.  Returns false on give-up.
template <int NW>
__device__ __forceinline__ bool x_collect(const XArgs& a, const unsigned long long* src, int n,
                                          uint32_t tag, int nprobe, int stride, uint32_t* dst) {
  const int lane = threadIdx.x & 63;
  int64_t polls = 0;
  for (;;) {
    bool ok = true;
    if (lane < nprobe) ok = (uint32_t)(x_ld64(src + lane * stride) >> 32) == tag;
    if (__builtin_amdgcn_readfirstlane((int)__all(ok))) break;
    if (!x_again(a, polls)) return false;
  }
  for (;;) {
    bool ok = true;
    // passes of up to 8 words per lane, each pass's loads in flight together
    for (int base = 0; base < 64 * NW; base += 64 * 8) {
      unsigned long long v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int i = base + lane + 64 * m;
        v[m] = (64 * m < 64 * NW - base && i < n) ? x_ld64(src + i) : 0ull;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int i = base + lane + 64 * m;
        if (64 * m < 64 * NW - base && i < n) {
          ok &= (uint32_t)(v[m] >> 32) == tag;
          dst[i] = (uint32_t)v[m];
        }
      }
    }
    if (__builtin_amdgcn_readfirstlane((int)__all(ok))) return true;
    if (!x_again(a, polls)) return false;
  }
}

// ----------------------------------------------------------- weight sets
// gate/up rows of a compute wave: row pair m is row q = wave + 7 m of the
// workgroup (RW rows; a wave with fewer re-reads the workgroup's last row
// and ignores it).  Lane = 32-input chunk.
template <int NPW>
struct XGu {
  uint4 qg[NPW], qu[NPW];
  uint32_t sg[NPW], bg[NPW], su[NPW], bu[NPW];
  uint32_t Bg[NPW], Bu[NPW];
};
template <int RW, int NPW>
__device__ __forceinline__ void x_load_gu(const XArgs& a, const uint8_t* b, int i0, XGu<NPW>& u) {
  const int lane = tid_here() & 63, wave = tid_here() >> 6;
  const int d = a.d, ng = d / a.g, r = a.r;
  const uint32_t* gq = reinterpret_cast<const uint32_t*>(b + a.lay.gate_q);
  const uint32_t* uq = reinterpret_cast<const uint32_t*>(b + a.lay.up_q);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(b + a.lay.gate_s);
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(b + a.lay.gate_b);
  const uint16_t* us = reinterpret_cast<const uint16_t*>(b + a.lay.up_s);
  const uint16_t* ub = reinterpret_cast<const uint16_t*>(b + a.lay.up_b);
  const int grp = (32 * lane) / a.g;
  const int rc = r > 0 ? r : 1, rl = lane % rc;
  const uint16_t* Bgp = reinterpret_cast<const uint16_t*>(b + (r > 0 ? a.lay.b_gate : 0));
  const uint16_t* Bup = reinterpret_cast<const uint16_t*>(b + (r > 0 ? a.lay.b_up : 0));
#pragma unroll
  for (int m = 0; m < NPW; ++m) {
    const int q = min(wave + kXWaves * m, RW - 1);
    const int row = i0 + q;
    u.qg[m] = reinterpret_cast<const uint4*>(gq + (size_t)row * (d / 8))[lane];
    u.qu[m] = reinterpret_cast<const uint4*>(uq + (size_t)row * (d / 8))[lane];
    u.sg[m] = gs[row * ng + grp];
    u.bg[m] = gb[row * ng + grp];
    u.su[m] = us[row * ng + grp];
    u.bu[m] = ub[row * ng + grp];
    u.Bg[m] = Bgp[(size_t)row * rc + rl];
    u.Bu[m] = Bup[(size_t)row * rc + rl];
  }
}

// LoRA A rows of the expert (2r rows, gate then up) or, for a router layer
// before its top-K, the workgroup's router rows (row m = router row
// j + 32 m), copied into LDS by the compute waves' direct-to-LDS loads:
// piece n (1 KiB = 64 lanes x 16 bytes) is row n / 4, quarter n % 4; compute
// wave v issues pieces v, v + 7, ...  The loads count in the wave's vmcnt.
__device__ __forceinline__ void x_stage_piece(XLds& s, const uint16_t* row, int n) {
  const int lane = tid_here() & 63;
  const uint16_t* src = row + 512 * (n & 3) + 8 * lane;
  __builtin_amdgcn_global_load_lds((x_glb_void*)(src), (x_lds_void*)(&s.arow[n >> 2][64 * (n & 3)]),
                                   16, 0, 0);
}
__device__ __forceinline__ void x_stage_a(const XArgs& a, const uint8_t* b, XLds& s) {
  const int r = a.r, wave = tid_here() >> 6;
  for (int n = wave; n < 8 * r; n += kXWaves) {
    const int ar = n >> 2;
    const uint16_t* row = reinterpret_cast<const uint16_t*>(
                              b + (ar >= r ? a.lay.a_up : a.lay.a_gate)) +
                          (size_t)(ar >= r ? ar - r : ar) * kXD;
    x_stage_piece(s, row, n);
  }
}
__device__ __forceinline__ void x_stage_router(const XArgs& a, int L, int j, XLds& s) {
  const int nrw = (a.E + kXPerXcd - 1) / kXPerXcd, wave = tid_here() >> 6;
  const uint16_t* base = a.routers[L];
  for (int n = wave; n < 4 * nrw; n += kXWaves)
    x_stage_piece(s, base + (size_t)min(j + kXPerXcd * (n >> 2), a.E - 1) * kXD, n);
}
// wait for this wave's direct-to-LDS loads (vmcnt(0); expcnt, lgkmcnt not waited)
__device__ __forceinline__ void x_wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// dot of LDS row `row` (bf16) with x (LDS), by one wave: lane l takes
// pieces l + 64 m (16 bytes each, lane-contiguous: no bank conflicts)
__device__ __forceinline__ float x_row_dot(const XLds& s, int row, const uint4 (&xv)[4]) {
  const int lane = tid_here() & 63;
  float p = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 av = s.arow[row][lane + 64 * m];
    p = dot2bf(av.x, xv[m].x, p);
    p = dot2bf(av.y, xv[m].y, p);
    p = dot2bf(av.z, xv[m].z, p);
    p = dot2bf(av.w, xv[m].w, p);
  }
  return p;
}

// down tiles of a compute wave (chunk cc = wave + 7 m of the slice, output
// row 64 j + lane); A_down over the slice (ranks wave + 7 t, lane columns
// lane * Ix/64 ..); B_down row of the lane's output row
template <int NPW, int CPL>
struct XDn {
  uint4 q[NPW];
  uint32_t sv[NPW], bv[NPW];
  uint32_t ad[kXTdRows][CPL];
  uint4 bd[2];
};
template <int RW, int NPW, int CPL>
__device__ __forceinline__ void x_load_dn(const XArgs& a, const uint8_t* b, int j, int c0,
                                          XDn<NPW, CPL>& u) {
  const int lane = tid_here() & 63, wave = tid_here() >> 6;
  const int d = a.d, NC = a.I / 32, r = a.r;
  const int o = 64 * j + lane;
#pragma unroll
  for (int m = 0; m < NPW; ++m) {
    const int cc = min(wave + kXWaves * m, RW - 1);
    const int c = c0 + cc;
    u.q[m] = reinterpret_cast<const uint4*>(b + a.lay.down_q)[((size_t)j * NC + c) * 64 + lane];
    const int grp = (32 * c) / a.g;
    u.sv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_s)[(size_t)grp * d + o];
    u.bv[m] = reinterpret_cast<const uint16_t*>(b + a.lay.down_b)[(size_t)grp * d + o];
  }
  // A_down words (2 columns) per lane and rank: CPL = RW / 4
#pragma unroll
  for (int t = 0; t < kXTdRows; ++t) {
    const int rr = min(wave + kXWaves * t, r > 0 ? r - 1 : 0);
    const uint32_t* adr = reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const uint16_t*>(b + (r > 0 ? a.lay.a_down : 0)) + (size_t)rr * a.I +
        32 * c0 + lane * 2 * CPL);
#pragma unroll
    for (int m = 0; m < CPL; ++m) u.ad[t][m] = r > 0 ? adr[m] : 0u;
  }
  const uint4* Bdp = reinterpret_cast<const uint4*>(
      reinterpret_cast<const uint16_t*>(b + (r > 0 ? a.lay.b_down : 0)) + (size_t)o * (r > 0 ? r : 8));
  u.bd[0] = Bdp[0];
  u.bd[1] = r > 8 ? Bdp[1] : make_uint4(0, 0, 0, 0);
}

// measurement aid: point p of the traced layer (one lane per call site)
#define X_MARK(p)                                                              \
  do {                                                                         \
    if (tr && lane == 0) tr[p] = __builtin_amdgcn_s_memrealtime();             \
  } while (0)

template <int RW>
__global__ __launch_bounds__(kXThreads) void k_xstep(XArgs a) {
  constexpr int NPW = (RW + kXWaves - 1) / kXWaves;  // row pairs and down tiles per compute wave
  constexpr int CPL = RW / 4;                         // A_down words per lane and rank
  __shared__ XLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool ctl = wave == kXWaves;
  const int w = blockIdx.x, X = w % 8, j = w / 8;
  const int d = a.d, K = a.K, r = a.r, E = a.E;
  const int k = X / a.P, part = X % a.P;
  const int i0 = part * a.Ix + j * RW;  // first gate/up row of this workgroup
  const int c0 = part * a.Ix / 32;      // first down chunk of the XCD slice
  const bool lead = w == 0;
  unsigned long long* yb = a.yb + (size_t)X * (kXD / 2);        // this XCD's copy of y
  unsigned long long* xh = a.xh + (size_t)X * kXMaxIx;          // this XCD's h slice
  unsigned long long* xlog = a.xlog + (size_t)X * kXMaxE;       // this XCD's router logits

  // launch prologue: the slots and weights of this workgroup's expert in
  // every prediction-routed layer; h0 (every thread holds 4 elements)
  if (ctl) {
    for (int L = lane; L < a.n_layers; L += 64) {
      int slot = -1;
      float wv = 0.f;
      if (x_is_pred(a, L)) {
        const int id = a.pred_ids[L * K + k];
        wv = a.pred_w[L * K + k];
        slot = (id >= 0 && id < E) ? a.tables[(size_t)L * E + id] : -1;
        if (slot < 0 || slot >= a.n_slots) {
          slot = -1;
          set_error(a.err, EDGE0_ERANGE);
        }
      }
      s.slot_of[L] = slot;
      s.w_of[L] = wv;
    }
    if (lane == 0) s.go = 1;
  }
  float hreg[4];
  {
    const uint2 hv = reinterpret_cast<const uint2*>(a.h)[tid];  // h[0] = h0
    hreg[0] = bf_lo(hv.x);
    hreg[1] = bf_hi(hv.x);
    hreg[2] = bf_lo(hv.y);
    hreg[3] = bf_hi(hv.y);
  }
  XGu<NPW> gu;
  XDn<NPW, CPL> dn;
  // layer 0 is a router layer (prediction-routed layers start at 1)
  if (!ctl) x_stage_router(a, 0, j, s);
  __syncthreads();

  const Q4Consts kq = q4_consts();
  for (int L = 0; L < a.n_layers; ++L) {
    const bool pred = x_is_pred(a, L);
    const bool next_pred = L + 1 < a.n_layers && x_is_pred(a, L + 1);
    const uint32_t tag = a.tag0 + (uint32_t)L;  // this layer's hand-offs
    unsigned long long* tr =
        (a.trace != nullptr && L == a.trace_layer) ? a.trace + 32 * (size_t)w : nullptr;
    if (wave == 0) X_MARK(0);
    if (wave == 0 && tr && lane == 0) tr[12] = __builtin_amdgcn_s_memtime();

    // (the previous layer's y is in s.yw, collected at its end)
    // ---- h = bf16(h + y); x = bf16(RMSNorm(h)) (all 8 waves)
    uint2 yrec, xrec;  // this thread's 4 elements of y_{L-1} and x_L (records)
    {
      float ss = 0.f;
      const uint2 yv = L > 0 ? reinterpret_cast<const uint2*>(s.yw)[tid] : make_uint2(0, 0);
      yrec = yv;
      const float yf[4] = {bf_lo(yv.x), bf_hi(yv.x), bf_lo(yv.y), bf_hi(yv.y)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (L > 0) hreg[e] = bf2f(f2bf(hreg[e] + yf[e]));
        ss = fmaf(hreg[e], hreg[e], ss);
      }
      ss = wave_sum(ss);
      if (lane == 0) s.ss[wave] = ss;
    }
    __syncthreads();
    {
      float tot = 0.f;
#pragma unroll
      for (int v = 0; v <= kXWaves; ++v) tot += s.ss[v];
      const float inv = 1.f / sqrtf(tot / (float)d + a.eps);
      const uint2 xw = make_uint2(f2bf(hreg[0] * inv) | (f2bf(hreg[1] * inv) << 16),
                                  f2bf(hreg[2] * inv) | (f2bf(hreg[3] * inv) << 16));
      reinterpret_cast<uint2*>(s.xs)[tid] = xw;
      xrec = xw;
    }
    __syncthreads();
    // the lane's x chunk (inputs 32 lane .. 32 lane + 31), raw, for the int4
    // rows; and its pieces l + 64 m for the LDS rows
    XRaw xr;
    uint4 xv[4];
    if (!ctl) {
      load_x_raw(s.xs, lane, xr);
#pragma unroll
      for (int m = 0; m < 4; ++m) xv[m] = reinterpret_cast<const uint4*>(s.xs)[lane + 64 * m];
      if (wave == 0) X_MARK(16);
      x_wait_vm();  // this wave's staged rows have landed in LDS
      if (wave == 0) X_MARK(17);
    }
    __syncthreads();  // ... and every wave's
    if (wave == 0) X_MARK(2);

    // ---- router layer: logits (each XCD all E rows, router row e of the
    // XCD's workgroup e % 32), top-K, then this layer's expert loads
    if (!pred) {
      if (ctl)
        for (int e = lane; e < E; e += 64) s.tbl[e] = a.tables[(size_t)L * E + e];
      const int nrw = (E + kXPerXcd - 1) / kXPerXcd;  // router rows per workgroup (<= 8)
      if (!ctl) {
        for (int m = wave; m < nrw; m += kXWaves) {
          const float p = wave_sum(x_row_dot(s, m, xv));
          if (lane == 0) s.lgp[m] = p;
        }
      }
      __syncthreads();
      if (ctl) {
        if (lane < nrw && j + kXPerXcd * lane < E)
          x_st64(xlog + j + kXPerXcd * lane, x_word(tag, __float_as_uint(s.lgp[lane])));
        const bool ok = x_collect<kXMaxE / 64>(a, xlog, E, tag, min(E, 32), 1,
                                               reinterpret_cast<uint32_t*>(s.lg));
        if (lane == 0) s.go = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s.go) break;
      if (wave == 0) wave_topk_n<kXMaxE / 64, false>(s.lg, E, K, s.ids, s.wts);
      __syncthreads();
      if (tid == 0) {
        const int id = s.ids[k];
        int slot = (id >= 0 && id < E) ? s.tbl[id] : -1;
        if (slot < 0 || slot >= a.n_slots) {
          slot = -1;
          set_error(a.err, EDGE0_ERANGE);
        }
        s.slot_of[L] = slot;
        s.w_of[L] = s.wts[k];
      }
      if (lead && tid < K) {
        a.exec_ids[L * K + tid] = s.ids[tid];
        a.exec_w[L * K + tid] = s.wts[tid];
      }
      __syncthreads();
      if (!ctl) {
        const uint8_t* b = x_bundle(a, s.slot_of[L]);
        x_stage_a(a, b, s);
        x_load_gu<RW, NPW>(a, b, i0, gu);
        x_load_dn<RW, NPW, CPL>(a, b, j, c0, dn);
        x_wait_vm();
      }
      __syncthreads();
    }

    // ---- LoRA A x of the expert (A rows in LDS): compute wave v takes rows
    // v, v + 7, ...
    if (!ctl && r > 0) {
      for (int ar = wave; ar < 2 * r; ar += kXWaves) {
        const float p = wave_sum(x_row_dot(s, ar, xv));
        if (lane == 0) s.t_s[ar] = p;
      }
      if (wave == 0) X_MARK(18);
    }
    __syncthreads();
    if (wave == 0) X_MARK(3);

    // ---- gate/up rows, LoRA B t, SwiGLU -> this workgroup's h words
    if (!ctl) {
      uint32_t xp[16];
      const float Xs = x_pairs(xr, xp);  // the x chunk as activation pairs, and its sum
      constexpr int R = NPW <= 2 ? 2 : 4;  // reduction width (values per lane: 2R)
      float v[2 * R];
#pragma unroll
      for (int i = 0; i < 2 * R; ++i) v[i] = 0.f;
#pragma unroll
      for (int m = 0; m < NPW; ++m) {
        const float s1 = bf2f(gu.sg[m]), b1 = bf2f(gu.bg[m]);
        const float s2 = bf2f(gu.su[m]), b2 = bf2f(gu.bu[m]);
        float G = s1 * chunk_dot128(gu.qg[m], xp, kq) + (b1 - 128.f * s1) * Xs;
        float U = s2 * chunk_dot128(gu.qu[m], xp, kq) + (b2 - 128.f * s2) * Xs;
        if (r > 0 && lane < r) {
          G += a.scale * (bf2f(gu.Bg[m]) * s.t_s[lane]);
          U += a.scale * (bf2f(gu.Bu[m]) * s.t_s[r + lane]);
        }
        v[m] = G;
        v[R + m] = U;
      }
      if (wave == 0) X_MARK(24);
      const float w1 = wave_sums_2r<R>(v);
      const float Uo = __shfl_xor(w1, 32, kWave);
      constexpr int kSpan = 64 / (2 * R);
      if (lane < 32 && (lane % kSpan) == 0) {
        const int m = lane / kSpan;
        const int q = wave + kXWaves * m;
        if (m < NPW && q < RW) {
          const float hv = silu_f(w1) * Uo;
          const uint32_t hi = f2bf(hv);
          const uint32_t lo = f2bf(hv - bf2f(hi));
          s.hrow[q] = hi | (lo << 16);
        }
      }
      if (wave == 0) X_MARK(4);
    }
    __syncthreads();

    // ---- hand-off 1: the XCD slice's h (control wave)
    if (ctl) {
      if (lane < RW) x_st64(xh + j * RW + lane, x_word(tag, s.hrow[lane]));
      X_MARK(5);
      const bool ok = x_collect<RW / 2>(a, xh, a.Ix, tag, kXPerXcd, RW, s.hw);
      if (lane == 0) s.go = ok ? 1 : 0;
      X_MARK(7);
    }
    __syncthreads();
    if (!s.go) break;

    // ---- the slice's activation pairs (as the int4 dot expects them) and
    // chunk sums; A_down h over the slice
    if (!ctl) {
      if (tid < 4 * RW) {
        const int c = tid >> 2, m = tid & 3;
        const uint32_t* src = s.hw + 32 * c + 8 * m;
        uint32_t hi[4], lo[4];
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w0 = src[2 * e], w1 = src[2 * e + 1];
          hi[e] = (w0 & 0xFFFFu) | (w1 << 16);
          lo[e] = (w0 >> 16) | (w1 & 0xFFFF0000u);
          sm += (bf_lo(w0) + bf_hi(w0)) + (bf_lo(w1) + bf_hi(w1));
        }
        pair_perm8(hi[0], hi[1], hi[2], hi[3], &s.hp[c][4 * m]);
        pair_perm8(lo[0], lo[1], lo[2], lo[3], &s.hp[c][16 + 4 * m]);
        s.hsp[c][m] = sm;
      }
      if (wave == 0) X_MARK(19);
      if (r > 0) {
        const int col0 = lane * 2 * CPL;
        float p[kXTdRows];
#pragma unroll
        for (int t = 0; t < kXTdRows; ++t) {
          p[t] = 0.f;
#pragma unroll
          for (int m = 0; m < CPL; ++m) {
            const uint32_t h0 = s.hw[col0 + 2 * m], h1 = s.hw[col0 + 2 * m + 1];
            p[t] = fmaf(bf_lo(dn.ad[t][m]), bf_lo(h0) + bf_hi(h0), p[t]);
            p[t] = fmaf(bf_hi(dn.ad[t][m]), bf_lo(h1) + bf_hi(h1), p[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < kXTdRows; ++t) {
          const float sm = wave_sum(p[t]);
          const int rr = wave + kXWaves * t;
          if (lane == 0 && rr < r) s.td_s[rr] = sm;
        }
      }
      if (wave == 0) X_MARK(20);
    }
    __syncthreads();
    if (wave == 0) X_MARK(21);

    // ---- down tiles of the slice for output rows 64 j .. 64 j + 63
    if (!ctl) {
      float part_sum = 0.f;
#pragma unroll
      for (int m = 0; m < NPW; ++m) {
        const int cc = wave + kXWaves * m;
        if (cc < RW) {
          const float sv = bf2f(dn.sv[m]), bv = bf2f(dn.bv[m]);
          const uint32_t* hp = s.hp[cc];
          const float acc = chunk_dot128(dn.q[m], hp, kq) + chunk_dot128(dn.q[m], hp + 16, kq);
          const float hs = (s.hsp[cc][0] + s.hsp[cc][1]) + (s.hsp[cc][2] + s.hsp[cc][3]);
          part_sum += sv * acc + (bv - 128.f * sv) * hs;
        }
      }
      s.red[wave][lane] = part_sum;
      if (wave == 0) X_MARK(22);
    }
    __syncthreads();
    if (wave == 0) X_MARK(23);
    if (wave == 0) {
      float D = 0.f;
#pragma unroll
      for (int v = 0; v < kXWaves; ++v) D += s.red[v][lane];
      if (r > 0) {
        const uint32_t bw[8] = {dn.bd[0].x, dn.bd[0].y, dn.bd[0].z, dn.bd[0].w,
                                dn.bd[1].x, dn.bd[1].y, dn.bd[1].z, dn.bd[1].w};
        float dl = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (2 * q < r) {
            dl += bf_lo(bw[q]) * s.td_s[2 * q];
            dl += bf_hi(bw[q]) * s.td_s[2 * q + 1];
          }
        }
        D += a.scale * dl;
      }
      const float wk = s.slot_of[L] >= 0 ? s.w_of[L] : 0.f;
      s.ypart[lane] = wk * D;
      X_MARK(8);
    }
    __syncthreads();

    // records of the layer (workgroup 0: x_L, y_{L-1}, h_L), stored after
    // this layer's last wait on the wave's own loads - a vector store counts
    // in the same in-order counter as the loads, so an earlier store would
    // delay that wait (the control wave stores its part after its polls)
    auto records = [&]() {
      reinterpret_cast<uint2*>(a.x + (size_t)L * d)[tid] = xrec;
      if (L > 0) {
        reinterpret_cast<uint2*>(a.y + (size_t)(L - 1) * d)[tid] = yrec;
        reinterpret_cast<uint2*>(a.h + (size_t)L * d)[tid] =
            make_uint2(f2bf(hreg[0]) | (f2bf(hreg[1]) << 16), f2bf(hreg[2]) | (f2bf(hreg[3]) << 16));
      }
    };
    if (lead && !ctl) records();
    // ---- hand-offs 2 and 3 (control wave): the 8 XCDs' partials of rows
    // 64 j .. 64 j + 63 summed in XCD order, bf16 y of those rows to this
    // XCD's copy, then the whole of y from it.  Meanwhile the compute waves
    // issue the next layer's weight loads, now that this layer's are used
    // (a router layer's experts are loaded after its top-K).
    if (!ctl && L + 1 < a.n_layers) {
      if (next_pred) {
        const uint8_t* b = x_bundle(a, s.slot_of[L + 1]);
        x_stage_a(a, b, s);
        x_load_gu<RW, NPW>(a, b, i0, gu);
        x_load_dn<RW, NPW, CPL>(a, b, j, c0, dn);
      } else {
        x_stage_router(a, L + 1, j, s);
      }
    }
    if (ctl) {
      unsigned long long* yp = a.yp + (size_t)(L & 1) * 8 * kXD;
      x_st64(yp + (size_t)X * kXD + 64 * j + lane, x_word(tag, __float_as_uint(s.ypart[lane])));
      X_MARK(9);
      float y = 0.f;
      int64_t polls = 0;
      bool ok = true;
      for (;;) {
        uint32_t v[8];
        bool all = true;
#pragma unroll
        for (int x8 = 0; x8 < 8; ++x8) {
          const unsigned long long wv = x_ld64(yp + (size_t)x8 * kXD + 64 * j + lane);
          all &= (uint32_t)(wv >> 32) == tag;
          v[x8] = (uint32_t)wv;
        }
        if (__builtin_amdgcn_readfirstlane((int)__all(all))) {
          y = 0.f;
#pragma unroll
          for (int x8 = 0; x8 < 8; ++x8) y += __uint_as_float(v[x8]);
          break;
        }
        if (!x_again(a, polls)) {
          ok = false;
          break;
        }
      }
      const uint32_t yb16 = f2bf(y);
      const uint32_t other = __shfl_xor(yb16, 1, kWave);
      if ((lane & 1) == 0) x_st64(yb + 32 * j + lane / 2, x_word(tag, yb16 | (other << 16)));
      X_MARK(10);
      if (ok) ok = x_collect<kXD / 128>(a, yb, kXD / 2, tag, 32, kXD / 64, s.yw);
      if (lane == 0) s.go = ok ? 1 : 0;
      X_MARK(11);
      if (tr && lane == 0) tr[13] = __builtin_amdgcn_s_memtime();
      if (lead) records();
    }
    __syncthreads();
    if (!s.go) break;
  }

  // the last layer's output (collected in s.yw at its end) and the step's
  // final hidden state (workgroup 0)
  if (lead && s.go) {
    {
      const uint2 yv = reinterpret_cast<const uint2*>(s.yw)[tid];
      const float yf[4] = {bf_lo(yv.x), bf_hi(yv.x), bf_lo(yv.y), bf_hi(yv.y)};
      uint32_t hb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hb[e] = f2bf(hreg[e] + yf[e]);
      reinterpret_cast<uint2*>(a.y + (size_t)(a.n_layers - 1) * d)[tid] = yv;
      reinterpret_cast<uint2*>(a.h + (size_t)a.n_layers * d)[tid] =
          make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    }
  }
}

// ------------------------------------------------------------ one layer
// The same work split for one layer per launch.  y reaches the next layer
// across the kernel boundary (fixed-point atomics into acc_out here, plain
// loads of it there), so the only hand-off inside a launch is h within each
// XCD (and, on a router layer, the logits within each XCD).  A hand-off word
// holds tag 1 once written; each launch clears the other layer parity's
// words for the layer after it, and the y buffer of the layer after next.
__global__ void k_pred_slots(const int32_t* __restrict__ tables, const int32_t* __restrict__ ids,
                             int32_t* __restrict__ slots, int n, int E, int K, int n_slots,
                             uint32_t* err) {
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < n * K; t += gridDim.x * blockDim.x) {
    const int L = t / K, id = ids[t];
    int slot = (id >= 0 && id < E) ? tables[(size_t)L * E + id] : -1;
    if (slot < 0 || slot >= n_slots) slot = -1;
    slots[t] = slot;
  }
  (void)err;
}

template <int RW>
__global__ __launch_bounds__(kXThreads) void k_xlayer(XLArgs la) {
  constexpr int NPW = (RW + kXWaves - 1) / kXWaves;
  constexpr int CPL = RW / 4;
  const XArgs& a = la.base;
  __shared__ XLds s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool ctl = wave == kXWaves;
  const int w = blockIdx.x, X = w % 8, j = w / 8;
  const int K = a.K, r = a.r, E = a.E;
  const int k = X / a.P, part = X % a.P;
  const int i0 = part * a.Ix + j * RW;
  const int c0 = part * a.Ix / 32;
  const bool lead = w == 0;
  constexpr uint32_t tag = 1u;
  unsigned long long* xh = la.hx + (size_t)X * kXMaxIx;
  unsigned long long* xlog = la.lx + (size_t)X * kXMaxE;
  XGu<NPW> gu;
  XDn<NPW, CPL> dn;
  int slot = -1;
  float wk = 0.f;
  unsigned long long* tr =
      (a.trace != nullptr && la.layer == a.trace_layer) ? a.trace + 32 * (size_t)w : nullptr;
  if (wave == 0) X_MARK(0);

  // ---- loads first: a prediction-routed layer's expert (slot known), or a
  // router layer's router rows and slot-table row
  if (!la.router) {
    slot = la.pred_slot[k];
    wk = la.pred_w[k];
    if (!ctl) {
      const uint8_t* b = x_bundle(a, slot);
      x_stage_a(a, b, s);
      x_load_gu<RW, NPW>(a, b, i0, gu);
      x_load_dn<RW, NPW, CPL>(a, b, j, c0, dn);
    }
  } else {
    if (!ctl) {
      const int nrw = (E + kXPerXcd - 1) / kXPerXcd;
      for (int n = wave; n < 4 * nrw; n += kXWaves)
        x_stage_piece(s, la.w_router + (size_t)min(j + kXPerXcd * (n >> 2), E - 1) * kXD, n);
    } else {
      for (int e = lane; e < E; e += 64) s.tbl[e] = la.table_row[e];
    }
  }
  // the previous layer's output (written before this launch), the residual
  float hreg[4];
  uint2 yrec = make_uint2(0, 0);
  {
    const uint2 hv = reinterpret_cast<const uint2*>(la.h_prev)[tid];
    hreg[0] = bf_lo(hv.x);
    hreg[1] = bf_hi(hv.x);
    hreg[2] = bf_lo(hv.y);
    hreg[3] = bf_hi(hv.y);
    if (la.acc_in != nullptr) {
      const ulonglong2 a0 = reinterpret_cast<const ulonglong2*>(la.acc_in)[2 * tid];
      const ulonglong2 a1 = reinterpret_cast<const ulonglong2*>(la.acc_in)[2 * tid + 1];
      const uint32_t y0 = f2bf(from_fix(a0.x)), y1 = f2bf(from_fix(a0.y));
      const uint32_t y2 = f2bf(from_fix(a1.x)), y3 = f2bf(from_fix(a1.y));
      yrec = make_uint2(y0 | (y1 << 16), y2 | (y3 << 16));
      hreg[0] = bf2f(f2bf(hreg[0] + bf2f(y0)));
      hreg[1] = bf2f(f2bf(hreg[1] + bf2f(y1)));
      hreg[2] = bf2f(f2bf(hreg[2] + bf2f(y2)));
      hreg[3] = bf2f(f2bf(hreg[3] + bf2f(y3)));
    }
  }
  // clear what the next launches start from (control wave, plain stores:
  // they are read after this launch ends)
  if (ctl) {
    if (lane < kXD / kXG) la.acc_zero[(kXD / kXG) * w + lane] = 0ull;
    for (int i = lane; i < 8 * kXMaxIx / kXG; i += 64) la.hx_clear[(8 * kXMaxIx / kXG) * w + i] = 0ull;
    if (lane < 8 * kXMaxE / kXG) la.lx_clear[(8 * kXMaxE / kXG) * w + lane] = 0ull;
  }
  // ---- x = bf16(RMSNorm(h)) (all 8 waves)
  {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(hreg[e], hreg[e], ss);
    ss = wave_sum(ss);
    if (lane == 0) s.ss[wave] = ss;
  }
  __syncthreads();
  uint2 xrec;
  {
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v <= kXWaves; ++v) tot += s.ss[v];
    const float inv = 1.f / sqrtf(tot / (float)kXD + a.eps);
    xrec = make_uint2(f2bf(hreg[0] * inv) | (f2bf(hreg[1] * inv) << 16),
                      f2bf(hreg[2] * inv) | (f2bf(hreg[3] * inv) << 16));
    reinterpret_cast<uint2*>(s.xs)[tid] = xrec;
  }
  __syncthreads();
  XRaw xr;
  uint4 xv[4];
  if (!ctl) {
    load_x_raw(s.xs, lane, xr);
#pragma unroll
    for (int m = 0; m < 4; ++m) xv[m] = reinterpret_cast<const uint4*>(s.xs)[lane + 64 * m];
    if (wave == 0) X_MARK(1);
    x_wait_vm();  // this wave's staged rows (and register weights) have landed
    if (wave == 0) X_MARK(2);
  }
  __syncthreads();

  // ---- router layer: logits, hand-off of the logits within the XCD, top-K,
  // then this layer's expert
  if (la.router) {
    const int nrw = (E + kXPerXcd - 1) / kXPerXcd;
    if (!ctl) {
      for (int m = wave; m < nrw; m += kXWaves) {
        const float p = wave_sum(x_row_dot(s, m, xv));
        if (lane == 0) s.lgp[m] = p;
      }
    }
    __syncthreads();
    if (ctl) {
      if (lane < nrw && j + kXPerXcd * lane < E)
        x_st64(xlog + j + kXPerXcd * lane, x_word(tag, __float_as_uint(s.lgp[lane])));
      const bool ok = x_collect<kXMaxE / 64>(a, xlog, E, tag, min(E, 32), 1,
                                             reinterpret_cast<uint32_t*>(s.lg));
      if (lane == 0) s.go = ok ? 1 : 0;
    }
    __syncthreads();
    if (!s.go) return;
    if (wave == 0) wave_topk_n<kXMaxE / 64, false>(s.lg, E, K, s.ids, s.wts);
    __syncthreads();
    {
      const int id = s.ids[k];
      slot = (id >= 0 && id < E) ? s.tbl[id] : -1;
      if (slot < 0 || slot >= a.n_slots) slot = -1;
      wk = s.wts[k];
    }
    if (lead && tid < K) {
      la.exec_ids[tid] = s.ids[tid];
      la.exec_w[tid] = s.wts[tid];
    }
    __syncthreads();  // every wave has read the router rows from LDS
    if (!ctl) {
      const uint8_t* b = x_bundle(a, slot);
      x_stage_a(a, b, s);
      x_load_gu<RW, NPW>(a, b, i0, gu);
      x_load_dn<RW, NPW, CPL>(a, b, j, c0, dn);
      x_wait_vm();
    }
    __syncthreads();
  }
  if (tid == 0 && slot < 0) set_error(a.err, EDGE0_ERANGE);

  // ---- LoRA A x (A rows in LDS)
  if (!ctl && r > 0) {
    for (int ar = wave; ar < 2 * r; ar += kXWaves) {
      const float p = wave_sum(x_row_dot(s, ar, xv));
      if (lane == 0) s.t_s[ar] = p;
    }
  }
  __syncthreads();
  if (wave == 0) X_MARK(3);

  // ---- gate/up rows, LoRA B t, SwiGLU -> this workgroup's h words
  if (!ctl) {
    uint32_t xp[16];
    const float Xs = x_pairs(xr, xp);
    const Q4Consts kq = q4_consts();
    constexpr int R = NPW <= 2 ? 2 : 4;
    float v[2 * R];
#pragma unroll
    for (int i = 0; i < 2 * R; ++i) v[i] = 0.f;
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const float s1 = bf2f(gu.sg[m]), b1 = bf2f(gu.bg[m]);
      const float s2 = bf2f(gu.su[m]), b2 = bf2f(gu.bu[m]);
      float G = s1 * chunk_dot128(gu.qg[m], xp, kq) + (b1 - 128.f * s1) * Xs;
      float U = s2 * chunk_dot128(gu.qu[m], xp, kq) + (b2 - 128.f * s2) * Xs;
      if (r > 0 && lane < r) {
        G += a.scale * (bf2f(gu.Bg[m]) * s.t_s[lane]);
        U += a.scale * (bf2f(gu.Bu[m]) * s.t_s[r + lane]);
      }
      v[m] = G;
      v[R + m] = U;
    }
    const float w1 = wave_sums_2r<R>(v);
    const float Uo = __shfl_xor(w1, 32, kWave);
    constexpr int kSpan = 64 / (2 * R);
    if (lane < 32 && (lane % kSpan) == 0) {
      const int m = lane / kSpan;
      const int q = wave + kXWaves * m;
      if (m < NPW && q < RW) {
        const float hv = silu_f(w1) * Uo;
        const uint32_t hi = f2bf(hv);
        const uint32_t lo = f2bf(hv - bf2f(hi));
        s.hrow[q] = hi | (lo << 16);
      }
    }
  }
  __syncthreads();

  // ---- hand-off of h within the XCD (control wave)
  if (ctl) {
    if (lane < RW) x_st64(xh + j * RW + lane, x_word(tag, s.hrow[lane]));
    X_MARK(4);
    const bool ok = x_collect<RW / 2>(a, xh, a.Ix, tag, kXPerXcd, RW, s.hw);
    if (lane == 0) s.go = ok ? 1 : 0;
    X_MARK(5);
  }
  __syncthreads();
  if (!s.go) return;

  // ---- activation pairs and chunk sums of the slice; A_down h
  if (!ctl) {
    if (tid < 4 * RW) {
      const int c = tid >> 2, m = tid & 3;
      const uint32_t* src = s.hw + 32 * c + 8 * m;
      uint32_t hi[4], lo[4];
      float sm = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = src[2 * e], w1 = src[2 * e + 1];
        hi[e] = (w0 & 0xFFFFu) | (w1 << 16);
        lo[e] = (w0 >> 16) | (w1 & 0xFFFF0000u);
        sm += (bf_lo(w0) + bf_hi(w0)) + (bf_lo(w1) + bf_hi(w1));
      }
      pair_perm8(hi[0], hi[1], hi[2], hi[3], &s.hp[c][4 * m]);
      pair_perm8(lo[0], lo[1], lo[2], lo[3], &s.hp[c][16 + 4 * m]);
      s.hsp[c][m] = sm;
    }
    if (r > 0) {
      const int col0 = lane * 2 * CPL;
      float p[kXTdRows];
#pragma unroll
      for (int t = 0; t < kXTdRows; ++t) {
        p[t] = 0.f;
#pragma unroll
        for (int m = 0; m < CPL; ++m) {
          const uint32_t h0 = s.hw[col0 + 2 * m], h1 = s.hw[col0 + 2 * m + 1];
          p[t] = fmaf(bf_lo(dn.ad[t][m]), bf_lo(h0) + bf_hi(h0), p[t]);
          p[t] = fmaf(bf_hi(dn.ad[t][m]), bf_lo(h1) + bf_hi(h1), p[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < kXTdRows; ++t) {
        const float sm = wave_sum(p[t]);
        const int rr = wave + kXWaves * t;
        if (lane == 0 && rr < r) s.td_s[rr] = sm;
      }
    }
  }
  __syncthreads();

  // ---- down tiles, weighted, into the layer's fixed-point y
  if (wave == 0) X_MARK(6);
  if (!ctl) {
    const Q4Consts kq = q4_consts();
    float part_sum = 0.f;
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const int cc = wave + kXWaves * m;
      if (cc < RW) {
        const float sv = bf2f(dn.sv[m]), bv = bf2f(dn.bv[m]);
        const uint32_t* hp = s.hp[cc];
        const float acc = chunk_dot128(dn.q[m], hp, kq) + chunk_dot128(dn.q[m], hp + 16, kq);
        const float hs = (s.hsp[cc][0] + s.hsp[cc][1]) + (s.hsp[cc][2] + s.hsp[cc][3]);
        part_sum += sv * acc + (bv - 128.f * sv) * hs;
      }
    }
    s.red[wave][lane] = part_sum;
  }
  __syncthreads();
  if (wave == 0) {
    float D = 0.f;
#pragma unroll
    for (int v = 0; v < kXWaves; ++v) D += s.red[v][lane];
    if (r > 0) {
      const uint32_t bw[8] = {dn.bd[0].x, dn.bd[0].y, dn.bd[0].z, dn.bd[0].w,
                              dn.bd[1].x, dn.bd[1].y, dn.bd[1].z, dn.bd[1].w};
      float dl = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (2 * q < r) {
          dl += bf_lo(bw[q]) * s.td_s[2 * q];
          dl += bf_hi(bw[q]) * s.td_s[2 * q + 1];
        }
      }
      D += a.scale * dl;
    }
    X_MARK(7);
    atomicAdd(la.acc_out + 64 * j + lane, to_fix((slot >= 0 ? wk : 0.f) * D));
  }
  // records (workgroup 0): x_L, y_{L-1}, h_L
  if (lead) {
    reinterpret_cast<uint2*>(la.x_out)[tid] = xrec;
    if (la.acc_in != nullptr) reinterpret_cast<uint2*>(la.y_prev_out)[tid] = yrec;
    reinterpret_cast<uint2*>(la.h_out)[tid] =
        make_uint2(f2bf(hreg[0]) | (f2bf(hreg[1]) << 16), f2bf(hreg[2]) | (f2bf(hreg[3]) << 16));
  }
}

int launch_pred_slots(const int32_t* tables, const int32_t* ids, int32_t* slots, int n_layers,
                      int E, int K, int n_slots, uint32_t* err, hipStream_t stream) {
  k_pred_slots<<<1, 256, 0, stream>>>(tables, ids, slots, n_layers, E, K, n_slots, err);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

int launch_xlayer(const XLArgs& la, hipStream_t stream, const LaunchTiming* timing) {
  auto kern = la.base.RW == 12 ? k_xlayer<12> : la.base.RW == 24 ? k_xlayer<24> : nullptr;
  if (kern == nullptr) return EDGE0_EINVAL;
  if (timing && timing->which == 1) {
    hipExtLaunchKernelGGL(kern, dim3(kXG), dim3(kXThreads), 0, stream, timing->start, timing->stop,
                          0, la);
  } else {
    kern<<<kXG, kXThreads, 0, stream>>>(la);
  }
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}

bool xstep_shape_ok(const edge0_moe_shape& sh, int n_layers) {
  if (sh.d_model != kXD || sh.n_experts < 1 || sh.n_experts > kXMaxE) return false;
  if (!(sh.top_k == 1 || sh.top_k == 2 || sh.top_k == 4 || sh.top_k == 8)) return false;
  if (!(sh.lora_rank == 0 || sh.lora_rank == 8 || sh.lora_rank == 16)) return false;
  if (sh.group_size % 32 != 0 || n_layers < 1 || n_layers > kXMaxLayers) return false;
  const int P = 8 / sh.top_k;
  if (sh.d_inter % P != 0) return false;
  const int Ix = sh.d_inter / P;
  if (Ix % 128 != 0) return false;  // RW a multiple of 4: the A_down pieces are 8-byte loads
  const int RW = Ix / 32;
  return RW == 12 || RW == 24;  // the kernel's instances (Qwen3-MoE shapes at K = 4 and 8)
}

int xstep_coresident() {
  int dev = 0, cus = 0, per = 0, coop = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EDGE0_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess)
    return EDGE0_EHIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_xstep<24>, kXThreads, 0) !=
      hipSuccess)
    return EDGE0_EHIP;
  return (coop && per * cus >= kXG) ? EDGE0_OK : EDGE0_EINVAL;
}

int launch_xstep(const XArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<XArgs*>(&a)};
  const void* fn = nullptr;
  switch (a.RW) {
    case 12: fn = reinterpret_cast<const void*>(k_xstep<12>); break;
    case 24: fn = reinterpret_cast<const void*>(k_xstep<24>); break;
    default: return EDGE0_EINVAL;
  }
  if (hipLaunchCooperativeKernel(fn, dim3(kXG), dim3(kXThreads), args, 0, stream) != hipSuccess)
    return EDGE0_EHIP;
  return EDGE0_OK;
}

}  // namespace e0
