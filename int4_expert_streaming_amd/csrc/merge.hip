// Merging the LoRA into the int4 weights, the alternative the pages reject:
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction", §3.3 "Recovery LoRA: Unmerged by
// Design" and its footnote 2.  The LoRA delta (alpha/r) B A is added to the
// dequantised weight and the sum is requantised to int4 with the format's
// affine scheme; what survives is measured as sum(actual * delta) /
// sum(delta^2) per projection.
//
// Per element i of a group of row o: the weight s q + b (exact in fp32),
// delta = (alpha/r) * sum_k B[o][k] A[k][i] (the products of bf16 factors
// are exact; summed in fp32, then scaled), W' = W + delta.
// Per group: s' = bf16((max W' - min W') / 15), b' = bf16(min W') (nearest,
// ties to even), q' = round((W' - b') / s') to nearest-even clipped to 0..15
// (q' = 0 when s' is 0), written into the merged bundle (the LoRA-free
// layout of the same shape).  The quotient is taken as (W' - b') times the
// hardware fp32 reciprocal of s' (a few ulp from the exact quotient, so a
// code can differ only where the quotient is that close to k + 1/2).
// sum(actual delta) and sum(delta^2), actual = s' q' + b' - W, are added in
// fp64 (k_merge_mfma first adds each lane's 4 g/16 terms of a unit in fp32).
//
// k_merge_mfma (groups of 32, 64, 96 or 128 inputs): one wave per group and
// 16 rows of one projection; the 16 x g block of delta is one small matrix
// product on the matrix cores (bf16 factors, so every product is exact, fp32
// accumulation), and the requantisation runs on the lanes that hold it.
// k_merge_requant (wider groups): one thread per group; its delta is the
// fp32 sum in rank order, so the two kernels may differ in the last bit of
// delta (both are fp32 sums of the same exact products).
// Each workgroup writes its six partial sums; k_merge_sum adds them in a
// fixed order, so the figures do not depend on scheduling.  (A completion
// counter, the last workgroup adding them, measured slower: 1152 returning
// atomics on one address serialise.)
#include "moe_internal.h"

namespace e0 {

constexpr int kMergeThreads = 256;

struct MergeArgs {
  const uint8_t* src;  // bundle with its LoRA
  uint8_t* dst;        // bundle in the LoRA-free layout
  edge0_bundle_layout ls, ld;
  int d, I, g, r;
  float scale;
  int n_gate, n_up, n_down;  // groups per projection
  int u_gu, n_units;         // matrix-core path: units (16 rows x 1 group) per gate/up, in all
  double* partial;           // [gridDim][6]
};

// word w (8 inputs) of group G of row o: index into the projection's u32
// array (row-major [out][in/8] for gate/up, 1 KiB tiles [d/64][I/32][64][4]
// for down)
__device__ __forceinline__ size_t merge_word(int proj, int o, int G, int w, int d, int I, int g) {
  const int j = G * g + 8 * w;  // first input of the word
  if (proj < 2) return (size_t)o * (d / 8) + (size_t)(j >> 3);
  return (((size_t)(o >> 6) * (I / 32) + (j >> 5)) * 64 + (o & 63)) * 4 + ((j & 31) >> 3);
}

__global__ __launch_bounds__(kMergeThreads) void k_merge_requant(MergeArgs a) {
#pragma clang fp contract(off)
  __shared__ double red[kMergeThreads / 64][6];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * kMergeThreads + tid;
  const int d = a.d, I = a.I, g = a.g, r = a.r;
  double sad = 0.0, sdd = 0.0;
  int proj = -1;
  if (t < a.n_gate + a.n_up + a.n_down) {
    proj = t < a.n_gate ? 0 : (t < a.n_gate + a.n_up ? 1 : 2);
    const int u = t - (proj == 0 ? 0 : (proj == 1 ? a.n_gate : a.n_gate + a.n_up));
    const int n_in = proj < 2 ? d : I;  // inputs per row
    const int gpr = n_in / g;           // groups per row
    const int o = u / gpr, G = u % gpr; // row, group
    const edge0_bundle_layout& ls = a.ls;
    const edge0_bundle_layout& ld = a.ld;
    const int64_t oq = proj == 0 ? ls.gate_q : (proj == 1 ? ls.up_q : ls.down_q);
    const int64_t os = proj == 0 ? ls.gate_s : (proj == 1 ? ls.up_s : ls.down_s);
    const int64_t ob = proj == 0 ? ls.gate_b : (proj == 1 ? ls.up_b : ls.down_b);
    const int64_t dq = proj == 0 ? ld.gate_q : (proj == 1 ? ld.up_q : ld.down_q);
    const int64_t ds = proj == 0 ? ld.gate_s : (proj == 1 ? ld.up_s : ld.down_s);
    const int64_t db = proj == 0 ? ld.gate_b : (proj == 1 ? ld.up_b : ld.down_b);
    const int64_t oa = proj == 0 ? ls.a_gate : (proj == 1 ? ls.a_up : ls.a_down);
    const int64_t obb = proj == 0 ? ls.b_gate : (proj == 1 ? ls.b_up : ls.b_down);
    const uint32_t* qs = reinterpret_cast<const uint32_t*>(a.src + oq);
    uint32_t* qd = reinterpret_cast<uint32_t*>(a.dst + dq);
    const size_t si = proj < 2 ? (size_t)o * gpr + G : (size_t)G * d + o;  // scale/bias index
    const uint16_t* A = r > 0 ? reinterpret_cast<const uint16_t*>(a.src + oa) : nullptr;
    const uint16_t* B = r > 0 ? reinterpret_cast<const uint16_t*>(a.src + obb) + (size_t)o * r : nullptr;
    const float s = bf2f(reinterpret_cast<const uint16_t*>(a.src + os)[si]);
    const float b = bf2f(reinterpret_cast<const uint16_t*>(a.src + ob)[si]);
    // delta of input i (fp32, rank order), the same in both passes
    auto delta = [&](int i) {
      float dl = 0.f;
      for (int k = 0; k < r; ++k) dl = fmaf(bf2f(B[k]), bf2f(A[(size_t)k * n_in + i]), dl);
      return dl * a.scale;
    };
    const int nw = g / 8;
    float lo = INFINITY, hi = -INFINITY;
    for (int w = 0; w < nw; ++w) {
      const uint32_t word = qs[merge_word(proj, o, G, w, d, I, g)];
      for (int e = 0; e < 8; ++e) {
        const float Wm = fmaf(s, (float)((word >> (4 * e)) & 15u), b) + delta(G * g + 8 * w + e);
        lo = fminf(lo, Wm);
        hi = fmaxf(hi, Wm);
      }
    }
    const uint32_t s2b = f2bf((hi - lo) / 15.f), b2b = f2bf(lo);
    const float s2 = bf2f(s2b), b2 = bf2f(b2b);
    reinterpret_cast<uint16_t*>(a.dst + ds)[si] = (uint16_t)s2b;
    reinterpret_cast<uint16_t*>(a.dst + db)[si] = (uint16_t)b2b;
    for (int w = 0; w < nw; ++w) {
      const size_t wi = merge_word(proj, o, G, w, d, I, g);
      const uint32_t word = qs[wi];
      uint32_t out = 0;
      for (int e = 0; e < 8; ++e) {
        const float W = fmaf(s, (float)((word >> (4 * e)) & 15u), b);  // exact
        const float dl = delta(G * g + 8 * w + e);
        const float Wm = W + dl;
        const float rs2 = s2 > 0.f ? __builtin_amdgcn_rcpf(s2) : 0.f;
        const float qf = fminf(fmaxf(rintf((Wm - b2) * rs2), 0.f), 15.f);
        const uint32_t q2 = (uint32_t)qf;
        out |= q2 << (4 * e);
        const double act = ((double)s2 * (double)q2 + (double)b2) - (double)W;
        sad += act * (double)dl;
        sdd += (double)dl * (double)dl;
      }
      qd[wi] = out;
    }
  }
  // per-projection sums of the workgroup, in lane then wave order
  double v[6];
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    v[2 * p] = proj == p ? sad : 0.0;
    v[2 * p + 1] = proj == p ? sdd : 0.0;
  }
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    double x = v[q];
    for (int o2 = 32; o2 >= 1; o2 >>= 1) x += __shfl_xor(x, o2, kWave);
    if (lane == 0) red[wave][q] = x;
  }
  __syncthreads();
  if (tid < 6) {
    double x = 0.0;
    for (int w2 = 0; w2 < kMergeThreads / 64; ++w2) x += red[w2][tid];
    a.partial[(size_t)blockIdx.x * 6 + tid] = x;
  }
}

// one group of one projection: the offsets of its arrays in both bundles
struct MergeProj {
  const uint32_t* qs;
  uint32_t* qd;
  const uint16_t *ss, *sb, *A, *B;
  uint16_t *ds, *db;
};

__device__ __forceinline__ MergeProj merge_proj(const MergeArgs& a, int proj) {
  const edge0_bundle_layout& ls = a.ls;
  const edge0_bundle_layout& ld = a.ld;
  MergeProj m;
  const int64_t oq = proj == 0 ? ls.gate_q : (proj == 1 ? ls.up_q : ls.down_q);
  const int64_t os = proj == 0 ? ls.gate_s : (proj == 1 ? ls.up_s : ls.down_s);
  const int64_t ob = proj == 0 ? ls.gate_b : (proj == 1 ? ls.up_b : ls.down_b);
  const int64_t dq = proj == 0 ? ld.gate_q : (proj == 1 ? ld.up_q : ld.down_q);
  const int64_t ds = proj == 0 ? ld.gate_s : (proj == 1 ? ld.up_s : ld.down_s);
  const int64_t db = proj == 0 ? ld.gate_b : (proj == 1 ? ld.up_b : ld.down_b);
  const int64_t oa = proj == 0 ? ls.a_gate : (proj == 1 ? ls.a_up : ls.a_down);
  const int64_t obb = proj == 0 ? ls.b_gate : (proj == 1 ? ls.b_up : ls.b_down);
  m.qs = reinterpret_cast<const uint32_t*>(a.src + oq);
  m.qd = reinterpret_cast<uint32_t*>(a.dst + dq);
  m.ss = reinterpret_cast<const uint16_t*>(a.src + os);
  m.sb = reinterpret_cast<const uint16_t*>(a.src + ob);
  m.ds = reinterpret_cast<uint16_t*>(a.dst + ds);
  m.db = reinterpret_cast<uint16_t*>(a.dst + db);
  m.A = a.r > 0 ? reinterpret_cast<const uint16_t*>(a.src + oa) : nullptr;
  m.B = a.r > 0 ? reinterpret_cast<const uint16_t*>(a.src + obb) : nullptr;
  return m;
}

constexpr int kMergeRows = 16;  // rows of one projection per wave
constexpr int kMergeWaves = 4;  // waves per workgroup

typedef __attribute__((ext_vector_type(8))) __bf16 mg_bf16x8;
typedef __attribute__((ext_vector_type(4))) short mg_bf16x4;  // bf16 bits
typedef __attribute__((ext_vector_type(4))) float mg_f32x4;

// Order-preserving integer keys of finite floats (the magnitude bits of a
// negative value flipped), so a range step is one integer min or max with a
// DPP source and needs no float canonicalisation; the map is its own inverse.
__device__ __forceinline__ int f2key(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key2f(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
// min and max over the 16 lanes of a row of the wave (xor 1, xor 2, then the
// half-row and row mirrors): every lane of the 16 ends with the result
__device__ __forceinline__ void row16_minmax(float& lo, float& hi) {
  int kl = f2key(lo), kh = f2key(hi);
  kl = min(kl, dpp_i<0xB1>(kl));
  kh = max(kh, dpp_i<0xB1>(kh));
  kl = min(kl, dpp_i<0x4E>(kl));
  kh = max(kh, dpp_i<0x4E>(kh));
  kl = min(kl, dpp_i<0x141>(kl));
  kh = max(kh, dpp_i<0x141>(kh));
  kl = min(kl, dpp_i<0x140>(kl));
  kh = max(kh, dpp_i<0x140>(kh));
  lo = key2f(kl);
  hi = key2f(kh);
}

// One wave: 16 rows (row0 + 0..15) of one projection and one group of
// g = 16 NB inputs.  The delta of the 16 x g block is B[rows][0..r) times
// A[0..r)[group] on the matrix cores, per 16-input block one
// v_mfma_f32_16x16x16_bf16 for r <= 16 or v_mfma_f32_16x16x32_bf16 per
// chunk of 32 ranks (zero past r): lane l = (n = l % 16, j = l / 16)
// supplies row n's ranks 4j .. 4j + 3 (8j .. 8j + 7 of a chunk) and column
// n's same ranks, and holds the products for rows 4j + v (v < 4) at input n
// of each block m.  The
// lane's 4 NB elements are then requantised; each group's range is the
// lane's and then its 16-lane row's.  The codes are written as bytes into
// the wave's LDS tile [16][g] and read back 8 at a time as code words.
// DOWN selects the tiled layout of the down projection (code word of row o,
// inputs 8w .. 8w + 7 at ((o / 64) (I / 32) + w / 4) 256 + (o % 64) 4 + w % 4)
// or the row-major one of gate and up (o d / 8 + w), so a block's word
// offsets are constants.
template <int RK, int NB, bool DOWN>
__device__ __forceinline__ void merge_block(const MergeArgs& a, const MergeProj& m, int row0,
                                            int G, uint8_t* trow, float& sad, float& sdd) {
#pragma clang fp contract(off)
  constexpr int g = 16 * NB;
  constexpr int KC = (RK + 31) / 32;  // rank chunks
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, j = lane >> 4;
  const int d = a.d, I = a.I;
  const int n_in = DOWN ? I : d;
  const int gpr = n_in / g;
  // word index of (row o, word w of the group) in the projection's u32 array
  auto word_at = [&](int o, int w) -> size_t {
    if (DOWN)
      return ((size_t)(o >> 6) * (I / 32) + (G * g + 8 * w) / 32) * 256 + (o & 63) * 4 + (w & 3);
    return (size_t)o * (d / 8) + (size_t)G * (g / 8) + w;
  };
  auto sb_at = [&](int o) -> size_t { return DOWN ? (size_t)G * d + o : (size_t)o * gpr + G; };
  // every load first: the operands, the code words, the scales and biases.
  // Ranks 8 and 16 take one v_mfma_f32_16x16x16_bf16 per block (lane (n, j)
  // supplies ranks 4j .. 4j + 3), wider ranks chunks of 32.
  constexpr bool K16 = RK > 0 && RK <= 16;
  mg_bf16x8 opb[KC > 0 ? KC : 1], opa[KC > 0 ? KC : 1][NB];
  mg_bf16x4 opb4, opa4[NB];
  if constexpr (K16) {
    const int k0 = 4 * j;
    const bool kv = k0 < RK;
    const int kc = kv ? k0 : 0;
    const uint2 braw = *reinterpret_cast<const uint2*>(m.B + (size_t)(row0 + n) * RK + kc);
    opb4 = __builtin_bit_cast(mg_bf16x4, kv ? braw : make_uint2(0, 0));
    const uint16_t* ab = m.A + (size_t)kc * n_in + (size_t)G * g + n;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      const uint32_t w0 = (uint32_t)ab[16 * mb] | ((uint32_t)ab[(size_t)n_in + 16 * mb] << 16);
      const uint32_t w1 = (uint32_t)ab[(size_t)2 * n_in + 16 * mb] |
                          ((uint32_t)ab[(size_t)3 * n_in + 16 * mb] << 16);
      opa4[mb] = __builtin_bit_cast(mg_bf16x4, kv ? make_uint2(w0, w1) : make_uint2(0, 0));
    }
  }
#pragma unroll
  for (int c = 0; c < (K16 ? 0 : KC); ++c) {
    const int k0 = 32 * c + 8 * j;  // this lane's first rank of the chunk
    const bool kv = k0 < RK;
    const int kc = kv ? k0 : 0;
    const uint4 braw = *reinterpret_cast<const uint4*>(m.B + (size_t)(row0 + n) * RK + kc);
    opb[c] = __builtin_bit_cast(mg_bf16x8, kv ? braw : make_uint4(0, 0, 0, 0));
    const uint16_t* ab = m.A + (size_t)kc * n_in + (size_t)G * g + n;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      uint32_t w4[4];  // loaded whatever kv (ranks clamped to 0 .. 7), zeroed after
#pragma unroll
      for (int t = 0; t < 4; ++t)
        w4[t] = (uint32_t)ab[(size_t)(2 * t) * n_in + 16 * mb] |
                ((uint32_t)ab[(size_t)(2 * t + 1) * n_in + 16 * mb] << 16);
      opa[c][mb] = __builtin_bit_cast(
          mg_bf16x8, kv ? make_uint4(w4[0], w4[1], w4[2], w4[3]) : make_uint4(0, 0, 0, 0));
    }
  }
  uint32_t wq[4][NB];
  uint32_t sv[4], bv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int o = row0 + 4 * j + v;
    const uint32_t* qrow = m.qs + word_at(o, n >> 3);
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
      wq[v][mb] = qrow[DOWN ? (mb >> 1) * 256 + 2 * (mb & 1) : 2 * mb];
    sv[v] = m.ss[sb_at(o)];
    bv[v] = m.sb[sb_at(o)];
  }
  // the delta: acc[mb][v] = sum over ranks of B[row0 + 4j + v][k] A[k][16 mb + n]
  mg_f32x4 acc[NB];
#pragma unroll
  for (int mb = 0; mb < NB; ++mb) {
    acc[mb] = mg_f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (K16) {
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(opb4, opa4[mb], acc[mb], 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < KC; ++c)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opb[c], opa[c][mb], acc[mb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float s = bf2f(sv[v]), b = bf2f(bv[v]);
    float W[NB], dl[NB], Wm[NB];
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      W[mb] = fmaf(s, (float)((wq[v][mb] >> (4 * (n & 7))) & 15u), b);  // exact
      dl[mb] = acc[mb][v] * a.scale;  // rounded, then added (no contraction here)
      Wm[mb] = W[mb] + dl[mb];
      lo = fminf(lo, Wm[mb]);
      hi = fmaxf(hi, Wm[mb]);
    }
    row16_minmax(lo, hi);
    const uint32_t s2b = f2bf((hi - lo) / 15.f), b2b = f2bf(lo);
    const float s2 = bf2f(s2b), b2 = bf2f(b2b);
    const float rs2 = s2 > 0.f ? __builtin_amdgcn_rcpf(s2) : 0.f;
    const int o = row0 + 4 * j + v;
    if (n == 0) {
      m.ds[sb_at(o)] = (uint16_t)s2b;
      m.db[sb_at(o)] = (uint16_t)b2b;
    }
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
      const float qf = fminf(fmaxf(rintf((Wm[mb] - b2) * rs2), 0.f), 15.f);
      const float act = fmaf(s2, qf, b2) - W[mb];
      sad = fmaf(act, dl[mb], sad);
      sdd = fmaf(dl[mb], dl[mb], sdd);
      trow[(4 * j + v) * g + 16 * mb + n] = (uint8_t)qf;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the code words: word t of row rho holds the row's inputs 8t .. 8t + 7
#pragma unroll
  for (int t = 0; t < g / 32; ++t) {
    const int wi = lane + kWave * t, rho = wi / (g / 8), tw = wi - rho * (g / 8);
    const uint2 by = *reinterpret_cast<const uint2*>(trow + rho * g + 8 * tw);
    const uint32_t lo2 = by.x | (by.x >> 4), hi2 = by.y | (by.y >> 4);
    m.qd[word_at(row0 + rho, tw)] = __builtin_amdgcn_perm(hi2, lo2, 0x06040200u);
  }
}

// Where the registers allow it without spilling (up to 64 inputs per group
// and rank 32, or 32 inputs and rank 64, or no LoRA), at most 96 VGPRs: 5
// waves per SIMD, so a Qwen3-MoE-shaped expert's 4608 waves are resident at
// once.
constexpr int merge_waves_per_simd(int RK, int NB) {
  return NB * ((RK + 31) / 32 + 1) <= 8 ? 5 : 1;
}

template <int RK, int NB>
__global__ __launch_bounds__(kMergeWaves * kWave, merge_waves_per_simd(RK, NB))
void k_merge_mfma(MergeArgs a) {
  constexpr int g = 16 * NB;
  __shared__ double red[kMergeWaves][2];
  __shared__ __align__(16) uint8_t tile[kMergeWaves][kMergeRows * g];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // XCD-aware order: consecutive workgroups go to different XCDs (round-robin
  // over 8), so logical block L = (id % 8) (n / 8) + id / 8 gives each XCD a
  // contiguous range of units, whole 16-row blocks whose B rows then come
  // from memory once
  const int nb = gridDim.x;
  const int bid = nb % 8 == 0 ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
  const int unit = bid * kMergeWaves + wave;
  float sad = 0.f, sdd = 0.f;  // this lane's 4 NB terms
  if (unit < a.n_units) {
    // unit -> (projection, block of 16 rows, group); the group runs fastest
    const int proj = unit < a.u_gu ? 0 : (unit < 2 * a.u_gu ? 1 : 2);
    const int u = unit - (proj == 0 ? 0 : (proj == 1 ? a.u_gu : 2 * a.u_gu));
    const int gpr = (proj < 2 ? a.d : a.I) / g;
    const int rb = u / gpr, G = u - rb * gpr;
    const MergeProj m = merge_proj(a, proj);
    if (proj < 2)
      merge_block<RK, NB, false>(a, m, rb * kMergeRows, G, tile[wave], sad, sdd);
    else
      merge_block<RK, NB, true>(a, m, rb * kMergeRows, G, tile[wave], sad, sdd);
  }
  // the workgroup's two sums in fp64, in lane then wave order, filed under
  // the waves' projections
  double xs = (double)sad, xd = (double)sdd;
#pragma unroll
  for (int o2 = 32; o2 >= 1; o2 >>= 1) {
    xs += __shfl_xor(xs, o2, kWave);
    xd += __shfl_xor(xd, o2, kWave);
  }
  if (lane == 0) {
    red[wave][0] = xs;
    red[wave][1] = xd;
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    const int q = threadIdx.x;
    double x = 0.0;
    for (int w2 = 0; w2 < kMergeWaves; ++w2) {
      const int uw = bid * kMergeWaves + w2;
      const int pw = uw < a.u_gu ? 0 : (uw < 2 * a.u_gu ? 1 : 2);
      if (uw < a.n_units && pw == (q >> 1)) x += red[w2][q & 1];
    }
    a.partial[(size_t)bid * 6 + q] = x;
  }
}

// The six sums over the workgroups' partials: workgroup q adds figure q,
// thread t the partials t, t + 256, ... in order (loaded 8 at a time, so a
// batch is one memory round trip), then each wave's fixed butterfly and the
// four waves in order.
constexpr int kSumThreads = 256;
__global__ __launch_bounds__(kSumThreads) void k_merge_sum(const double* partial, int n,
                                                            double* out) {
  constexpr int kBatch = 8;
  __shared__ double ws[kSumThreads / kWave];
  const int q = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1);
  double x = 0.0;
  for (int i0 = 0; i0 < n; i0 += kBatch * kSumThreads) {
    double v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + t + kSumThreads * b;
      v[b] = partial[(size_t)(i < n ? i : n - 1) * 6 + q];
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (i0 + t + kSumThreads * b < n) x += v[b];
  }
  for (int o2 = 32; o2 >= 1; o2 >>= 1) x += __shfl_xor(x, o2, kWave);
  if (lane == 0) ws[t >> 6] = x;
  __syncthreads();
  if (t == 0) {
    double y = 0.0;
    for (int w = 0; w < kSumThreads / kWave; ++w) y += ws[w];
    out[q] = y;
  }
}

}  // namespace e0

using namespace e0;

namespace {

// the matrix-core kernel takes groups of 32, 64, 96 or 128 inputs
bool merge_wave_ok(const edge0_moe_shape* s) { return s->group_size <= 128; }

size_t merge_grid(const edge0_moe_shape* s) {
  const size_t groups = (size_t)s->d_inter * (s->d_model / s->group_size) * 2 +
                        (size_t)s->d_model * (s->d_inter / s->group_size);
  if (merge_wave_ok(s)) {
    const size_t units = groups / kMergeRows;  // d_model and d_inter are multiples of 64
    return (units + kMergeWaves - 1) / kMergeWaves;
  }
  return (groups + kMergeThreads - 1) / kMergeThreads;
}

template <int RK>
void launch_merge_wave(const MergeArgs& a, int grid, hipStream_t stream) {
  switch (a.g) {
    case 32: k_merge_mfma<RK, 2><<<grid, kMergeWaves * kWave, 0, stream>>>(a); break;
    case 64: k_merge_mfma<RK, 4><<<grid, kMergeWaves * kWave, 0, stream>>>(a); break;
    case 96: k_merge_mfma<RK, 6><<<grid, kMergeWaves * kWave, 0, stream>>>(a); break;
    default: k_merge_mfma<RK, 8><<<grid, kMergeWaves * kWave, 0, stream>>>(a); break;
  }
}

}  // namespace

extern "C" size_t edge0_merge_workspace_bytes(const edge0_moe_shape* shape) {
  if (!shape || !shape_ok(shape)) return 0;
  return merge_grid(shape) * 6 * sizeof(double);
}

extern "C" int edge0_merge_requant(const edge0_moe_shape* shape, const void* src_bundle,
                                   void* dst_bundle, double* stats_out, void* workspace,
                                   hipStream_t stream) {
  if (!shape || !shape_ok(shape) || !src_bundle || !dst_bundle ||
      !stats_out || !workspace || src_bundle == dst_bundle)
    return EDGE0_EINVAL;
  MergeArgs a{};
  edge0_moe_shape s0 = *shape;
  s0.lora_rank = 0;
  if (bundle_layout(shape, &a.ls) != EDGE0_OK || bundle_layout(&s0, &a.ld) != EDGE0_OK)
    return EDGE0_EINVAL;
  a.src = static_cast<const uint8_t*>(src_bundle);
  a.dst = static_cast<uint8_t*>(dst_bundle);
  a.d = shape->d_model;
  a.I = shape->d_inter;
  a.g = shape->group_size;
  a.r = shape->lora_rank;
  a.scale = a.r > 0 ? shape->lora_alpha / (float)a.r : 0.f;
  a.n_gate = a.I * (a.d / a.g);
  a.n_up = a.n_gate;
  a.n_down = a.d * (a.I / a.g);
  a.u_gu = a.n_gate / kMergeRows;
  a.n_units = (a.n_gate + a.n_up + a.n_down) / kMergeRows;
  a.partial = static_cast<double*>(workspace);
  const int grid = (int)merge_grid(shape);
  if (merge_wave_ok(shape)) {
    switch (a.r) {
      case 0: launch_merge_wave<0>(a, grid, stream); break;
      case 8: launch_merge_wave<8>(a, grid, stream); break;
      case 16: launch_merge_wave<16>(a, grid, stream); break;
      case 32: launch_merge_wave<32>(a, grid, stream); break;
      default: launch_merge_wave<64>(a, grid, stream); break;
    }
  } else {
    k_merge_requant<<<grid, kMergeThreads, 0, stream>>>(a);
  }
  E0_CHECK_LAUNCH();
  k_merge_sum<<<6, kSumThreads, 0, stream>>>(a.partial, grid, stats_out);
  E0_CHECK_LAUNCH();
  return EDGE0_OK;
}
