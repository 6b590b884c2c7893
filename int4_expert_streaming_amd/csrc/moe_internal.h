// Internal interface of the MoE-layer kernels, shared by the single-layer
// entry point and the stack runtime.
#pragma once

#include "common.h"

namespace e0 {

struct MoeArgs {
  const uint8_t* pool;
  int64_t slot_bytes;
  int32_t n_slots;
  const int32_t* table;
  const int32_t* ids;
  const float* w;
  const uint16_t* x;        // normalised input (bf16 [d])
  uint16_t* y;
  const uint16_t* h_norm;   // optional: the first kernel computes x = bf16(RMSNorm(h_norm))
  uint16_t* x_out;          //   and workgroup 0 stores it here (then x == x_out)
  float eps;
  const uint16_t* h_res;  // optional residual input: h_out = bf16(h_res + y)
  uint16_t* h_out;
  int d, E, I, K, g, r;
  float scale;  // alpha / r
  edge0_bundle_layout lay;
  uint32_t* err;
  uint32_t* cnt_down;
  float* t_in;
  float* hf;
  uint16_t* hp_hi;
  uint16_t* hp_lo;
  float* hs;
  float* tdpart;
  float* td;                // A_down h, [K][r]
  uint32_t* cnt_td;         // [K]
  float* dpart;
  int S;  // down slices
};

int fill_moe_args(const edge0_moe_shape* sh, const edge0_slot_pool* pool, const int32_t* table,
                  const int32_t* ids, const float* w, const void* x, void* y, void* workspace,
                  MoeArgs* a);
// Optional event pair recorded around one of the launches (measurement aid):
// which = 1 the gate/up GEMV, 2 the down GEMV + combine, 3 the LoRA-in GEMV.
struct LaunchTiming {
  int which;
  hipEvent_t start, stop;
};
int launch_moe(const MoeArgs& a, hipStream_t stream, const LaunchTiming* timing = nullptr);

int launch_router(const edge0_moe_shape* shape, const void* w_router, const void* x,
                  const uint16_t* h_norm, uint16_t* x_out, float eps, float* logits_out,
                  int32_t* ids_out, float* w_out, void* workspace, hipStream_t stream);

}  // namespace e0
