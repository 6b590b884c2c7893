// Host side of the C ABI: shape checks, the bundle and workspace layouts,
// error strings.
#include "common.h"

namespace e0 {

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool shape_ok(const edge0_moe_shape* s) {
  if (!s) return false;
  const int d = s->d_model, E = s->n_experts, I = s->d_inter, K = s->top_k, g = s->group_size;
  if (d < 64 || d % 64 != 0 || I < 64 || I % 64 != 0) return false;
  const int cpr = d / 32;
  if (!(cpr == 8 || cpr == 16 || cpr == 32 || cpr == 64 || cpr == 128 || cpr == 192 || cpr == 256))
    return false;
  if (g < 32 || g % 32 != 0 || d % g != 0 || I % g != 0) return false;
  if (E < 1 || E > 1024 || K < 1 || K > 16 || K > E) return false;
  const int r = s->lora_rank;
  if (!(r == 0 || r == 8 || r == 16 || r == 32 || r == 64)) return false;
  if (s->lora_rank > 0 && !(s->lora_alpha == s->lora_alpha)) return false;
  if (s->head_hidden < 0 || s->head_hidden % 64 != 0) return false;
  if (s->routing == EDGE0_ROUTE_SIGMOID_GROUP) {
    const int n = s->n_groups, G = s->top_groups;
    if (n < 1 || n > 64 || E % n != 0 || E / n < 2 || G < 1 || G > n || K > G * (E / n))
      return false;
    if (!(s->route_scale == s->route_scale) || s->route_scale == INFINITY ||
        s->route_scale == -INFINITY)
      return false;
  } else if (s->routing != EDGE0_ROUTE_SOFTMAX_TOPK) {
    return false;
  }
  return true;
}

int bundle_layout(const edge0_moe_shape* s, edge0_bundle_layout* out) {
  if (!shape_ok(s) || !out) return EDGE0_EINVAL;
  const size_t d = s->d_model, I = s->d_inter, g = s->group_size, r = s->lora_rank;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return (int64_t)o;
  };
  out->gate_q = take(I * d / 2);
  out->gate_s = take(I * (d / g) * 2);
  out->gate_b = take(I * (d / g) * 2);
  out->up_q = take(I * d / 2);
  out->up_s = take(I * (d / g) * 2);
  out->up_b = take(I * (d / g) * 2);
  out->down_q = take(d * I / 2);
  out->down_s = take(d * (I / g) * 2);
  out->down_b = take(d * (I / g) * 2);
  if (r > 0) {
    out->a_gate = take(r * d * 2);
    out->b_gate = take(I * r * 2);
    out->a_up = take(r * d * 2);
    out->b_up = take(I * r * 2);
    out->a_down = take(r * I * 2);
    out->b_down = take(d * r * 2);
  } else {
    out->a_gate = out->b_gate = out->a_up = out->b_up = out->a_down = out->b_down = -1;
  }
  out->bytes = (int64_t)off;
  return EDGE0_OK;
}

WsLayout ws_layout(const edge0_moe_shape* s) {
  WsLayout L{};
  const size_t d = s->d_model, E = s->n_experts, I = s->d_inter, K = s->top_k;
  const size_t r = s->lora_rank, H = s->head_hidden;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + (bytes ? bytes : 4));
    return o;
  };
  L.err = take(4);
  L.cnt_router = take(4);
  L.cnt_head = take(4);
  L.cnt_down = take(4 * (d / 64));
  L.logits = take(4 * E);
  L.head_a = take(4 * H);
  L.head_res = take(4 * E);
  L.t_in = take(4 * K * 2 * r);
  L.t_hand = take(4 * K * 2 * r);
  L.lg_hand = take(4 * 2 * E);
  L.gu_pre = take(8 * K * I);
  L.hp_hi = take(2 * K * I);
  L.hp_lo = take(2 * K * I);
  L.hs = take(4 * K * (I / 16));
  L.tdpart = take(4 * K * (I / 16) * r);
  L.slots = take(4 * K);
  L.head_logits = take(4 * E);
  L.acc = take(8 * 2 * d);
  L.total = off;
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? EDGE0_OK : EDGE0_EHIP; }

}  // namespace e0

using namespace e0;

extern "C" const char* edge0_strerror(int code) {
  switch (code) {
    case EDGE0_OK: return "ok";
    case EDGE0_EINVAL: return "invalid argument or unsupported shape";
    case EDGE0_EHIP: return "HIP runtime or launch error";
    case EDGE0_ENOSLOT: return "every slot of the pool is pinned";
    case EDGE0_ERANGE: return "expert id or slot index out of range";
    case EDGE0_ENOMEM: return "out of memory";
    case EDGE0_ESCRATCH: return "shape needs more scratch than the static workspace holds";
    default: return "unknown error";
  }
}

extern "C" int edge0_bundle_layout_of(const edge0_moe_shape* shape, edge0_bundle_layout* out) {
  return bundle_layout(shape, out);
}

extern "C" size_t edge0_workspace_bytes(const edge0_moe_shape* shape) {
  if (!shape_ok(shape)) return 0;
  return ws_layout(shape).total;
}

extern "C" int edge0_workspace_error(void* workspace, hipStream_t stream) {
  if (!workspace) return EDGE0_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return EDGE0_EHIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return EDGE0_EHIP;
  const uint32_t zero = 0;
  if (hipMemcpy(workspace, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return EDGE0_EHIP;
  return v ? EDGE0_ERANGE : EDGE0_OK;
}
