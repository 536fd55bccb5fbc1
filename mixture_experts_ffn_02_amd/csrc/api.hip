// extern "C" entry points of libmoe_lora.so: argument validation, then launches.
// The contract of every call is documented in include/moe_lora.h.
#include <stdint.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

// Scratch of moe_lora_forward_noalloc: one fixed device array per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel or a copy (on the host
// the name is only a stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current (scratch_address).
static __device__ __attribute__((aligned(256))) unsigned char scratch[MOE_LORA_NOALLOC_SCRATCH_BYTES];

namespace {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const moe_lora_dims *d) {
  if (!d) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (d->num_tokens < 0 || d->hidden <= 0 || d->inter <= 0 || d->num_experts <= 0 || d->top_k <= 0)
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (d->num_experts > MOE_LORA_MAX_EXPERTS || d->top_k > MOE_LORA_MAX_TOPK ||
      d->top_k > d->num_experts)
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if ((d->hidden % 8) != 0 || (d->inter % 8) != 0) return MOE_LORA_ERR_UNSUPPORTED;
  if ((long long)d->num_tokens * d->top_k > (1ll << 30)) return MOE_LORA_ERR_UNSUPPORTED;
  // one expert's gate_up matrix stays below 2 GiB (the GEMMs address it with 32-bit offsets)
  if ((long long)2 * d->inter * d->hidden >= (1ll << 30)) return MOE_LORA_ERR_UNSUPPORTED;
  return MOE_LORA_OK;
}

// slot count and ranks only (what the workspace size depends on)
int check_lora_shape(const moe_lora_adapters *l) {
  if (!l) return MOE_LORA_OK;
  if (l->num_slots < 0 || l->num_slots > MOE_LORA_MAX_SLOTS) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (l->shared_outer != 0 && l->shared_outer != 1) return MOE_LORA_ERR_INVALID_ARGUMENT;
  for (int s = 0; s < l->num_slots; ++s) {
    if (l->rank[s] <= 0) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (l->rank[s] > MOE_LORA_MAX_RANK) return MOE_LORA_ERR_UNSUPPORTED;
  }
  return MOE_LORA_OK;
}

int check_lora(const moe_lora_adapters *l) {
  int st = check_lora_shape(l);
  if (st != MOE_LORA_OK || !l || l->num_slots == 0) return st;
  if (!l->token_slot || !aligned16(l->token_slot)) return MOE_LORA_ERR_INVALID_ARGUMENT;
  for (int s = 0; s < l->num_slots; ++s) {
    if (!l->a_gate_up[s] || !l->b_gate_up[s] || !l->a_down[s] || !l->b_down[s])
      return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (!aligned16(l->a_gate_up[s]) || !aligned16(l->b_gate_up[s]) || !aligned16(l->a_down[s]) ||
        !aligned16(l->b_down[s]))
      return MOE_LORA_ERR_INVALID_ARGUMENT;
  }
  return MOE_LORA_OK;
}

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// device address of the current device's scratch array (looked up on the first call there)
int scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_LORA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_LORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_LORA_OK;
}

}  // namespace

extern "C" {

const char *moe_lora_status_string(int status) {
  switch (status) {
    case MOE_LORA_OK: return "ok";
    case MOE_LORA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_LORA_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case MOE_LORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_LORA_ERR_HIP: return "HIP launch error";
    case MOE_LORA_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more than the fixed scratch of moe_lora_forward_noalloc (64 MiB)";
    default: return "unknown status";
  }
}

int moe_lora_version(void) { return 1; }

size_t moe_lora_route_workspace_size(const moe_lora_dims *d) {
  if (check_dims(d) != MOE_LORA_OK || d->num_tokens == 0) return 0;
  return moe::route_workspace_bytes(d->num_tokens, d->num_experts, d->top_k);
}

int moe_lora_route(const moe_lora_dims *d, int routing, const moe_lora_grouped *g,
                   const uint16_t *logits, int32_t *topk_ids, float *topk_weights,
                   int32_t *expert_offsets, int32_t *e2p, int32_t *p2e, void *ws, size_t ws_bytes,
                   moe_lora_stream_t stream) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if (routing != MOE_LORA_ROUTING_RENORMALIZE && routing != MOE_LORA_ROUTING_DEEPSEEK_V3)
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  const int E = d->num_experts, K = d->top_k;
  if (d->num_tokens > moe::route_max_tokens(E, K, routing == MOE_LORA_ROUTING_DEEPSEEK_V3))
    return MOE_LORA_ERR_UNSUPPORTED;
  moe::RouteArgs a{};
  if (routing == MOE_LORA_ROUTING_DEEPSEEK_V3) {
    if (!g) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (g->n_group <= 0 || g->n_group > 64 || E % g->n_group != 0) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (g->topk_group <= 0 || g->topk_group > g->n_group) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (K > g->topk_group * (E / g->n_group)) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (g->correction_bias && !aligned16(g->correction_bias)) return MOE_LORA_ERR_INVALID_ARGUMENT;
    a.n_group = g->n_group;
    a.topk_group = g->topk_group;
    a.rsf = g->routed_scaling_factor;
    a.bias = g->correction_bias;
  }
  if (!expert_offsets || !aligned16(expert_offsets)) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (d->num_tokens > 0) {
    if (!logits || !topk_ids || !topk_weights || !e2p || !p2e) return MOE_LORA_ERR_INVALID_ARGUMENT;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_weights) || !aligned16(e2p) ||
        !aligned16(p2e))
      return MOE_LORA_ERR_INVALID_ARGUMENT;
  }
  const size_t need = moe_lora_route_workspace_size(d);
  if (ws_bytes < need) return MOE_LORA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (!ws || !aligned16(ws))) return MOE_LORA_ERR_INVALID_ARGUMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (d->num_tokens == 0) return moe::launch_zero_offsets(expert_offsets, E, s);  // all experts empty
  a.logits = logits;
  a.T = d->num_tokens;
  a.E = E;
  a.K = K;
  a.method = routing;
  a.ids = topk_ids;
  a.weights = topk_weights;
  a.offsets = expert_offsets;
  a.e2p = e2p;
  a.p2e = p2e;
  a.hist = static_cast<int32_t *>(ws);
  return moe::launch_route(a, s);
}

int moe_lora_permute(const moe_lora_dims *d, const uint16_t *x, const int32_t *p2e,
                     uint16_t *x_perm, moe_lora_stream_t stream) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if (d->num_tokens == 0) return MOE_LORA_OK;
  if (!x || !p2e || !x_perm || !aligned16(x) || !aligned16(p2e) || !aligned16(x_perm))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  return moe::launch_permute(x, p2e, x_perm, d->num_tokens * d->top_k, d->hidden, d->top_k,
                             reinterpret_cast<hipStream_t>(stream));
}

int moe_lora_pack_weights(const moe_lora_dims *d, const uint16_t *w_gate_up, const uint16_t *w_down,
                          uint16_t *w_gate_up_packed, uint16_t *w_down_packed,
                          moe_lora_stream_t stream) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if (d->hidden % 128 != 0 || d->inter % 64 != 0) return MOE_LORA_ERR_UNSUPPORTED;
  const bool do1 = w_gate_up || w_gate_up_packed, do2 = w_down || w_down_packed;
  if (!do1 && !do2) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (do1 && (!w_gate_up || !w_gate_up_packed || !aligned16(w_gate_up) || !aligned16(w_gate_up_packed)))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (do2 && (!w_down || !w_down_packed || !aligned16(w_down) || !aligned16(w_down_packed)))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  const size_t n1 = (size_t)d->num_experts * 2 * d->inter * d->hidden, n2 = (size_t)d->num_experts * d->hidden * d->inter;
  const uintptr_t a1 = reinterpret_cast<uintptr_t>(w_gate_up), b1 = reinterpret_cast<uintptr_t>(w_gate_up_packed);
  const uintptr_t a2 = reinterpret_cast<uintptr_t>(w_down), b2 = reinterpret_cast<uintptr_t>(w_down_packed);
  if ((do1 && a1 < b1 + 2 * n1 && b1 < a1 + 2 * n1) || (do2 && a2 < b2 + 2 * n2 && b2 < a2 + 2 * n2))
    return MOE_LORA_ERR_INVALID_ARGUMENT;  // in-place packing is not supported
  return moe::launch_pack_weights(*d, w_gate_up, w_down, w_gate_up_packed, w_down_packed,
                                  reinterpret_cast<hipStream_t>(stream));
}

int moe_lora_pack_weights_fp8(const moe_lora_dims *d, const uint8_t *w_gate_up, const uint8_t *w_down,
                              uint8_t *w_gate_up_packed, uint8_t *w_down_packed, moe_lora_stream_t stream) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if (d->hidden % 128 != 0 || d->inter % 128 != 0) return MOE_LORA_ERR_UNSUPPORTED;
  const bool do1 = w_gate_up || w_gate_up_packed, do2 = w_down || w_down_packed;
  if (!do1 && !do2) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (do1 && (!w_gate_up || !w_gate_up_packed || !aligned16(w_gate_up) || !aligned16(w_gate_up_packed)))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (do2 && (!w_down || !w_down_packed || !aligned16(w_down) || !aligned16(w_down_packed)))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  const size_t n1 = (size_t)d->num_experts * 2 * d->inter * d->hidden, n2 = (size_t)d->num_experts * d->hidden * d->inter;
  const uintptr_t a1 = reinterpret_cast<uintptr_t>(w_gate_up), b1 = reinterpret_cast<uintptr_t>(w_gate_up_packed);
  const uintptr_t a2 = reinterpret_cast<uintptr_t>(w_down), b2 = reinterpret_cast<uintptr_t>(w_down_packed);
  if ((do1 && a1 < b1 + n1 && b1 < a1 + n1) || (do2 && a2 < b2 + n2 && b2 < a2 + n2))
    return MOE_LORA_ERR_INVALID_ARGUMENT;  // in-place packing is not supported
  return moe::launch_pack_weights_fp8(*d, w_gate_up, w_down, w_gate_up_packed, w_down_packed,
                                      reinterpret_cast<hipStream_t>(stream));
}

size_t moe_lora_forward_workspace_size(const moe_lora_dims *d, const moe_lora_adapters *lora) {
  if (check_dims(d) != MOE_LORA_OK || check_lora_shape(lora) != MOE_LORA_OK) return 0;
  return moe::forward_workspace_size(*d, lora);
}

namespace {

// argument checks and launch shared by the bf16 and FP8 forward entry points (the FP8 one
// passes the block scales; weights are then byte arrays of E4M3 codes)
int forward_checked(const moe_lora_dims *d, const uint16_t *x, const uint16_t *x_perm,
                    const int32_t *expert_offsets, const int32_t *p2e, const void *w_gate_up,
                    const void *w_down, const float *w1_scale, const float *w2_scale,
                    const moe_lora_adapters *lora, uint16_t *y_perm, void *ws, size_t ws_bytes,
                    moe_lora_stream_t main, moe_lora_stream_t side, const moe_lora_options *opts,
                    bool fp8, bool noalloc = false) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if ((st = check_lora(lora)) != MOE_LORA_OK) return st;
  if (opts && (opts->force_path < 0 || opts->force_path > 2)) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (opts && (opts->packed_weights < 0 || opts->packed_weights > 3)) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (opts && (opts->fp8_pow2_scales < 0 || opts->fp8_pow2_scales > 1)) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (opts && opts->packed_weights && (d->hidden % 128 != 0 || d->inter % 64 != 0))
    return MOE_LORA_ERR_UNSUPPORTED;
  if (noalloc && opts && opts->force_path == 2) return MOE_LORA_ERR_UNSUPPORTED;
  if (fp8) {
    if (d->hidden % 128 != 0 || d->inter % 128 != 0) return MOE_LORA_ERR_UNSUPPORTED;
    if (d->hidden > 8192 || d->inter > 8192) return MOE_LORA_ERR_UNSUPPORTED;  // per-tile scale table
    if (opts && opts->force_path == 2) return MOE_LORA_ERR_UNSUPPORTED;
  }
  if (d->num_tokens == 0) return MOE_LORA_OK;
  if (!x && !x_perm) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if ((x && !aligned16(x)) || (x_perm && !aligned16(x_perm))) return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (!expert_offsets || !p2e || !w_gate_up || !w_down || !y_perm)
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (!aligned16(expert_offsets) || !aligned16(p2e) || !aligned16(w_gate_up) ||
      !aligned16(w_down) || !aligned16(y_perm))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  if (fp8 && (!w1_scale || !w2_scale || !aligned16(w1_scale) || !aligned16(w2_scale)))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  const size_t need = moe::forward_workspace_size(*d, lora, noalloc);
  if (noalloc) {
    if (need > (size_t)MOE_LORA_NOALLOC_SCRATCH_BYTES) return MOE_LORA_ERR_SCRATCH_TOO_SMALL;
    if ((st = scratch_address(&ws)) != MOE_LORA_OK) return st;
    ws_bytes = MOE_LORA_NOALLOC_SCRATCH_BYTES;
    side = nullptr;
  }
  if (ws_bytes < need) return MOE_LORA_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && (!ws || !aligned16(ws))) return MOE_LORA_ERR_INVALID_ARGUMENT;
  return moe::launch_forward(*d, x, x_perm, expert_offsets, p2e, static_cast<const uint16_t *>(w_gate_up),
                             static_cast<const uint16_t *>(w_down), lora, y_perm, ws, ws_bytes,
                             reinterpret_cast<hipStream_t>(main), reinterpret_cast<hipStream_t>(side), opts,
                             fp8 ? w1_scale : nullptr, fp8 ? w2_scale : nullptr, noalloc);
}

}  // namespace

int moe_lora_forward(const moe_lora_dims *d, const uint16_t *x, const uint16_t *x_perm,
                     const int32_t *expert_offsets, const int32_t *p2e, const uint16_t *w_gate_up,
                     const uint16_t *w_down, const moe_lora_adapters *lora, uint16_t *y_perm,
                     void *ws, size_t ws_bytes, moe_lora_stream_t main, moe_lora_stream_t side,
                     const moe_lora_options *opts) {
  return forward_checked(d, x, x_perm, expert_offsets, p2e, w_gate_up, w_down, nullptr, nullptr, lora,
                         y_perm, ws, ws_bytes, main, side, opts, false);
}

int moe_lora_forward_noalloc(const moe_lora_dims *d, const uint16_t *x, const uint16_t *x_perm,
                             const int32_t *expert_offsets, const int32_t *p2e, const uint16_t *w_gate_up,
                             const uint16_t *w_down, const moe_lora_adapters *lora, uint16_t *y_perm,
                             moe_lora_stream_t main, const moe_lora_options *opts) {
  return forward_checked(d, x, x_perm, expert_offsets, p2e, w_gate_up, w_down, nullptr, nullptr, lora,
                         y_perm, nullptr, 0, main, nullptr, opts, false, true);
}

int moe_lora_forward_fp8(const moe_lora_dims *d, const uint16_t *x, const uint16_t *x_perm,
                         const int32_t *expert_offsets, const int32_t *p2e, const uint8_t *w_gate_up,
                         const float *w_gate_up_scale, const uint8_t *w_down, const float *w_down_scale,
                         const moe_lora_adapters *lora, uint16_t *y_perm, void *ws, size_t ws_bytes,
                         moe_lora_stream_t main, moe_lora_stream_t side, const moe_lora_options *opts) {
  return forward_checked(d, x, x_perm, expert_offsets, p2e, w_gate_up, w_down, w_gate_up_scale,
                         w_down_scale, lora, y_perm, ws, ws_bytes, main, side, opts, true);
}

int moe_lora_finalize(const moe_lora_dims *d, const uint16_t *y_perm, const float *topk_weights,
                      const int32_t *e2p, uint16_t *out, moe_lora_stream_t stream) {
  int st = check_dims(d);
  if (st != MOE_LORA_OK) return st;
  if (d->num_tokens == 0) return MOE_LORA_OK;
  if (!y_perm || !topk_weights || !e2p || !out || !aligned16(y_perm) || !aligned16(topk_weights) ||
      !aligned16(e2p) || !aligned16(out))
    return MOE_LORA_ERR_INVALID_ARGUMENT;
  return moe::launch_finalize(y_perm, topk_weights, e2p, out, d->num_tokens, d->hidden, d->top_k,
                              reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
