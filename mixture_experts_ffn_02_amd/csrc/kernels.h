// Host-side launchers of the gfx950 kernels (internal; the public ABI is include/moe_lora.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_lora.h"

namespace moe {

// ---- routing ------------------------------------------------------------
struct RouteArgs {
  const uint16_t *logits;
  int T, E, K;
  int method;  // moe_lora_routing
  int n_group, topk_group;
  float rsf;
  const float *bias;
  int32_t *ids;
  float *weights;
  int32_t *offsets;
  int32_t *e2p;
  int32_t *p2e;
  int32_t *hist;  // workspace [num_wg][E]
};
size_t route_workspace_bytes(int T, int E, int K);
int route_max_tokens(int E, int K, bool dsv3);
int launch_route(const RouteArgs &a, hipStream_t s);
int launch_zero_offsets(int32_t *offsets, int E, hipStream_t s);

// ---- permute / finalize ---------------------------------------------------
int launch_permute(const uint16_t *x, const int32_t *p2e, uint16_t *x_perm, int R, int H, int K,
                   hipStream_t s);
int launch_finalize(const uint16_t *y_perm, const float *w, const int32_t *e2p, uint16_t *out,
                    int T, int H, int K, hipStream_t s);

// ---- tile-packed expert weights ---------------------------------------------------
int launch_pack_weights_fp8(const moe_lora_dims &d, const uint8_t *w1, const uint8_t *w2, uint8_t *w1p,
                            uint8_t *w2p, hipStream_t s);
int launch_pack_weights(const moe_lora_dims &d, const uint16_t *w1, const uint16_t *w2, uint16_t *w1p,
                        uint16_t *w2p, hipStream_t s);

// ---- expert FFN (grouped GEMMs + LoRA) -----------------------------------------
// fused_only: the workspace (and the call) leave out the decomposed two-stream path
size_t forward_workspace_size(const moe_lora_dims &d, const moe_lora_adapters *lora, bool fused_only = false);
int launch_forward(const moe_lora_dims &d, const uint16_t *x, const uint16_t *x_perm,
                   const int32_t *offsets, const int32_t *p2e, const uint16_t *w1,
                   const uint16_t *w2, const moe_lora_adapters *lora, uint16_t *y_perm, void *ws,
                   size_t ws_bytes, hipStream_t main, hipStream_t side,
                   const moe_lora_options *opts, const float *w1_scale = nullptr,
                   const float *w2_scale = nullptr, bool fused_only = false);

}  // namespace moe
