/*
 * moe_lora.h — C ABI of the MI355X (gfx950) routed MoE-LoRA expert layer.
 *
 * The layer (one MoE block with per-expert LoRA adapters) is split into the four
 * stages the pages' bf16 pipeline names — routing -> permute -> gate_up GEMM,
 * activation, down GEMM -> finalize (sglang PR "[LoRA] bf16 MoE-LoRA for trtllm
 * backend with two-stream overlap + routing opts", Files-changed table, launcher
 * row; section 1(A) single-stream flow) — as four calls:
 *
 *   moe_lora_route     top-k routing + expert-sorted pack, one launch
 *   moe_lora_permute   gather token rows into expert-sorted order
 *   moe_lora_forward   gate_up GEMM + LoRA delta (before SwiGLU) + SwiGLU
 *                      + down GEMM + down LoRA delta, unweighted, permuted rows
 *   moe_lora_finalize  routing-weighted top-k reduction back to token order
 *
 * Conventions (all calls):
 *   - Tensor pointers are DEVICE pointers unless marked [host].  bf16 tensors are
 *     passed as uint16_t bit patterns.  Every device pointer must be 16-byte aligned.
 *   - All layouts are row-major with the last dimension contiguous.
 *   - The caller owns every buffer, including the workspaces sized by the
 *     *_workspace_size functions; the library never allocates device memory
 *     (the capture-safety lesson of sglang PR "[LoRA] Fix experimental fast-path
 *     multi-adapter correctness ...", Motivation item 3 and Modifications).  The one
 *     exception is static: the fixed scratch array of moe_lora_forward_noalloc, part
 *     of the library's code object on each GPU.
 *   - Work is enqueued on the given stream(s) (a hipStream_t passed as void*;
 *     NULL = the null stream) and is asynchronous.  No call synchronizes the device.
 *   - Errors: arguments are validated on the host first; on any error nothing is
 *     enqueued and a nonzero moe_lora_status is returned.  A launch failure returns
 *     MOE_LORA_ERR_HIP.  Device-side faults surface at the caller's next
 *     synchronization.  num_tokens == 0 is a valid no-op.
 *   - Row indices: the expanded index of (token t, choice j) is t*top_k + j (vLLM API
 *     page "trtllm_lora_moe", _unpermute_activation).  "Permuted" rows are ordered by
 *     expert, and inside one expert by ascending expanded index.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moe_lora_stream_t; /* hipStream_t */

typedef enum {
  MOE_LORA_OK = 0,
  MOE_LORA_ERR_INVALID_ARGUMENT = 1,
  MOE_LORA_ERR_UNSUPPORTED = 2,
  MOE_LORA_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_LORA_ERR_HIP = 4,
  MOE_LORA_ERR_SCRATCH_TOO_SMALL = 5 /* moe_lora_forward_noalloc: the problem needs more scratch */
} moe_lora_status;

/* Routing methods (vLLM API page "trtllm_lora_moe", TrtLlmBf16LoRAExperts
 * ._supports_routing_method).  RenormalizeNaive computes the same ids and weights
 * as Renormalize (softmax is monotone), so it shares the enum value. */
typedef enum {
  MOE_LORA_ROUTING_RENORMALIZE = 0,
  MOE_LORA_ROUTING_DEEPSEEK_V3 = 1
} moe_lora_routing;

#define MOE_LORA_MAX_SLOTS 8
#define MOE_LORA_MAX_RANK 64   /* direct-expand limit, section 2 of the bf16 PR */
#define MOE_LORA_MAX_EXPERTS 512
#define MOE_LORA_MAX_TOPK 32
/* fixed per-GPU scratch of moe_lora_forward_noalloc (64 MiB) */
#define MOE_LORA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Problem size (the (E, M, N=2I, K=H, topk) tuple of the vLLM API page,
 * _TrtLlmLoRAExpertsBase.moe_problem_size). */
typedef struct {
  int32_t num_tokens;  /* T >= 0 */
  int32_t hidden;      /* H, multiple of 8 */
  int32_t inter;       /* I, multiple of 8 (expert intermediate size); 2*I*H < 2^30 */
  int32_t num_experts; /* E in [1, MOE_LORA_MAX_EXPERTS] */
  int32_t top_k;       /* k in [1, min(E, MOE_LORA_MAX_TOPK)] */
} moe_lora_dims;

/* DeepSeek-V3 grouped routing parameters (the n_group / topk_group /
 * routed_scaling_factor arguments of the routed op on the vLLM API page). */
typedef struct {
  int32_t n_group;              /* E % n_group == 0, n_group <= 64 */
  int32_t topk_group;           /* 1 <= topk_group <= n_group */
  float routed_scaling_factor;  /* folded into the returned weights */
  const float *correction_bias; /* [E] fp32, selection only; NULL = zeros */
} moe_lora_grouped;

/* Resident LoRA adapter slots.  A token's slot comes from token_slot[t]; a value
 * outside [0, num_slots) means "no adapter" for that token (the -1 sentinel of the
 * bf16 PR, section 2).  Slot, rank and scaling are looked up per token (sglang PR
 * "[LoRA] Fix experimental fast-path multi-adapter correctness ...", Motivation
 * item 2).  Weights are stored per slot, compactly (no padding to the largest rank):
 *   a_gate_up[s]: [E, rank[s], H]     b_gate_up[s]: [E, 2I, rank[s]]  (rows: gate then up)
 *   a_down[s]:    [E, rank[s], I]     b_down[s]:    [E, H, rank[s]]
 * The gate_up delta s*B1(A1 x) is added before SwiGLU and is not routing-weighted;
 * the down delta s*B2(A2 h) is added to the expert output (so finalize weights it). */
typedef struct {
  int32_t num_slots;           /* 0..MOE_LORA_MAX_SLOTS; 0 = base MoE */
  const int32_t *token_slot;   /* [T] */
  int32_t rank[MOE_LORA_MAX_SLOTS];   /* 1..MOE_LORA_MAX_RANK */
  float scaling[MOE_LORA_MAX_SLOTS];
  const uint16_t *a_gate_up[MOE_LORA_MAX_SLOTS];
  const uint16_t *b_gate_up[MOE_LORA_MAX_SLOTS];
  const uint16_t *a_down[MOE_LORA_MAX_SLOTS];
  const uint16_t *b_down[MOE_LORA_MAX_SLOTS];
  /* 0: the routed layout above.  1: shared-outer LoRA (bf16 PR, section 2 "Shared-outer
   * LoRA"): the gate_up A and the down B are one weight set per slot that every expert
   * uses, a_gate_up[s]: [rank[s], H] and b_down[s]: [H, rank[s]]; b_gate_up and a_down
   * keep their per-expert layouts.  Other values -> MOE_LORA_ERR_INVALID_ARGUMENT. */
  int32_t shared_outer;
} moe_lora_adapters;

/* Optional knobs of moe_lora_forward (NULL = defaults). */
typedef struct {
  int32_t two_stream_max_tokens; /* side stream used only when T <= this (default 256) */
  int32_t force_path;            /* 0 auto, 1 fused epilogues, 2 decomposed (delta + activation kernels) */
  /* Optional hipEvent_t handles (NULL = none) recorded on `main` immediately before and
   * after the gate_up GEMM launch, so a caller can time that kernel alone. */
  void *gate_up_event_begin;
  void *gate_up_event_end;
  /* Which weights are the tile-packed copies written by moe_lora_pack_weights: bit 0
   * w_gate_up, bit 1 w_down (0 = both row-major).  Any packed weight needs
   * hidden % 128 == 0 and inter % 64 == 0 (else MOE_LORA_ERR_UNSUPPORTED); values
   * outside 0..3 -> MOE_LORA_ERR_INVALID_ARGUMENT. */
  int32_t packed_weights;
  /* moe_lora_forward_fp8 only: 1 = every block scale is a power of two (as in E8M0 /
   * MX-style scaling), which lets the staging use gfx950's fused scaled FP8 -> bf16
   * conversion (it applies only the scale's exponent); every weight is then exact in
   * bf16 and the result has the bits of moe_lora_forward on those dequantized weights.
   * 0 = arbitrary fp32 scales.  Other values ->
   * MOE_LORA_ERR_INVALID_ARGUMENT; a scale that is not a power of two with 1 set gives
   * wrong weights (the library does not read the scales on the host). */
  int32_t fp8_pow2_scales;
  int32_t reserved[2];
} moe_lora_options;

/* Human-readable name of a status code (static storage). */
const char *moe_lora_status_string(int status);

/* Library ABI version (incremented on any signature change). */
int moe_lora_version(void);

/* ---------------------------------------------------------------- route
 * Top-k routing and the expert-sorted pack fused (sglang PR "[LoRA] Experimental fast
 * LoRA path ...", Optimizations: top-k and the routed pack in a single launch).
 *   Renormalize: top-k of the bf16 logits (ties -> lower expert index), weights =
 *     softmax over the k selected logits.
 *   DeepSeek-V3: s = sigmoid(logit), key = s + correction_bias; groups are contiguous
 *     blocks of E/n_group experts scored by the sum of their two largest keys; the
 *     best topk_group groups (ties -> lower group index) are kept; the top-k keys in
 *     them are chosen (ties -> lower index); weights = rsf * s / sum(s).
 * Outputs:
 *   topk_ids [T, k] int32 (descending key), topk_weights [T, k] fp32,
 *   expert_offsets [E+1] int32 (exclusive prefix of per-expert counts),
 *   expanded_to_permuted [T*k] int32, permuted_to_expanded [T*k] int32.
 * Workspace: moe_lora_route_workspace_size(dims) bytes (may be 0 -> ws may be NULL).
 * Batches of up to 64 tokens take one launch; larger ones take two (per-block counts,
 * then final positions).
 * grouped must be non-NULL for MOE_LORA_ROUTING_DEEPSEEK_V3 and is ignored otherwise.
 * A batch runs on at most 256 workgroups of at most min(256, 32768 / E) tokens each, fewer
 * where the method's LDS footprint (DeepSeek-V3 keeps fp64 keys) would pass 160 KiB;
 * num_tokens above that limit returns MOE_LORA_ERR_UNSUPPORTED (route such batches in
 * chunks).  Limits: 65536 tokens for E = 128, 32768 for E = 256, 16384 for E = 512 with
 * Renormalize and 14848 with DeepSeek-V3 at k = 8. */
size_t moe_lora_route_workspace_size(const moe_lora_dims *dims);
int moe_lora_route(const moe_lora_dims *dims, int routing, const moe_lora_grouped *grouped,
                   const uint16_t *logits, int32_t *topk_ids, float *topk_weights,
                   int32_t *expert_offsets, int32_t *expanded_to_permuted,
                   int32_t *permuted_to_expanded, void *ws, size_t ws_bytes,
                   moe_lora_stream_t stream);

/* ---------------------------------------------------------------- permute
 * x_perm[p, :] = x[permuted_to_expanded[p] / top_k, :]  (bf16 gather; the bf16 PR's
 * "permute bf16 hidden" step).  x [T, H], x_perm [T*k, H]. */
int moe_lora_permute(const moe_lora_dims *dims, const uint16_t *x,
                     const int32_t *permuted_to_expanded, uint16_t *x_perm,
                     moe_lora_stream_t stream);

/* ---------------------------------------------------------------- forward
 * For every permuted row p (token t = permuted_to_expanded[p] / top_k, expert e,
 * slot a = token_slot[t]):
 *   g = W1[e] x_t + [a valid] s_a B1[a][e] (A1[a][e] x_t)        (2I)
 *   h = silu(g[0:I]) * g[I:2I]                                   (I)
 *   y_perm[p] = W2[e] h + [a valid] s_a B2[a][e] (A2[a][e] h)    (H), unweighted
 * (bf16 PR: Files-changed launcher row and section 2(A) steps 1-4; vLLM API page,
 * _TrtLlmLoRAExpertsBase.apply.)  fp32 accumulation; bf16 output.
 *   x       [T, H] token-order rows, or NULL when x_perm is given
 *   x_perm  [T*k, H] permuted rows, or NULL: then rows are gathered from x on load
 *   w_gate_up [E, 2I, H] (rows [0,I) gate, [I,2I) up), w_down [E, H, I]
 *   lora    NULL or num_slots == 0 -> the base MoE (same kernels, no LoRA work)
 *   y_perm  [T*k, H] output
 *   side    optional second stream.  With LoRA and T <= two_stream_max_tokens (default and
 *           maximum 256) the layer takes the decomposed path of the bf16 PR's two-stream
 *           flow: the gate_up LoRA shrink and expand (delta) run on `side` while `main`
 *           runs the base gate_up GEMM; `main` waits on the library's lora_ready event
 *           right before the activation kernel, the delta's only consumer.  On return all
 *           work is ordered before later work on `main`.  NULL = one stream: the fused
 *           path (LoRA expand appended to the GEMM's K loop, SwiGLU in its epilogue).
 *   opts    NULL = defaults.  force_path = 1 forces the fused path, 2 the decomposed path
 *           (on one stream when side is NULL; MOE_LORA_ERR_UNSUPPORTED when T > 256); other
 *           values -> MOE_LORA_ERR_INVALID_ARGUMENT.
 * Workspace: moe_lora_forward_workspace_size(dims, lora) bytes; it includes the
 * decomposed path's fp32 buffers when LoRA is present and T <= 256.
 * Concurrency: the fork/join events are per device and shared by all calls; calls that
 * use a side stream must not run concurrently on one device from several host threads. */
size_t moe_lora_forward_workspace_size(const moe_lora_dims *dims, const moe_lora_adapters *lora);
int moe_lora_forward(const moe_lora_dims *dims, const uint16_t *x, const uint16_t *x_perm,
                     const int32_t *expert_offsets, const int32_t *permuted_to_expanded,
                     const uint16_t *w_gate_up, const uint16_t *w_down,
                     const moe_lora_adapters *lora, uint16_t *y_perm, void *ws, size_t ws_bytes,
                     moe_lora_stream_t main, moe_lora_stream_t side,
                     const moe_lora_options *opts);

/* ---------------------------------------------------------------- forward, no allocation
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  moe_lora_forward on one
 * stream (the fused path) with its workspace taken from a scratch array the library holds
 * on each GPU it runs on: MOE_LORA_NOALLOC_SCRATCH_BYTES of device memory, reserved when
 * the library's code is loaded on that GPU and kept until the process ends.  The call
 * makes no allocation of any kind.
 *   Arguments as for moe_lora_forward (x or x_perm, routing outputs, weights, lora,
 *   y_perm: caller-owned device buffers).  opts: as for moe_lora_forward, except that
 *   force_path = 2 (the decomposed path) -> MOE_LORA_ERR_UNSUPPORTED; there is no side
 *   stream.
 *   Returns MOE_LORA_ERR_SCRATCH_TOO_SMALL, enqueuing nothing, when the problem's fused
 *   workspace (moe_lora_forward_workspace_size without the decomposed path's buffers)
 *   exceeds the scratch: the decode-sized batches fit (64 tokens of a hidden-2048,
 *   128-expert, top-8 layer with a rank-16 adapter need ~1.3 MiB; 256 tokens with four
 *   adapters up to rank 64 ~10 MiB); 8192-token prefill batches of that layer (150 MiB)
 *   and 1024 tokens of a hidden-7168, 256-expert layer (67 MiB) do not.
 * Concurrency: every call on one GPU uses the same scratch, which keeps the last call's
 * contents (nothing in it needs to start at zero).  Calls that overlap on one GPU, from
 * several host threads or on several streams without ordering between them, race on it
 * and give wrong results; order them on one stream. */
int moe_lora_forward_noalloc(const moe_lora_dims *dims, const uint16_t *x, const uint16_t *x_perm,
                             const int32_t *expert_offsets, const int32_t *permuted_to_expanded,
                             const uint16_t *w_gate_up, const uint16_t *w_down,
                             const moe_lora_adapters *lora, uint16_t *y_perm, moe_lora_stream_t main,
                             const moe_lora_options *opts);

/* ---------------------------------------------------------------- forward, FP8 weights
 * moe_lora_forward with FP8 expert weights (fast-path PR, title and Optimizations: the
 * LoRA deltas are applied around an FP8 fused MoE; the LoRA matrices stay bf16).
 *   w_gate_up [E, 2I, H], w_down [E, H, I]: OCP E4M3 codes, one byte per weight
 *     (sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7f / 0xff are NaN).
 *   w_gate_up_scale [E, 2I/128, H/128], w_down_scale [E, H/128, I/128]: fp32, one scale
 *     per 128 x 128 block; weight = value(code) * scale of its block.
 * Tiles of up to 64 rows (batches averaging up to 128 routed rows per expert) feed the
 * codes to the bf16 MFMAs unscaled (every E4M3 value is exact in bf16) and add each
 * 128-wide K block's fp32 sum times its scale; 128-row tiles round each weight times its
 * scale to bf16 once (round to nearest even) before the MFMA.  Everything else is as in
 * moe_lora_forward, whose workspace size applies.
 * All four weight pointers are device pointers, 16-byte aligned (else
 * MOE_LORA_ERR_INVALID_ARGUMENT).  Requires hidden and inter multiples of 128 and at most
 * 8192, and
 * runs the fused path only: opts->force_path == 2 -> MOE_LORA_ERR_UNSUPPORTED; a side
 * stream is not used.  opts->packed_weights bits say which weights are in the FP8
 * tile-packed layout of moe_lora_pack_weights_fp8 (the scales are never packed). */
int moe_lora_forward_fp8(const moe_lora_dims *dims, const uint16_t *x, const uint16_t *x_perm,
                         const int32_t *expert_offsets, const int32_t *permuted_to_expanded,
                         const uint8_t *w_gate_up, const float *w_gate_up_scale,
                         const uint8_t *w_down, const float *w_down_scale,
                         const moe_lora_adapters *lora, uint16_t *y_perm, void *ws, size_t ws_bytes,
                         moe_lora_stream_t main, moe_lora_stream_t side,
                         const moe_lora_options *opts);

/* ---------------------------------------------------------------- pack weights
 * Tile-packed copies of the expert weights for moe_lora_forward with
 * opts->packed_weights = 1.  The grouped GEMMs read each expert's weights one 64-wide K
 * step at a time for 128 output rows; the packed layout makes that piece one contiguous
 * 16 KB block instead of 128 row segments 4 KB or more apart.  Layout of a weight with N
 * rows and K columns per expert: blocks (e, s, t) in that order, s over the K / 64
 * column steps and t over the N / 128 row tiles, each block the 128 x 64 sub-matrix
 * row-major.  w_gate_up tiles are in the GEMM's gate/up pairing order: tile t holds the
 * 64 gate rows of intermediate columns [64 t, 64 t + 64), then the 64 up rows of the
 * same columns.  w_down tiles are rows [128 t, 128 t + 128) of [E, H, I].
 *   w_gate_up [E, 2I, H] -> w_gate_up_packed (same size); w_down [E, H, I] ->
 *   w_down_packed (same size).  Device pointers, 16-byte aligned, not overlapping; a
 *   pair given as two NULLs is skipped (at least one pair is needed).
 * Requires hidden % 128 == 0 and inter % 64 == 0 (else MOE_LORA_ERR_UNSUPPORTED).
 * A one-time transform, enqueued on `stream`; the library keeps no reference. */
int moe_lora_pack_weights(const moe_lora_dims *dims, const uint16_t *w_gate_up, const uint16_t *w_down,
                          uint16_t *w_gate_up_packed, uint16_t *w_down_packed,
                          moe_lora_stream_t stream);

/* ---------------------------------------------------------------- pack FP8 weights
 * Tile-packed copies of FP8 expert weights for moe_lora_forward_fp8 (the LDS staging
 * needs no change: only the codes' order in memory differs).  Same block order as
 * moe_lora_pack_weights, each block 128 rows x 64 codes (8 KB, row-major), so a 64-wide
 * K step of 128 output rows is one contiguous 8 KB read instead of 128 pieces of 64 bytes.
 *   w_gate_up [E, 2I, H] -> w_gate_up_packed, w_down [E, H, I] -> w_down_packed, uint8
 *   codes, device pointers, 16-byte aligned, not overlapping; a pair of two NULLs is
 *   skipped (at least one pair is needed).  Requires hidden % 128 == 0 and
 *   inter % 128 == 0 (else MOE_LORA_ERR_UNSUPPORTED).  Enqueued on `stream`. */
int moe_lora_pack_weights_fp8(const moe_lora_dims *dims, const uint8_t *w_gate_up, const uint8_t *w_down,
                              uint8_t *w_gate_up_packed, uint8_t *w_down_packed, moe_lora_stream_t stream);

/* ---------------------------------------------------------------- finalize
 * out[t, :] = bf16( sum_j topk_weights[t, j] * y_perm[expanded_to_permuted[t*k+j], :] ),
 * summed in fp32 in j order (vLLM API page, _finalize_with_w2_lora).  out [T, H]. */
int moe_lora_finalize(const moe_lora_dims *dims, const uint16_t *y_perm,
                      const float *topk_weights, const int32_t *expanded_to_permuted,
                      uint16_t *out, moe_lora_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
