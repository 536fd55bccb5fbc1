// Permute (bf16 row gather) and finalize (routing-weighted top-k reduction).
//
// Pages: sglang PR "[LoRA] bf16 MoE-LoRA for trtllm backend ...", Files-changed table
// (permute = bf16 gather of the hidden rows; finalize after the down GEMM); vLLM API
// page "trtllm_lora_moe", _finalize_with_w2_lora (per token, sum over top_k of the
// weighted permuted rows).
//
// Both kernels are HBM-bound row copies: one wavefront moves one 16-byte vector per
// lane per step, so every row is read and written with fully coalesced accesses.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRowThreads = 256;

// One wavefront per permuted row.
__global__ __launch_bounds__(kRowThreads) void permute_kernel(const uint16_t *__restrict__ x,
                                                              const int32_t *__restrict__ p2e,
                                                              uint16_t *__restrict__ x_perm, int R,
                                                              int H, int K) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int p = blockIdx.x * (kRowThreads / 64) + wave;
  if (p >= R) return;
  const int t = p2e[p] / K;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + (size_t)t * H);
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(x_perm + (size_t)p * H);
  const int nvec = H / 8;
  for (int v = lane; v < nvec; v += 64) dst[v] = src[v];
}

// One workgroup per token; each thread owns 8 consecutive hidden elements per step.
__global__ __launch_bounds__(kRowThreads) void finalize_kernel(const uint16_t *__restrict__ y,
                                                               const float *__restrict__ w,
                                                               const int32_t *__restrict__ e2p,
                                                               uint16_t *__restrict__ out, int H,
                                                               int K) {
  const int t = blockIdx.x;
  __shared__ int rows[MOE_LORA_MAX_TOPK];
  __shared__ float wts[MOE_LORA_MAX_TOPK];
  if (threadIdx.x < K) {
    rows[threadIdx.x] = e2p[(size_t)t * K + threadIdx.x];
    wts[threadIdx.x] = w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  const int nvec = H / 8;
  for (int v = threadIdx.x; v < nvec; v += kRowThreads) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < K; ++j) {
      const u32x4_t q = reinterpret_cast<const u32x4_t *>(y + (size_t)rows[j] * H)[v];
      const float wj = wts[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] += wj * bf16_to_f32(q[c] & 0xffffu);
        acc[2 * c + 1] += wj * bf16_to_f32(q[c] >> 16);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(acc[2 * c], acc[2 * c + 1]);
    reinterpret_cast<u32x4_t *>(out + (size_t)t * H)[v] = o;
  }
}

}  // namespace

int launch_permute(const uint16_t *x, const int32_t *p2e, uint16_t *x_perm, int R, int H, int K,
                   hipStream_t s) {
  if (R == 0) return ST_OK;
  const int rows_per_block = kRowThreads / 64;
  permute_kernel<<<(R + rows_per_block - 1) / rows_per_block, kRowThreads, 0, s>>>(x, p2e, x_perm,
                                                                                    R, H, K);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

int launch_finalize(const uint16_t *y_perm, const float *w, const int32_t *e2p, uint16_t *out,
                    int T, int H, int K, hipStream_t s) {
  if (T == 0) return ST_OK;
  finalize_kernel<<<T, kRowThreads, 0, s>>>(y_perm, w, e2p, out, H, K);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

}  // namespace moe
