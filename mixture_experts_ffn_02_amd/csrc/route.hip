// Routing + expert-sorted pack in one cooperative launch (gfx950).
//
// Pages: sglang PR "[LoRA] Experimental fast LoRA path ... FP8 and NVFP4 models",
// Optimizations (top-k and the routed pack fused in one launch); vLLM API page
// "trtllm_lora_moe" (routing methods Renormalize / DeepSeekV3 and their n_group,
// topk_group, routed_scaling_factor arguments; expanded index = token*top_k + k).
//
// Phase 1 (one wavefront per token): each lane holds a contiguous run of EPL experts.
//   Renormalize keys are 32-bit words (order-preserving bf16 bits << 16 | (0xffff - e)),
//   so one wave max picks the largest logit and, among equal logits, the lower index.
//   DeepSeek-V3 keys are fp64 (sigmoid + bias) compared lexicographically with the
//   expert index.  Each workgroup accumulates a per-expert histogram in LDS.
// grid.sync()
// Phase 2: every workgroup derives the global expert offsets and its own base inside
//   each expert from all histograms, then wave 0 scatters its expanded rows in order;
//   the stable rank among equal experts inside a 64-row chunk comes from ballots over
//   the bits of the expert id.
#include <hip/hip_cooperative_groups.h>

#include "common.h"
#include "kernels.h"

namespace cg = cooperative_groups;

namespace moe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxE = MOE_LORA_MAX_EXPERTS;

struct RouteParams {
  RouteArgs a;
  int tok_per_wg;
  int num_wg;
};

MOE_DEV uint32_t bf16_order_key(uint32_t b) {
  b &= 0xffffu;
  if (b == 0x8000u) b = 0u;  // -0 == +0
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

MOE_DEV bool better(double va, int ia, double vb, int ib) { return va > vb || (va == vb && ia < ib); }

MOE_DEV void wave_argmax(double &v, int &i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    double ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

MOE_DEV double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Renormalize: returns in lane j < K the j-th expert; fp64 softmax over the k logits.
template <int EPL>
MOE_DEV void topk_renormalize(const uint16_t *row, int E, int K, int lane, int &my_e, double &my_w) {
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane * EPL + i;
    key[i] = (e < E) ? ((bf16_order_key(row[e]) << 16) | (0xffffu - (uint32_t)e)) : 0u;
  }
  my_e = -1;
  for (int j = 0; j < K; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      uint32_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    int e = (int)(0xffffu - (best & 0xffffu));
    if (lane == e / EPL) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i == e % EPL) key[i] = 0u;
    }
    if (lane == j) my_e = e;
  }
  double l = (my_e >= 0) ? (double)bf16_to_f32(row[my_e]) : 0.0;
  double m = __shfl(l, 0);
  double ex = (my_e >= 0) ? exp(l - m) : 0.0;
  double sum = wave_sum(ex);
  my_w = ex / sum;
}

// DeepSeek-V3 grouped routing, keys in fp64.
template <int EPL>
MOE_DEV void topk_dsv3(const uint16_t *row, const float *bias, int E, int K, int n_group,
                       int topk_group, float rsf, int lane, double *keys_lds, int &my_e,
                       double &my_w) {
  double key[EPL];
  int idx[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane * EPL + i;
    if (e < E) {
      double l = (double)bf16_to_f32(row[e]);
      double s = 1.0 / (1.0 + exp(-l));
      key[i] = s + (bias ? (double)bias[e] : 0.0);
      idx[i] = e;
      keys_lds[e] = key[i];
    } else {
      key[i] = -INFINITY;
      idx[i] = 0x7fffffff;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int per = E / n_group;
  // group score: sum of the two largest keys of the group (one if the group has one)
  double gv = -INFINITY;
  int gi = 0x7fffffff;
  if (lane < n_group) {
    double b0 = -INFINITY, b1 = -INFINITY;
    for (int q = 0; q < per; ++q) {
      double v = keys_lds[lane * per + q];
      if (v > b0) {
        b1 = b0;
        b0 = v;
      } else if (v > b1) {
        b1 = v;
      }
    }
    gv = per >= 2 ? b0 + b1 : b0;
    gi = lane;
  }
  uint64_t chosen = 0;
  for (int r = 0; r < topk_group; ++r) {
    double v = gv;
    int i = gi;
    wave_argmax(v, i);
    chosen |= 1ull << i;
    if (lane == i) {
      gv = -INFINITY;
      gi = 0x7fffffff;
    }
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    if (idx[i] != 0x7fffffff && !((chosen >> (idx[i] / per)) & 1ull)) {
      key[i] = -INFINITY;
      idx[i] = 0x7fffffff;
    }
  }
  my_e = -1;
  for (int j = 0; j < K; ++j) {
    double v = key[0];
    int i0 = idx[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i)
      if (better(key[i], idx[i], v, i0)) {
        v = key[i];
        i0 = idx[i];
      }
    wave_argmax(v, i0);
    if (lane == i0 / EPL) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (idx[i] == i0) {
          key[i] = -INFINITY;
          idx[i] = 0x7fffffff;
        }
    }
    if (lane == j) my_e = i0;
  }
  double s = 0.0;
  if (my_e >= 0) s = 1.0 / (1.0 + exp(-(double)bf16_to_f32(row[my_e])));
  double sum = wave_sum(s);
  my_w = (double)rsf * s / sum;
}

template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteParams P) {
  const RouteArgs &a = P.a;
  __shared__ int32_t hist[kMaxE];
  __shared__ int32_t start[kMaxE];
  __shared__ double keys[kRouteWaves][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < a.E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();

  const int t0 = blockIdx.x * P.tok_per_wg;
  const int t1 = min(a.T, t0 + P.tok_per_wg);
  for (int t = t0 + wave; t < t1; t += kRouteWaves) {
    const uint16_t *row = a.logits + (size_t)t * a.E;
    int my_e;
    double my_w;
    if (a.method == MOE_LORA_ROUTING_DEEPSEEK_V3)
      topk_dsv3<EPL>(row, a.bias, a.E, a.K, a.n_group, a.topk_group, a.rsf, lane, keys[wave], my_e,
                     my_w);
    else
      topk_renormalize<EPL>(row, a.E, a.K, lane, my_e, my_w);
    if (lane < a.K) {
      a.ids[(size_t)t * a.K + lane] = my_e;
      a.weights[(size_t)t * a.K + lane] = (float)my_w;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += kRouteThreads) a.hist[(size_t)blockIdx.x * a.E + e] = hist[e];

  cg::this_grid().sync();

  // per-expert totals and this workgroup's base inside each expert
  for (int e = tid; e < a.E; e += kRouteThreads) {
    int before = 0, total = 0;
    for (int b = 0; b < P.num_wg; ++b) {
      int h = a.hist[(size_t)b * a.E + e];
      total += h;
      before += (b < (int)blockIdx.x) ? h : 0;
    }
    hist[e] = total;
    start[e] = before;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the totals, EPL' consecutive experts per lane
    const int per_lane = (a.E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per_lane; ++q) {
      int e = lane * per_lane + q;
      local += (e < a.E) ? hist[e] : 0;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int q = 0; q < per_lane; ++q) {
      int e = lane * per_lane + q;
      if (e < a.E) {
        int c = hist[e];
        if (blockIdx.x == 0) a.offsets[e] = run;
        start[e] += run;
        run += c;
      }
    }
    if (blockIdx.x == 0 && lane == 63) a.offsets[a.E] = incl;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // stable scatter of this workgroup's expanded rows
    const int j0 = t0 * a.K;
    const int j1 = t1 * a.K;
    int nbits = 0;
    while ((1 << nbits) < a.E) ++nbits;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = j0; base < j1; base += 64) {
      const int j = base + lane;
      const bool valid = j < j1;
      const int e = valid ? a.ids[j] : 0;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(valid && bit);
        peers &= bit ? m : ~m;
      }
      const int rank = __popcll(peers & lt);
      int s = 0;
      if (valid) s = start[e];
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int pos = s + rank;
        a.e2p[j] = pos;
        a.p2e[pos] = j;
        if ((peers & lt) == 0ull) start[e] = s + __popcll(peers);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

__global__ void zero_offsets_kernel(int32_t *offsets, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) offsets[i] = 0;
}

struct CoopLimit {
  int dev = -1;
  int max_wg[4] = {0, 0, 0, 0};
};

template <int EPL>
int max_coresident(int slot) {
  static CoopLimit cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  CoopLimit &c = cache[dev & 15];
  if (c.dev != dev || c.max_wg[slot] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, route_kernel<EPL>, kRouteThreads, 0) !=
        hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    c.dev = dev;
    c.max_wg[slot] = per_cu * cus;
  }
  return c.max_wg[slot];
}

template <int EPL>
int launch_epl(const RouteArgs &a, hipStream_t s, int slot) {
  RouteParams P;
  P.a = a;
  int nwg = route_num_wg(a.T);
  int lim = max_coresident<EPL>(slot);
  if (lim <= 0) return ST_HIP;
  if (nwg > lim) nwg = lim;
  P.num_wg = nwg;
  P.tok_per_wg = (a.T + nwg - 1) / nwg;
  void *args[] = {&P};
  hipError_t err = hipLaunchCooperativeKernel((const void *)route_kernel<EPL>, dim3(nwg),
                                              dim3(kRouteThreads), args, 0, s);
  return err == hipSuccess ? ST_OK : ST_HIP;
}

}  // namespace

int route_num_wg(int T) {
  int n = (T + 63) / 64;
  if (n < 1) n = 1;
  if (n > 128) n = 128;
  return n;
}

int launch_zero_offsets(int32_t *offsets, int E, hipStream_t s) {
  zero_offsets_kernel<<<1, 256, 0, s>>>(offsets, E + 1);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

int launch_route(const RouteArgs &a, hipStream_t s) {
  const int need = (a.E + 63) / 64;
  if (need <= 1) return launch_epl<1>(a, s, 0);
  if (need <= 2) return launch_epl<2>(a, s, 1);
  if (need <= 4) return launch_epl<4>(a, s, 2);
  return launch_epl<8>(a, s, 3);
}

}  // namespace moe
