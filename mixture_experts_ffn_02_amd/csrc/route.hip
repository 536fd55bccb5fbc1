// Routing + expert-sorted pack in one launch (gfx950).
//
// Pages: sglang PR "[LoRA] Experimental fast LoRA path ... FP8 and NVFP4 models",
// Optimizations (top-k and the routed pack fused in one launch); vLLM API page
// "trtllm_lora_moe" (routing methods Renormalize / DeepSeekV3 and their n_group,
// topk_group, routed_scaling_factor arguments; expanded index = token*top_k + k).
//
// Phase 1 (one wavefront per token, tokens of a wave contiguous): each lane holds a
//   contiguous run of EPL experts.  Renormalize keys are 32-bit words
//   (order-preserving bf16 bits << 16 | (0xffff - e)), so one DPP wave max picks the
//   largest logit and, among equal logits, the lower index.  DeepSeek-V3 keys are fp64
//   (sigmoid + bias); their wave argmax compares the high 32 bits of the
//   order-preserving 64-bit pattern with a DPP max, and only on a tie of those bits
//   falls back to the low bits and then to the lower index, so the selection is exact.
//   Each wave counts its experts in an LDS histogram row of its own.
// Batches of up to 64 tokens run in one workgroup and one launch (at 256 tokens the two
//   launches below measured ~8 us faster than one workgroup).  Larger batches run on
//   several workgroups: each writes its per-expert counts and the positions of its rows
//   relative to its own block; a second, equally wide launch derives the expert offsets
//   and each block's base and makes the positions final.  (A grid-wide barrier in one
//   cooperative launch measured ~20 us slower per call than the second launch.)
// Phase 2: every wave scatters its own contiguous run of expanded rows; the stable
//   rank among equal experts inside a 64-row chunk comes from ballots over the bits of
//   the expert id, the base from the per-wave, per-workgroup prefix counts.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kSingleMaxT = 64;     // one workgroup handles the whole batch up to this
constexpr int kMaxTokPerWg = 256;   // LDS bound of the per-workgroup id buffer
constexpr int kMaxRouteWg = 256;    // workgroups of one routing launch

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

MOE_DEV float order_key_to_f32(uint32_t o) {
  const uint32_t b = (o & 0x8000u) ? (o & 0x7fffu) : (~o & 0xffffu);
  return bf16_to_f32(b);
}

MOE_DEV uint64_t f64_order_key(double v) {
  if (v == 0.0) v = 0.0;  // -0 == +0
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

MOE_DEV bool better(double va, int ia, double vb, int ib) { return va > vb || (va == vb && ia < ib); }

MOE_DEV uint32_t wave_max_u32(uint32_t v) { return __reduce_max_sync(~0ull, v); }
MOE_DEV int wave_min_i32(int v) { return __reduce_min_sync(~0ull, v); }

// Exact wave argmax of (key desc, index asc) over lanes with valid == true; returns the
// winning index (wave-uniform).  At least one lane must be valid.
MOE_DEV int wave_argmax_f64(double key, int idx, bool valid) {
  const uint64_t u = valid ? f64_order_key(key) : 0ull;
  const uint32_t hi = (uint32_t)(u >> 32);
  const uint32_t mh = wave_max_u32(hi);
  uint64_t mask = __ballot(valid && hi == mh);
  if (__popcll(mask) > 1) {
    const bool in = valid && hi == mh;
    const uint32_t lo = in ? (uint32_t)u : 0u;
    const uint32_t ml = wave_max_u32(lo);
    const bool in2 = in && lo == ml;
    mask = __ballot(in2);
    if (__popcll(mask) > 1) return wave_min_i32(in2 ? idx : 0x7fffffff);
  }
  const int lane = __ffsll((unsigned long long)mask) - 1;
  return __builtin_amdgcn_readlane(idx, lane);
}

// Renormalize: lane j < K ends with the j-th expert and its weight (softmax over the k
// selected logits, fp32).
template <int EPL>
MOE_DEV void topk_renormalize(const uint16_t (&v)[EPL], int E, int K, int lane, int &my_e,
                              float &my_w) {
  uint32_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    key[i] = (e < E) ? ((bf16_order_key(v[i]) << 16) | (0xffffu - (uint32_t)e)) : 0u;
  }
  my_e = -1;
  uint32_t my_key = 0u;
  for (int j = 0; j < K; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t m = wave_max_u32(best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (key[i] == m) key[i] = 0u;
    if (lane == j) my_key = m;
  }
  // softmax over the k selected logits (lane j holds the j-th, the largest in lane 0)
  const float my_l = order_key_to_f32(my_key >> 16);
  const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_l), 0));
  const float ex = (lane < K) ? expf(my_l - l0) : 0.f;
  float sum = 0.f;
  for (int j = 0; j < K; ++j) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < K) my_e = (int)(0xffffu - (my_key & 0xffffu));
  my_w = (lane < K) ? ex / sum : 0.f;
}

// DeepSeek-V3 grouped routing, keys in fp64 (selection); weights in fp32.
template <int EPL>
MOE_DEV void topk_dsv3(const uint16_t (&v)[EPL], const float *bias, int E, int K, int n_group,
                       int topk_group, float rsf, int lane, double *keys_lds, int &my_e,
                       float &my_w) {
  double key[EPL];
  int idx[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    if (e < E) {
      const double l = (double)bf16_to_f32(v[i]);
      key[i] = 1.0 / (1.0 + exp(-l)) + (bias ? (double)bias[e] : 0.0);
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
  // group score: sum of the two largest keys of the group (the key itself for one expert)
  double gv = -INFINITY;
  if (lane < n_group) {
    double b0 = -INFINITY, b1 = -INFINITY;
    for (int q = 0; q < per; ++q) {
      const double x = keys_lds[lane * per + q];
      if (x > b0) {
        b1 = b0;
        b0 = x;
      } else if (x > b1) {
        b1 = x;
      }
    }
    gv = per >= 2 ? b0 + b1 : b0;
  }
  __builtin_amdgcn_wave_barrier();
  uint64_t chosen = 0;
  for (int r = 0; r < topk_group; ++r) {
    const bool valid = lane < n_group && !((chosen >> lane) & 1ull);
    const int g = wave_argmax_f64(gv, lane, valid);
    chosen |= 1ull << g;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    if (idx[i] != 0x7fffffff && !((chosen >> (idx[i] / per)) & 1ull)) idx[i] = 0x7fffffff;
  }
  my_e = -1;
  float sum = 0.f, my_s = 0.f;
  for (int j = 0; j < K; ++j) {
    double bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (idx[i] != 0x7fffffff && (bi == 0x7fffffff || better(key[i], idx[i], bv, bi))) {
        bv = key[i];
        bi = idx[i];
      }
    const int e = wave_argmax_f64(bv, bi, bi != 0x7fffffff);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (idx[i] == e) idx[i] = 0x7fffffff;
    int vb = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i == e % EPL) vb = (int)v[i];
    const float s = 1.0f / (1.0f + expf(-bf16_to_f32((uint32_t)__builtin_amdgcn_readlane(vb, e / EPL))));
    sum += s;
    if (lane == j) {
      my_e = e;
      my_s = s;
    }
  }
  my_w = (my_e >= 0) ? rsf * my_s / sum : 0.f;
}

// All-reduce over the 16 lanes of a DPP row (quad swaps, then rotations by 4 and 8).
MOE_DEV uint32_t row_max_u32(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // xor 1
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // xor 2
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);  // row_ror 4
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror 8
  return o > v ? o : v;
}

MOE_DEV float row_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  return v;
}

// Renormalize for four tokens at once: each 16-lane row of the wavefront owns one token
// (EPR experts per lane); used when k <= 16.  Row-local DPP reductions need no cross-row
// traffic, so one instruction stream selects for four tokens.
template <int EPR>
MOE_DEV void topk_renormalize_rows(const uint16_t *row_logits, bool valid, int E, int K, int lr,
                                   int &my_e, float &my_w) {
  uint32_t key[EPR];
#pragma unroll
  for (int i = 0; i < EPR; ++i) {
    const int e = lr * EPR + i;
    key[i] = (valid && e < E) ? ((bf16_order_key(row_logits[e]) << 16) | (0xffffu - (uint32_t)e)) : 0u;
  }
  uint32_t my_key = 0u, m0 = 0u;
  for (int j = 0; j < K; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPR; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t m = row_max_u32(best);
#pragma unroll
    for (int i = 0; i < EPR; ++i)
      if (key[i] == m) key[i] = 0u;
    if (j == 0) m0 = m;
    if (lr == j) my_key = m;
  }
  const bool mine = valid && lr < K;
  const float l0 = order_key_to_f32(m0 >> 16);
  const float ex = mine ? expf(order_key_to_f32(my_key >> 16) - l0) : 0.f;
  const float sum = row_sum_f32(ex);
  my_e = mine ? (int)(0xffffu - (my_key & 0xffffu)) : -1;
  my_w = mine ? ex / sum : 0.f;
}

template <int EPL>
MOE_DEV void load_row(const uint16_t *row, int E, int lane, uint16_t (&v)[EPL]) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    v[i] = (e < E) ? row[e] : (uint16_t)0;
  }
}

// Dynamic LDS: hist_w [waves][E] int | ids [tok_per_wg*K] int | tot [E] | wgbase [E]
//              | keys [waves][E] double (DeepSeek-V3 only)
template <int EPL, bool MULTI>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteParams P) {
  const RouteArgs &a = P.a;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int E = a.E, K = a.K;
  int32_t *hist_w = reinterpret_cast<int32_t *>(smem);
  int32_t *ids_l = hist_w + kRouteWaves * E;
  int32_t *tot = ids_l + P.tok_per_wg * K;
  int32_t *wgbase = tot + E;
  double *keys = reinterpret_cast<double *>(
      smem + (((size_t)(kRouteWaves * E + P.tok_per_wg * K + 2 * E) * 4 + 15) & ~(size_t)15));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist_w[i] = 0;

  const int t_begin = blockIdx.x * P.tok_per_wg;
  const int t_end = min(a.T, t_begin + P.tok_per_wg);
  // this workgroup's logits block [t_begin, t_end) x E, copied with 16-byte loads
  uint16_t *lg = reinterpret_cast<uint16_t *>(
      smem + (((size_t)(kRouteWaves * E + P.tok_per_wg * K + 2 * E) * 4 + 15) & ~(size_t)15) +
      (a.method == MOE_LORA_ROUTING_DEEPSEEK_V3 ? (size_t)kRouteWaves * E * sizeof(double) : 0));
  {
    const size_t n = (size_t)(t_end - t_begin) * E;  // elements
    const uint16_t *src = a.logits + (size_t)t_begin * E;
    const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0);
    if (vec) {
      for (size_t v = tid; v < n / 8; v += kRouteThreads)
        reinterpret_cast<u32x4_t *>(lg)[v] = reinterpret_cast<const u32x4_t *>(src)[v];
      for (size_t i = (n / 8) * 8 + tid; i < n; i += kRouteThreads) lg[i] = src[i];
    } else {
      for (size_t i = tid; i < n; i += kRouteThreads) lg[i] = src[i];
    }
  }
  __syncthreads();
  const int tpw = (P.tok_per_wg + kRouteWaves - 1) / kRouteWaves;
  const int w_begin = min(t_end, t_begin + wave * tpw);
  const int w_end = min(t_end, w_begin + tpw);
  const bool dsv3 = a.method == MOE_LORA_ROUTING_DEEPSEEK_V3;

  // ---- phase 1: top-k per token
  if (!dsv3 && K <= 16) {
    const int rrow = lane >> 4, lr = lane & 15;
    for (int t0 = w_begin; t0 < w_end; t0 += 4) {
      const int t = t0 + rrow;
      const bool tv = t < w_end;
      int my_e;
      float my_w;
      topk_renormalize_rows<4 * EPL>(lg + (size_t)(tv ? t - t_begin : 0) * E, tv, E, K, lr, my_e, my_w);
      if (my_e >= 0) {
        a.ids[(size_t)t * K + lr] = my_e;
        a.weights[(size_t)t * K + lr] = my_w;
        ids_l[(t - t_begin) * K + lr] = my_e;
        atomicAdd(&hist_w[wave * E + my_e], 1);
      }
    }
  }
  uint16_t cur[EPL];
  for (int t = (!dsv3 && K <= 16) ? w_end : w_begin; t < w_end; ++t) {
    load_row<EPL>(lg + (size_t)(t - t_begin) * E, E, lane, cur);
    int my_e;
    float my_w;
    if (dsv3)
      topk_dsv3<EPL>(cur, a.bias, E, K, a.n_group, a.topk_group, a.rsf, lane, keys + wave * E, my_e,
                     my_w);
    else
      topk_renormalize<EPL>(cur, E, K, lane, my_e, my_w);
    if (lane < K) {
      a.ids[(size_t)t * K + lane] = my_e;
      a.weights[(size_t)t * K + lane] = my_w;
      ids_l[(t - t_begin) * K + lane] = my_e;
      hist_w[wave * E + my_e] += 1;  // the k experts of one token are distinct
    }
  }
  __syncthreads();

  // ---- per-wave starting positions inside this workgroup, workgroup totals
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = hist_w[w * E + e];
      hist_w[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
    if (MULTI) a.hist[(size_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  if (!MULTI && wave == 0) {
    // one workgroup: offsets are the exclusive scan of its totals
    const int per_lane = (E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per_lane; ++q) {
      const int e = lane * per_lane + q;
      local += (e < E) ? tot[e] : 0;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int q = 0; q < per_lane; ++q) {
      const int e = lane * per_lane + q;
      if (e < E) {
        a.offsets[e] = run;
        wgbase[e] = run;
        run += tot[e];
      }
    }
    if (lane == 63) a.offsets[E] = incl;
  }
  if (MULTI)
    for (int e = tid; e < E; e += kRouteThreads) wgbase[e] = 0;
  __syncthreads();

  // ---- stable scatter of this wave's expanded rows.  One workgroup writes final
  // positions; with several, each writes its positions relative to its own block
  // (into e2p) and the last workgroup to finish adds the global bases.
  int32_t *start = hist_w + wave * E;
  const int j0 = w_begin * K, j1 = w_end * K;
  const int jl0 = t_begin * K;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = j0; base < j1; base += 64) {
    const int j = base + lane;
    const bool valid = j < j1;
    const int e = valid ? ids_l[j - jl0] : 0;
    uint64_t peers = __ballot(valid);
    for (int bb = 0; bb < nbits; ++bb) {
      const bool bit = (e >> bb) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    int sp = 0;
    if (valid) sp = start[e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int pos = wgbase[e] + sp + rank;
      a.e2p[j] = pos;
      if (!MULTI) a.p2e[pos] = j;
      if ((peers & lt) == 0ull) start[e] = sp + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Second launch for multi-workgroup batches: every workgroup reads all per-workgroup
// expert counts, derives the expert offsets and its own block's base, and turns the
// block-relative positions of its rows (left in e2p) into final ones.
__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(RouteParams P) {
  const RouteArgs &a = P.a;
  const int E = a.E, K = a.K;
  __shared__ int32_t tot[MOE_LORA_MAX_EXPERTS];
  __shared__ int32_t base[MOE_LORA_MAX_EXPERTS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) {
    tot[e] = 0;
    base[e] = 0;
  }
  __syncthreads();
  // (expert, 16-workgroup chunk) pairs over all threads
  const int chunks = (P.num_wg + 15) / 16;
  for (int q = tid; q < E * chunks; q += kRouteThreads) {
    const int e = q % E, b0 = (q / E) * 16;
    int h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) h[i] = (b0 + i < P.num_wg) ? a.hist[(size_t)(b0 + i) * E + e] : 0;
    int total = 0, before = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      total += h[i];
      before += (b0 + i < (int)blockIdx.x) ? h[i] : 0;
    }
    atomicAdd(&tot[e], total);
    atomicAdd(&base[e], before);
  }
  __syncthreads();
  if (wave == 0) {
    const int per_lane = (E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per_lane; ++q) {
      const int e = lane * per_lane + q;
      local += (e < E) ? tot[e] : 0;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int q = 0; q < per_lane; ++q) {
      const int e = lane * per_lane + q;
      if (e < E) {
        if (blockIdx.x == 0) a.offsets[e] = run;
        base[e] += run;
        run += tot[e];
      }
    }
    if (blockIdx.x == 0 && lane == 63) a.offsets[E] = incl;
  }
  __syncthreads();
  const int j0 = blockIdx.x * P.tok_per_wg * K;
  const int j1 = min(a.T, (blockIdx.x + 1) * P.tok_per_wg) * K;
  for (int j = j0 + tid; j < j1; j += kRouteThreads) {
    const int pos = base[a.ids[j]] + a.e2p[j];
    a.e2p[j] = pos;
    a.p2e[pos] = j;
  }
}

__global__ void zero_offsets_kernel(int32_t *offsets, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) offsets[i] = 0;
}

size_t route_lds_bytes(int E, int K, int tok_per_wg, bool dsv3) {
  size_t b = ((size_t)(kRouteWaves * E + tok_per_wg * K + 2 * E) * 4 + 15) & ~(size_t)15;
  if (dsv3) b += (size_t)kRouteWaves * E * sizeof(double);
  b += (size_t)tok_per_wg * E * sizeof(uint16_t);  // logits block
  return b;
}

template <int EPL, bool MULTI>
bool allow_lds(size_t lds) {
  static size_t granted = 64 * 1024;
  if (lds <= granted) return true;
  if (hipFuncSetAttribute((const void *)route_kernel<EPL, MULTI>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  granted = lds;
  return true;
}

constexpr size_t kRouteLdsMax = 160 * 1024;  // LDS of one gfx950 workgroup

// tokens per workgroup: bounded by the LDS copy of the logits block (64 KiB), the id
// buffer, and the whole LDS footprint of the method (the fp64 DeepSeek-V3 key rows take
// 16 * E * 8 bytes: at E = 512 and k = 8 only 58 tokens fit beside them)
int max_tok_per_wg(int E, int K, bool dsv3) {
  int m = 32768 / E;
  if (m > kMaxTokPerWg) m = kMaxTokPerWg;
  const size_t fixed = route_lds_bytes(E, K, 0, dsv3) + 16;  // + 16: the alignment pad
  const size_t per_tok = (size_t)K * 4 + (size_t)E * sizeof(uint16_t);
  const int fit = fixed < kRouteLdsMax ? (int)((kRouteLdsMax - fixed) / per_tok) : 0;
  return m < fit ? m : fit;
}

int plan_route(int T, int E, int K, bool dsv3, int &tok_per_wg) {
  const int mx = max_tok_per_wg(E, K, dsv3);
  if (mx < 1) return 0;
  if (T <= kSingleMaxT && T <= mx) {
    tok_per_wg = T;
    return 1;
  }
  int tpw = dsv3 ? 16 : 64;
  if (tpw > mx) tpw = mx;
  int n = (T + tpw - 1) / tpw;
  if (n > kMaxRouteWg) {
    n = kMaxRouteWg;
    if ((T + n - 1) / n > mx) return 0;
  }
  tok_per_wg = (T + n - 1) / n;
  return n;
}

template <int EPL>
int launch_epl(const RouteArgs &a, hipStream_t s) {
  RouteParams P;
  P.a = a;
  const bool dsv3 = a.method == MOE_LORA_ROUTING_DEEPSEEK_V3;
  const int nwg = plan_route(a.T, a.E, a.K, dsv3, P.tok_per_wg);
  if (nwg <= 0) return ST_UNSUPPORTED;
  P.num_wg = nwg;
  const size_t lds = route_lds_bytes(a.E, a.K, P.tok_per_wg, dsv3);
  if (nwg == 1) {
    if (!allow_lds<EPL, false>(lds)) return ST_HIP;
    route_kernel<EPL, false><<<1, kRouteThreads, lds, s>>>(P);
    return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
  }
  if (!allow_lds<EPL, true>(lds)) return ST_HIP;
  route_kernel<EPL, true><<<nwg, kRouteThreads, lds, s>>>(P);
  if (hipGetLastError() != hipSuccess) return ST_HIP;
  route_finish_kernel<<<nwg, kRouteThreads, 0, s>>>(P);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

}  // namespace

size_t route_workspace_bytes(int T, int E, int K) {
  // enough for either routing method
  int tpw = 0, n = 0;
  for (int m = 0; m < 2; ++m) {
    const int nm = plan_route(T, E, K, m == 1, tpw);
    n = nm > n ? nm : n;
  }
  return n > 1 ? (size_t)n * E * sizeof(int32_t) : 0;
}

int route_max_tokens(int E, int K, bool dsv3) { return kMaxRouteWg * max_tok_per_wg(E, K, dsv3); }

int launch_zero_offsets(int32_t *offsets, int E, hipStream_t s) {
  zero_offsets_kernel<<<1, 256, 0, s>>>(offsets, E + 1);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

int launch_route(const RouteArgs &a, hipStream_t s) {
  const int need = (a.E + 63) / 64;
  if (need <= 1) return launch_epl<1>(a, s);
  if (need <= 2) return launch_epl<2>(a, s);
  if (need <= 4) return launch_epl<4>(a, s);
  return launch_epl<8>(a, s);
}

}  // namespace moe
