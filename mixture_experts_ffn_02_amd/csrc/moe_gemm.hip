// Grouped bf16 MFMA GEMMs of the MoE-LoRA expert FFN (gfx950).
//
// Pages: sglang PR "[LoRA] bf16 MoE-LoRA for trtllm backend ...", Files-changed table
// (gate_up GEMM with K = hidden, N = 2*inter; activation adding gate_up_lora_delta
// before SwiGLU and capturing the activation for the down LoRA; down GEMM with
// K = inter, N = hidden) and section 2(A) steps 1-5; sglang PR "[LoRA] Experimental fast
// LoRA path ...", Optimizations (LoRA deltas applied inside the fused MoE; split-K LoRA
// shrink with the fp32 -> bf16 cast fused into the LoRA-B expand).
//
// One kernel template serves every contraction of the layer:
//   MODE_SHRINK   u_part[split][p][0:r] = A_lora[slot(p)][e] . a_row(p)   (split-K, fp32 partials)
//   MODE_GATEUP   act[p] = silu(g) * u,  [g | u] = W1[e] . x_p  (+ s * B1 . bf16(sum u_part))
//   MODE_DOWN     y[p]   = W2[e] . act_p (+ s * B2 . bf16(sum v_part))
//   MODE_GATEUP_F32 / MODE_EXPAND_F32: the same contraction with a plain fp32 store,
//     used by the decomposed two-stream pipeline (base gate_up result and LoRA delta
//     produced separately, then joined by the activation kernel).
// The LoRA expand is not a separate pass: it is appended to the GEMM's K loop as one
// extra 64-wide K step per adapter slot present in the tile, whose A operand is the
// split-K partial sum scaled by s_a and rounded to bf16 on the way into LDS, and whose
// B operand is the slot's B matrix (rows masked to the tile rows of that slot).
//
// Tiling: BM token rows x BN weight rows per workgroup, BK = 64, both operands staged
// through double-buffered LDS (row pitch 72 elements so that the 16-byte fragment reads
// of 16 consecutive rows fall in distinct banks), v_mfma_f32_16x16x32_bf16 on 64-wide
// wavefronts.  Work tiles are (expert, m-tile, n-tile) triples found on the device from
// expert_offsets; block ids are remapped so each XCD runs a contiguous range of them,
// keeping an expert's weight and activation tiles in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_SHRINK = 2, MODE_GATEUP_F32 = 3, MODE_EXPAND_F32 = 4 };

constexpr int BK = 64;
constexpr int LDSP = BK + 8;

struct GemmParams {
  const uint16_t *a;  // A rows: x [T, K] when a_gather, else [R, K] in permuted order
  const int32_t *p2e;
  int a_gather;
  const uint16_t *w;  // [E, N, K] (unused by SHRINK / EXPAND)
  int N, K, I;
  const int32_t *offsets;
  int E, top_k, R;
  int n_cols;  // n-tiles (GEMM modes) or K splits (SHRINK)
  int k_steps_per_split;
  int num_slots;
  const int32_t *token_slot;
  int rank[MOE_LORA_MAX_SLOTS];
  float scaling[MOE_LORA_MAX_SLOTS];
  const uint16_t *lora_w[MOE_LORA_MAX_SLOTS];  // SHRINK: A [E, r, K]; ext: B [E, N, r]
  const float *part;                            // ext A source [splits][R][rmax]
  int part_splits;
  int rmax;
  uint16_t *out_bf16;
  float *out_f32;
};

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM *WN * 64) void moe_gemm_kernel(const GemmParams P) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_CH = BM * (BK / 8), B_CH = BN * (BK / 8);
  constexpr int A_IT = (A_CH + NT - 1) / NT, B_IT = (B_CH + NT - 1) / NT;
  constexpr bool kGateUp = (MODE == MODE_GATEUP);
  constexpr bool kHasMain = (MODE != MODE_EXPAND_F32);
  constexpr bool kHasExt = (MODE == MODE_GATEUP || MODE == MODE_DOWN || MODE == MODE_EXPAND_F32);
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(!kGateUp || (FN % 2 == 0), "gate/up pairing needs an even fragment count");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDSP];
  __shared__ int s_src[BM];
  __shared__ int s_slot[BM];
  __shared__ int s_info[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- which (expert, m-tile, column) this block owns
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int L = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int mt = L / P.n_cols, col = L % P.n_cols;
  if (wave == 0) {
    if (lane == 0) {
      s_info[0] = -1;
      s_info[3] = 0;
    }
    const int per = (P.E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < P.E) local += (P.offsets[e + 1] - P.offsets[e] + BM - 1) / BM;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < P.E) {
        const int lo = P.offsets[e], cnt = P.offsets[e + 1] - lo;
        const int tiles = (cnt + BM - 1) / BM;
        if (mt >= run && mt < run + tiles) {
          const int m0 = (mt - run) * BM;
          s_info[0] = e;
          s_info[1] = lo + m0;
          s_info[2] = min(BM, cnt - m0);
        }
        run += tiles;
      }
    }
  }
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;
  const int row0 = s_info[1], rows = s_info[2];

  const bool need_tok = P.a_gather || P.num_slots > 0;
  for (int r = tid; r < BM; r += NT) {
    int src = -1, slot = -1;
    if (r < rows) {
      const int p = row0 + r;
      const int tok = need_tok ? P.p2e[p] / P.top_k : 0;
      src = P.a_gather ? tok : p;
      if (P.num_slots > 0) {
        const int s = P.token_slot[tok];
        slot = (s >= 0 && s < P.num_slots) ? s : -1;
      }
    }
    s_src[r] = src;
    s_slot[r] = slot;
    if (slot >= 0) atomicOr(&s_info[3], 1 << slot);
  }
  __syncthreads();
  const int slot_mask = s_info[3];

  // ---- per-thread chunk geometry (fixed for the whole K loop)
  const uint16_t *a_ptr[A_IT];
  int a_lds[A_IT], a_row[A_IT], a_c8[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int c = tid + i * NT;
    a_row[i] = -1;
    a_ptr[i] = nullptr;
    a_lds[i] = 0;
    a_c8[i] = c & 7;
    if (c < A_CH) {
      const int r = c >> 3;
      a_row[i] = r;
      a_lds[i] = r * LDSP + (c & 7) * 8;
      const int src = s_src[r];
      if (src >= 0 && kHasMain && MODE != MODE_EXPAND_F32)
        a_ptr[i] = P.a + (size_t)src * P.K + (c & 7) * 8;
    }
  }
  int b_wrow[B_IT], b_lds[B_IT], b_c8[B_IT];
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int c = tid + i * NT;
    b_wrow[i] = -1;
    b_lds[i] = 0;
    b_c8[i] = c & 7;
    if (c < B_CH) {
      const int n = c >> 3;
      b_lds[i] = n * LDSP + (c & 7) * 8;
      if (MODE == MODE_SHRINK) {
        b_wrow[i] = n;  // rank row, checked against the slot's rank
      } else if (kGateUp) {
        const int wnn = n / WTN, cc = n % WTN;
        const int half = cc / (WTN / 2), j = cc % (WTN / 2);
        const int icol = col * (BN / 2) + wnn * (WTN / 2) + j;
        b_wrow[i] = (icol < P.I) ? half * P.I + icol : -1;
      } else {
        const int ng = col * BN + n;
        b_wrow[i] = (ng < P.N) ? ng : -1;
      }
    }
  }

  u32x4_t ra[A_IT], rb[B_IT];
  f32x4_t acc[FM][FN];

  auto zero_acc = [&]() {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // main K step: A rows and B (= W or the slot's LoRA A) rows from global memory
  auto load_main = [&](int k0, const uint16_t *bbase, int bcount) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      ra[i] = zero_u32x4();
      if (a_ptr[i] && k0 + a_c8[i] * 8 < P.K) ra[i] = *reinterpret_cast<const u32x4_t *>(a_ptr[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      rb[i] = zero_u32x4();
      const int wr = b_wrow[i];
      if (wr >= 0 && wr < bcount && k0 + b_c8[i] * 8 < P.K)
        rb[i] = *reinterpret_cast<const u32x4_t *>(bbase + (size_t)wr * P.K + k0 + b_c8[i] * 8);
    }
  };

  // LoRA expand step for slot a: A = bf16(s_a * sum of partials) on rows of that slot,
  // B = B_lora[a][e] rows (rank columns), zero beyond the rank.
  auto load_ext = [&](int a) {
    const int ra_rank = P.rank[a];
    const float sc = P.scaling[a];
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      ra[i] = zero_u32x4();
      const int r = a_row[i];
      const int j0 = a_c8[i] * 8;
      if (r >= 0 && j0 < ra_rank && s_slot[r] == a) {
        const int p = row0 + r;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < P.part_splits; ++s) {
          const f32x4_t *src =
              reinterpret_cast<const f32x4_t *>(P.part + ((size_t)s * P.R + p) * P.rmax + j0);
          const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] += x0[q];
            v[4 + q] += x1[q];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = (j0 + 2 * q < ra_rank) ? v[2 * q] * sc : 0.f;
          const float hi = (j0 + 2 * q + 1 < ra_rank) ? v[2 * q + 1] * sc : 0.f;
          ra[i][q] = pack_bf16x2(lo, hi);
        }
      }
    }
    const uint16_t *bl = P.lora_w[a];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      rb[i] = zero_u32x4();
      const int wr = b_wrow[i];
      const int j0 = b_c8[i] * 8;
      if (wr >= 0 && j0 < ra_rank) {
        const uint16_t *src = bl + ((size_t)e * P.N + wr) * ra_rank + j0;
        if ((ra_rank & 7) == 0) {
          rb[i] = *reinterpret_cast<const u32x4_t *>(src);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (j0 + 2 * q < ra_rank) ? src[2 * q] : 0u;
            const uint32_t hi = (j0 + 2 * q + 1 < ra_rank) ? src[2 * q + 1] : 0u;
            rb[i][q] = lo | (hi << 16);
          }
        }
      }
    }
  };

  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i)
      if (a_row[i] >= 0) *reinterpret_cast<u32x4_t *>(&As[buf][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_IT; ++i)
      if (tid + i * NT < B_CH) *reinterpret_cast<u32x4_t *>(&Bs[buf][b_lds[i]]) = rb[i];
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const u32x4_t *>(
            &As[buf][(wm * WTM + fm * 16 + (lane & 15)) * LDSP + kk * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = *reinterpret_cast<const u32x4_t *>(
            &Bs[buf][(wn * WTN + fn * 16 + (lane & 15)) * LDSP + kk * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(af[fm], bfr[fn], acc[fm][fn]);
    }
  };

  if constexpr (MODE == MODE_SHRINK) {
    const int steps_total = (P.K + BK - 1) / BK;
    const int s0 = col * P.k_steps_per_split;
    const int s1 = min(steps_total, s0 + P.k_steps_per_split);
    for (int a = 0; a < P.num_slots; ++a) {
      if (!((slot_mask >> a) & 1)) continue;
      const int r_a = P.rank[a];
      const uint16_t *bbase = P.lora_w[a] + (size_t)e * r_a * P.K;
      zero_acc();
      load_main(s0 * BK, bbase, r_a);
      store_lds(0);
      __syncthreads();
      for (int s = s0; s < s1; ++s) {
        const int cur = (s - s0) & 1;
        if (s + 1 < s1) load_main((s + 1) * BK, bbase, r_a);
        compute(cur);
        if (s + 1 < s1) store_lds(cur ^ 1);
        __syncthreads();
      }
      // rows of this slot, rank columns
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            const int n = wn * WTN + fn * 16 + (lane & 15);
            if (r < rows && n < r_a && s_slot[r] == a)
              P.out_f32[((size_t)col * P.R + row0 + r) * P.rmax + n] = acc[fm][fn][i];
          }
    }
    return;
  } else {
    const int main_steps = kHasMain ? (P.K + BK - 1) / BK : 0;
    const int n_ext = kHasExt ? __popc(slot_mask) : 0;
    const int nsteps = main_steps + n_ext;
    const uint16_t *wbase = kHasMain ? P.w + (size_t)e * P.N * P.K : nullptr;
    const int wcount = kGateUp ? 2 * P.I : P.N;
    auto load_step = [&](int s) {
      if (s < main_steps) {
        load_main(s * BK, wbase, wcount);
      } else {
        int m = slot_mask;
        for (int q = 0; q < s - main_steps; ++q) m &= m - 1;
        load_ext(__ffs(m) - 1);
      }
    };
    zero_acc();
    if (nsteps > 0) {
      load_step(0);
      store_lds(0);
      __syncthreads();
      for (int s = 0; s < nsteps; ++s) {
        const int cur = s & 1;
        if (s + 1 < nsteps) load_step(s + 1);
        compute(cur);
        if (s + 1 < nsteps) store_lds(cur ^ 1);
        __syncthreads();
      }
    }

    if constexpr (kGateUp) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fh = 0; fh < FN / 2; ++fh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            const int icol = col * (BN / 2) + wn * (WTN / 2) + fh * 16 + (lane & 15);
            if (r < rows && icol < P.I) {
              const float g = acc[fm][fh][i];
              const float u = acc[fm][fh + FN / 2][i];
              const float h = g / (1.0f + expf(-g)) * u;
              P.out_bf16[(size_t)(row0 + r) * P.I + icol] = (uint16_t)f32_to_bf16(h);
            }
          }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            const int n = col * BN + wn * WTN + fn * 16 + (lane & 15);
            if (r < rows && n < P.N) {
              if constexpr (MODE == MODE_DOWN)
                P.out_bf16[(size_t)(row0 + r) * P.N + n] = (uint16_t)f32_to_bf16(acc[fm][fn][i]);
              else
                P.out_f32[(size_t)(row0 + r) * P.N + n] = acc[fm][fn][i];
            }
          }
    }
  }
}

// ---------------------------------------------------------------- host side
struct TileCfg {
  int bm;
};

inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int mtile_bound(int R, int E, int BM) {
  const long long nonempty = R < E ? R : E;
  return (int)((R + nonempty * (BM - 1) + BM - 1) / BM);
}

// tile height from the mean rows per expert (the routed load is only known on device)
int pick_bm(int R, int E) {
  const int avg = R / (E > 0 ? E : 1);
  if (avg <= 16) return 16;
  if (avg <= 48) return 32;
  if (avg <= 128) return 64;
  return 128;
}

int shrink_bm(int R, int E) { return (R / (E > 0 ? E : 1)) <= 48 ? 32 : 128; }

int shrink_splits(int R, int E, int K, int &steps_per_split) {
  const int steps = cdiv(K, BK);
  const int tiles = mtile_bound(R, E, shrink_bm(R, E));
  int want = cdiv(2048, tiles > 0 ? tiles : 1);
  if (want < 1) want = 1;
  if (want > steps) want = steps;
  steps_per_split = cdiv(steps, want);
  return cdiv(steps, steps_per_split);
}

int rmax8(const moe_lora_adapters *lora) {
  int r = 0;
  for (int s = 0; s < lora->num_slots; ++s) r = lora->rank[s] > r ? lora->rank[s] : r;
  return (r + 7) & ~7;
}

template <int BM, int BN, int WM, int WN, int MODE>
int launch_cfg(const GemmParams &P, int n_cols, hipStream_t s) {
  int tiles = mtile_bound(P.R, P.E, BM);
  long long blocks = (long long)tiles * n_cols;
  blocks = (blocks + 7) & ~7ll;
  if (blocks == 0) return ST_OK;
  GemmParams Q = P;
  Q.n_cols = n_cols;
  moe_gemm_kernel<BM, BN, WM, WN, MODE><<<dim3((unsigned)blocks), dim3(WM * WN * 64), 0, s>>>(Q);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

template <int MODE>
int launch_gemm(const GemmParams &P, int bm, hipStream_t s) {
  const int BN = 128;
  const int ncols = (MODE == MODE_GATEUP) ? cdiv(P.I, BN / 2) : cdiv(P.N, BN);
  switch (bm) {
    case 16: return launch_cfg<16, 128, 1, 4, MODE>(P, ncols, s);
    case 32: return launch_cfg<32, 128, 1, 4, MODE>(P, ncols, s);
    case 64: return launch_cfg<64, 128, 2, 2, MODE>(P, ncols, s);
    default: return launch_cfg<128, 128, 2, 2, MODE>(P, ncols, s);
  }
}

int launch_shrink(const GemmParams &P, int bm, int splits, hipStream_t s) {
  if (bm <= 32) return launch_cfg<32, 64, 2, 2, MODE_SHRINK>(P, splits, s);
  return launch_cfg<128, 64, 2, 2, MODE_SHRINK>(P, splits, s);
}

struct FwdLayout {
  size_t u_part = 0, act = 0, v_part = 0, total = 0;
  int splits1 = 0, steps1 = 0, splits2 = 0, steps2 = 0, rmax = 0;
};

FwdLayout layout(const moe_lora_dims &d, const moe_lora_adapters *lora) {
  FwdLayout L;
  const size_t R = (size_t)d.num_tokens * d.top_k;
  const bool has_lora = lora && lora->num_slots > 0;
  size_t off = 0;
  if (has_lora) {
    L.rmax = rmax8(lora);
    L.splits1 = shrink_splits((int)R, d.num_experts, d.hidden, L.steps1);
    L.splits2 = shrink_splits((int)R, d.num_experts, d.inter, L.steps2);
    L.u_part = off;
    off = align256(off + (size_t)L.splits1 * R * L.rmax * sizeof(float));
  }
  L.act = off;
  off = align256(off + R * d.inter * sizeof(uint16_t));
  if (has_lora) {
    L.v_part = off;
    off = align256(off + (size_t)L.splits2 * R * L.rmax * sizeof(float));
  }
  L.total = off;
  return L;
}

}  // namespace

size_t forward_workspace_size(const moe_lora_dims &d, const moe_lora_adapters *lora) {
  return layout(d, lora).total;
}

int launch_forward(const moe_lora_dims &d, const uint16_t *x, const uint16_t *x_perm,
                   const int32_t *offsets, const int32_t *p2e, const uint16_t *w1,
                   const uint16_t *w2, const moe_lora_adapters *lora, uint16_t *y_perm, void *ws,
                   size_t ws_bytes, hipStream_t main, hipStream_t side,
                   const moe_lora_options *opts) {
  (void)side;
  const int R = d.num_tokens * d.top_k;
  if (R == 0) return ST_OK;
  const FwdLayout L = layout(d, lora);
  if (ws_bytes < L.total) return ST_WS_SMALL;
  char *wsb = static_cast<char *>(ws);
  const bool has_lora = lora && lora->num_slots > 0;
  uint16_t *act = reinterpret_cast<uint16_t *>(wsb + L.act);
  float *u_part = has_lora ? reinterpret_cast<float *>(wsb + L.u_part) : nullptr;
  float *v_part = has_lora ? reinterpret_cast<float *>(wsb + L.v_part) : nullptr;

  GemmParams base{};
  base.p2e = p2e;
  base.offsets = offsets;
  base.E = d.num_experts;
  base.top_k = d.top_k;
  base.R = R;
  base.I = d.inter;
  if (has_lora) {
    base.num_slots = lora->num_slots;
    base.token_slot = lora->token_slot;
    for (int s = 0; s < lora->num_slots; ++s) {
      base.rank[s] = lora->rank[s];
      base.scaling[s] = lora->scaling[s];
    }
    base.rmax = L.rmax;
  }
  const uint16_t *a_src = x_perm ? x_perm : x;
  const int a_gather = x_perm ? 0 : 1;
  const int bm = pick_bm(R, d.num_experts);
  int st;

  // 1) gate_up LoRA shrink: u_part = A1 . x  (split over H)
  if (has_lora) {
    GemmParams P = base;
    P.a = a_src;
    P.a_gather = a_gather;
    P.K = d.hidden;
    P.N = 0;
    P.k_steps_per_split = L.steps1;
    for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->a_gate_up[s];
    P.out_f32 = u_part;
    if ((st = launch_shrink(P, shrink_bm(R, d.num_experts), L.splits1, main)) != ST_OK) return st;
  }
  // 2) gate_up GEMM + LoRA expand + SwiGLU -> act
  {
    GemmParams P = base;
    P.a = a_src;
    P.a_gather = a_gather;
    P.w = w1;
    P.K = d.hidden;
    P.N = 2 * d.inter;
    if (has_lora) {
      for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->b_gate_up[s];
      P.part = u_part;
      P.part_splits = L.splits1;
    }
    P.out_bf16 = act;
    hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->gate_up_event_begin) : nullptr;
    hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->gate_up_event_end) : nullptr;
    if (ev0 && hipEventRecord(ev0, main) != hipSuccess) return ST_HIP;
    if ((st = launch_gemm<MODE_GATEUP>(P, bm, main)) != ST_OK) return st;
    if (ev1 && hipEventRecord(ev1, main) != hipSuccess) return ST_HIP;
  }
  // 3) down LoRA shrink: v_part = A2 . act  (split over I)
  if (has_lora) {
    GemmParams P = base;
    P.a = act;
    P.a_gather = 0;
    P.K = d.inter;
    P.N = 0;
    P.k_steps_per_split = L.steps2;
    for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->a_down[s];
    P.out_f32 = v_part;
    if ((st = launch_shrink(P, shrink_bm(R, d.num_experts), L.splits2, main)) != ST_OK) return st;
  }
  // 4) down GEMM + down LoRA expand -> y_perm (unweighted)
  {
    GemmParams P = base;
    P.a = act;
    P.a_gather = 0;
    P.w = w2;
    P.K = d.inter;
    P.N = d.hidden;
    if (has_lora) {
      for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->b_down[s];
      P.part = v_part;
      P.part_splits = L.splits2;
    }
    P.out_bf16 = y_perm;
    if ((st = launch_gemm<MODE_DOWN>(P, bm, main)) != ST_OK) return st;
  }
  return ST_OK;
}

}  // namespace moe
