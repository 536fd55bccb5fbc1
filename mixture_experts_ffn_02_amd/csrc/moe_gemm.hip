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
// through double-buffered LDS (unpadded 128-byte rows, 16-byte chunks XOR-swizzled by
// row), v_mfma_f32_16x16x32_bf16 on 64-wide wavefronts.  Work tiles are (expert,
// m-tile, n-tile) triples found on the device from expert_offsets; block ids are
// remapped so each XCD runs a contiguous range of them, keeping an expert's weight and
// activation tiles in that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

enum { MODE_GATEUP = 0, MODE_DOWN = 1, MODE_SHRINK = 2, MODE_GATEUP_F32 = 3, MODE_EXPAND_F32 = 4 };

constexpr int BK = 64;
// LDS tiles hold rows of BK = 64 bf16 (128 bytes, unpadded) with the row's eight 16-byte
// chunks XOR-swizzled by (row & 7): the staging stores (8 lanes per row) and the MFMA
// fragment reads (16 rows per instruction) then both run at full LDS bandwidth on gfx950,
// where a padded 72-element pitch halves the fragment read rate.
MOE_DEV int lds_off(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

// One 16-byte chunk per lane from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l of the wave writes LDS bytes [base + 16 l, base + 16 l + 16).
// No registers hold the data and nothing waits for it here; like any vector load it counts
// in vmcnt, so a later wait for a younger load also covers it.  M0 carries the wave's LDS
// base and is restored afterwards.
MOE_DEV void lds_dma16(const void *src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

MOE_DEV uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void *)p));
}

struct GemmParams {
  const uint16_t *a;  // A rows: x [T, K] when a_gather, else [R, K] in permuted order
  const int32_t *p2e;
  int a_gather;
  const uint16_t *w;  // [E, N, K] (unused by SHRINK / EXPAND)
  int N, K, I;
  const int32_t *offsets;
  int E, top_k, R;
  int n_cols;  // n-tiles (GEMM modes) or K splits x slot groups (SHRINK)
  int k_steps_per_split;
  int slot_groups;  // SHRINK: blocks per (m-tile, K split), one per BN-wide chunk of each slot's ranks
  int num_slots;
  const int32_t *token_slot;
  int rank[MOE_LORA_MAX_SLOTS];
  float scaling[MOE_LORA_MAX_SLOTS];
  const uint16_t *lora_w[MOE_LORA_MAX_SLOTS];  // SHRINK: A [E, r, K]; ext: B [E, N, r]
  int lora_w_shared;  // lora_w holds one matrix per slot for all experts (shared-outer)
  int w_packed;       // w is in the tile-packed layout (128-row x 64-column blocks)
  // FP8 weights (kernels instantiated with W8 = 1, or 2 when every block scale is a power
  // of two): w holds E4M3 codes [E, N, K] (one byte each) and w_scale one fp32 scale per
  // 128 x 128 block, [E, N/128, K/128]
  const float *w_scale;
  const float *part;                            // ext A source [splits][R][rmax]
  int part_splits;
  // ext A source already reduced over the splits, scaled and rounded: bf16 [R][rmax]
  // (zero past each row's rank); when set, part / part_splits are not read
  const uint16_t *part_bf16;
  int rmax;
  uint16_t *out_bf16;
  float *out_f32;
  // gate_up only: fused down-LoRA shrink partials v_part[n_tile][p][0:r] = A2[slot][e] . act
  // over the tile's I columns (NULL = not fused)
  const uint16_t *down_a[MOE_LORA_MAX_SLOTS];  // [E, r, I]
  float *down_part;                            // [n_tiles][R][rmax]
  // adapter slot of each permuted row (-1 = none): written by the gate_up shrink, read by
  // the later LoRA kernels instead of token_slot[p2e[p] / k] (one dependent load fewer)
  int32_t *row_slot_out;
  const int32_t *row_slot;
  // persistent tiles only: walk each expert's tiles m-tile first (the m-tiles that read one
  // weight slice run side by side on one XCD and share it in its L2) in per-XCD shares
  int mt_fast;
};

// Register budget: two waves per SIMD (256 VGPRs), or three (168 VGPRs, as many 16-row
// blocks as the LDS holds) for the 16-row down tiles and the 16-row FP8 gate_up tiles,
// which run two register stages at that budget (decode down 72 -> 67.5 us; FP8 gate_up
// 78 -> 75.6 us, FP8 down 54 -> 51 us).  The bf16 16-row gate_up keeps two waves and four
// stages: with three it is ~1 % slower, and with four stages at three waves its stages
// and LoRA code spill to scratch on every tile (155 against 131 us).
template <int BM, int BN, int WM, int WN, int MODE, int PF, int W8 = 0>
__global__ __launch_bounds__(WM *WN * 64)
__attribute__((amdgpu_waves_per_eu((BM <= 16 && (MODE == MODE_DOWN || (W8 && MODE == MODE_GATEUP))) ? 3 : 2)))
void moe_gemm_kernel(const GemmParams P) {
  static_assert(!W8 || MODE == MODE_GATEUP || MODE == MODE_DOWN, "FP8 weights feed the gate_up and down GEMMs");
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_CH = BM * (BK / 8), B_CH = BN * (BK / 8);
  // FP8 weights: 16-byte chunks of 16 codes (two bf16 LDS chunks each, or one chunk of
  // codes on the 16-row tiles)
  constexpr int B8_CH = BN * (BK / 16), B8_IT = (B8_CH + WM * WN * 64 - 1) / (WM * WN * 64);
  // slots whose expand B rows ride in the register stages at once (a deep FP8 pipeline
  // would otherwise multiply those registers)
  constexpr int EB = PF < 4 ? PF : 4;
  constexpr int A_IT = (A_CH + NT - 1) / NT, B_IT = (B_CH + NT - 1) / NT;
  constexpr bool kGateUp = (MODE == MODE_GATEUP);
  constexpr bool kHasMain = (MODE != MODE_EXPAND_F32);
  constexpr bool kHasExt = (MODE == MODE_GATEUP || MODE == MODE_DOWN || MODE == MODE_EXPAND_F32);
  // Decode-height tiles whose expert has no other m-tile read each weight row exactly once
  // per launch: those stream it past the caches (non-temporal loads, ~10-15 % more HBM
  // read bandwidth on MI355X); weights shared by several m-tiles keep normal loads so the
  // other blocks hit in L2.
  constexpr bool kStreamB = BM <= 64 && MODE != MODE_SHRINK;
  constexpr bool kPersistent = BM >= 64;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(!kGateUp || (FN % 2 == 0), "gate/up pairing needs an even fragment count");
  static_assert(PF >= 2 && PF % 2 == 0, "prefetch depth must be even (two LDS buffers)");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  // FP8 weights with block-sum scaling on 16-row tiles: the B stages hold the E4M3 codes
  // themselves (rows of 64 codes, 16-byte chunks XOR-swizzled by (row / 4) % 4, so that
  // the 8-byte fragment reads of a half-wave hit 32 distinct bank pairs), and each wave
  // converts its own fragments after reading them: half the LDS bytes written and read per
  // K step (decode FP8 gate_up 75.4 -> 73.8 us, down 49.6 -> 48.5 us).  The four blocks
  // per CU that the smaller LDS would allow need 128 registers, and the spills that takes
  // cost more (gate_up 85.6 us).  The expand and the epilogue see both halves as one bf16
  // buffer.
  constexpr bool kW8Raw = W8 == 1 && BM <= 16;
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kW8Raw ? BN * BK / 2 : BN * BK];
  constexpr int kBsElems = 2 * (kW8Raw ? BN * BK / 2 : BN * BK);
  __shared__ int s_src[BM];
  __shared__ int s_slot[BM];
  __shared__ int s_mask[2];  // slots present in the tile, by tile parity
  __shared__ int s_off[MOE_LORA_MAX_EXPERTS + 1];   // expert_offsets
  __shared__ int s_tpre[MOE_LORA_MAX_EXPERTS + 1];  // first m-tile index of each expert
  // rank of each slot, for code that looks it up by a row's slot (P.rank[a] with a
  // per-lane a is a vector load from the argument block, which waits behind the weight
  // stream)
  __shared__ int s_rank[MOE_LORA_MAX_SLOTS];
  __shared__ float s_scal[MOE_LORA_MAX_SLOTS];  // and its scaling
  // FP8 weights: the tile's block scales, [2 row blocks][K / 128 <= 64] (gate_up: the gate
  // and the up block of the tile's columns; down: the tile's one or two row blocks)
  __shared__ float s_wsc[W8 ? 2 * 64 : 1];
  // LoRA expand A operand of the tile: row r holds bf16(s_a * sum of shrink partials) over
  // the rank columns of its own slot (zero elsewhere); built once, masked per slot later
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kHasExt ? BM * BK : 8];
  // gate_up with the fused down shrink on tiles of 64 rows or more: the tile's A2 slices,
  // copied into LDS when the tile starts so that their latency overlaps the K loop instead
  // of the epilogue (rows of all slots packed at 16-row granularity, HC elements per row
  // with the 16-byte chunks XOR-swizzled by row).  Decode-height tiles keep the LDS and
  // registers this would take (other blocks on the CU hide their epilogue).
  constexpr int HC = BN / 2, HP = HC + 8;
  constexpr bool kA2Pre = kGateUp && BM >= 64;
  constexpr int kA2Rows = 128;
  static_assert((kA2Rows * HC / 8) % 64 == 0, "A2 region must be whole wave copies");
  __shared__ __attribute__((aligned(16))) uint16_t A2p[kA2Pre ? kA2Rows * HC : 8];
  // Tiles whose rows all use one adapter slot of rank <= 32 (a multiple of 8): that slot's
  // B rows for the tile's BN output columns, copied into LDS when the tile starts (32
  // ranks per row, 16-byte chunks XOR-swizzled by row / 4), so the expand is one unmasked
  // 32-wide K step from LDS instead of a register-staged step that waits for its loads
  // at the end of the tile.  Decode-height tiles and the 64-row down GEMM have the LDS
  // for it (on the 128x256 down tile the extra addressing spilled in the K loop; the
  // 32-row down tile fits three blocks per CU only without it).
  constexpr bool kExtLds = kHasExt && kHasMain && (BM <= 16 || (MODE == MODE_DOWN && BM == 64));
  constexpr int kEbRank = 32;
  static_assert(!kExtLds || (BN * kEbRank / 8) % 64 == 0, "expand B region must be whole wave copies");
  __shared__ __attribute__((aligned(16))) uint16_t Eb[kExtLds ? BN * kEbRank : 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile list, once per block: expert offsets and each expert's first m-tile index in
  // LDS.  Tall tiles (prefill) run persistent blocks that loop over tiles; decode-height
  // tiles take one tile per block.  The hardware places block b on XCD b % 8.
  for (int i = tid; i <= P.E; i += NT) s_off[i] = P.offsets[i];
#pragma unroll
  for (int s2 = 0; s2 < MOE_LORA_MAX_SLOTS; ++s2)
    if (tid == s2) {
      s_rank[s2] = P.rank[s2];
      s_scal[s2] = P.scaling[s2];
    }
  __syncthreads();
  if (wave == 0) {
    const int per = (P.E + 63) / 64;
    int local = 0;
    for (int q = 0; q < per; ++q) {
      const int ex = lane * per + q;
      if (ex < P.E) local += (s_off[ex + 1] - s_off[ex] + BM - 1) / BM;
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int run = incl - local;
    for (int q = 0; q < per; ++q) {
      const int ex = lane * per + q;
      if (ex < P.E) {
        s_tpre[ex] = run;
        run += (s_off[ex + 1] - s_off[ex] + BM - 1) / BM;
      }
    }
    if (lane == 63) s_tpre[P.E] = incl;
    if (lane < 2) s_mask[lane] = 0;
  }
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(s_tpre[P.E]) * P.n_cols;

  // ---- the (m-tile, column) work tiles of this block.  Persistent blocks (a grid of
  // resident blocks, a multiple of 8): block j of XCD x walks a contiguous share of the
  // tiles, so the blocks of an XCD work on neighbouring tiles at any moment.  Otherwise
  // (grid = a bound on the tile count, padded to a multiple of 8) one tile per block,
  // consecutive tiles on one XCD; the loop below then runs at most once.
  int L, L_end, L_step;
  if constexpr (kPersistent) {
    const int per_xcd = (total + 7) >> 3;
    L = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    L_end = min(total, (int)(blockIdx.x & 7) * per_xcd + per_xcd);
    L_step = (int)(gridDim.x >> 3);
    if (BM <= 64 && P.w_packed && !P.mt_fast && total >= 8 * (int)gridDim.x) {
      // 64-row tiles, many per block: on packed weights the grid walks the tiles in
      // launch order, front to back through the packed buffer (DeepSeek-V3-sized layer,
      // 16 and 28 tiles per block: 3.53 -> 3.28 ms).  128-row tiles keep the per-XCD
      // shares, whose L2 reuse they need (prefill 1.18 ms against 1.29 ms otherwise), and
      // so do grids with a few tiles per block (multi-adapter T=256, 3 and 4: ~1 % faster)
      L = (int)blockIdx.x;
      L_end = total;
      L_step = (int)gridDim.x;
    }
  } else {
    // One tile per block, each XCD a contiguous share of the tiles (consecutive tiles of an
    // expert share its weights and adapter rows in that XCD's L2).  The shares are cut
    // from the actual tile count: the grid is only a bound (every expert may add a partial
    // m-tile), and shares of the bound left the last XCDs without tiles (multi-adapter
    // T=256: ~190 of 248 m-tiles exist, so two of the eight XCDs idled through the LoRA
    // shrink; decode on row-major weights, gate_up 146 -> 130 us).  With the shares cut
    // this way the tile-packed weights stream as fast as in launch order (decode gate_up
    // 123 us either way).  Blocks past their XCD's share take no tile.
    const int per_xcd = (total + 7) >> 3, j = (int)(blockIdx.x >> 3);
    L = (int)(blockIdx.x & 7) * per_xcd + j;
    L_end = j < per_xcd ? total : 0;
    L_step = 0;
  }
  int parity = 0;
  for (; L < L_end; L += L_step, parity ^= 1) {
  // tile L -> (m-tile, column): column fastest, or m-tile fastest within the expert (the
  // expert's tiles fill the same range of L either way)
  int mt = L / P.n_cols, col = L % P.n_cols;
  // expert of m-tile mt: last e with s_tpre[e] <= mt (binary search, same in every lane)
  int lo_e = 0, hi_e = P.E;  // invariant: s_tpre[lo_e] <= mt < s_tpre[hi_e]
  while (hi_e - lo_e > 1) {
    const int mid = (lo_e + hi_e) >> 1;
    if (s_tpre[mid] <= mt) lo_e = mid;
    else hi_e = mid;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo_e);  // block-uniform values in SGPRs
  if (kPersistent && P.mt_fast) {
    const int t0 = __builtin_amdgcn_readfirstlane(s_tpre[e]);
    const int nm = __builtin_amdgcn_readfirstlane(s_tpre[e + 1]) - t0;
    const int local = L - t0 * P.n_cols;
    col = local / nm;
    mt = t0 + local % nm;
  }
  const int cnt = __builtin_amdgcn_readfirstlane(s_off[e + 1] - s_off[e]);
  const int m0 = (mt - __builtin_amdgcn_readfirstlane(s_tpre[e])) * BM;
  const int row0 = __builtin_amdgcn_readfirstlane(s_off[e]) + m0;
  const int rows = min(BM, cnt - m0);

  const bool need_tok = P.a_gather || (P.num_slots > 0 && !P.row_slot);
  for (int r = tid; r < BM; r += NT) {
    int src = -1, slot = -1;
    if (r < rows) {
      const int p = row0 + r;
      const int tok = need_tok ? P.p2e[p] / P.top_k : 0;
      src = P.a_gather ? tok : p;
      if (P.num_slots > 0) {
        const int s = P.row_slot ? P.row_slot[p] : P.token_slot[tok];
        slot = (s >= 0 && s < P.num_slots) ? s : -1;
      }
      if (MODE == MODE_SHRINK && P.row_slot_out && col == 0) P.row_slot_out[p] = slot;
    }
    s_src[r] = src;
    s_slot[r] = slot;
    if (slot >= 0) atomicOr(&s_mask[parity], 1 << slot);
  }
  if constexpr (W8) {
    const int KB = P.K / 128, NB = P.N / 128;
    for (int q = tid; q < 2 * KB; q += NT) {
      const int j = q / KB, kb = q % KB;
      const int rblk = kGateUp ? ((j ? P.I : 0) + col * (BN / 2)) / 128 : (col * BN) / 128 + j;
      s_wsc[q] = rblk < NB ? P.w_scale[((size_t)e * NB + rblk) * KB + kb] : 0.f;
    }
  }
  __syncthreads();
  const int slot_mask = __builtin_amdgcn_readfirstlane(s_mask[parity]);
  // the expert's rows fit this one tile: its weight rows are read by no other block
  const bool single_mtile = cnt <= BM;

  // ---- per-thread chunk geometry (fixed for the whole K loop).  Threads without a chunk,
  // padding rows and weight rows past N read a valid row instead (never stored or masked
  // out later), so the steady-state loads carry no predicate and stay in flight.
  const int src0 = s_src[0];
  const uint16_t *a_ptr[A_IT];
  int a_lds[A_IT], a_row[A_IT], a_c8[A_IT];
  bool a_has[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int c = tid + i * NT;
    const int cc = c < A_CH ? c : c % A_CH;
    const int r = cc >> 3;
    a_has[i] = c < A_CH;
    a_row[i] = r;
    a_c8[i] = cc & 7;
    a_lds[i] = lds_off(r, cc & 7);
    const int src = s_src[r] >= 0 ? s_src[r] : src0;
    a_ptr[i] = (kHasMain && src >= 0) ? P.a + (size_t)src * P.K + (cc & 7) * 8 : nullptr;
  }
  int b_wrow[B_IT], b_lds[B_IT], b_c8[B_IT];
  int b_pk[B_IT];  // tile-packed weights: offset of the chunk in its expert's block at K step 0
  bool b_has[B_IT];
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int c = tid + i * NT;
    const int cc = c < B_CH ? c : c % B_CH;
    const int n = cc >> 3;
    b_has[i] = c < B_CH;
    b_c8[i] = cc & 7;
    b_lds[i] = lds_off(n, cc & 7);
    if (MODE == MODE_SHRINK) {
      b_wrow[i] = n;  // rank row, checked against the slot's rank
    } else if (kGateUp || MODE == MODE_GATEUP_F32) {
      // gate/up row blocks (see brow()); the fp32 gate_up GEMM of the decomposed path keeps
      // them too, so that both read the packed layout, and maps them back on its store
      const int icol = col * (BN / 2) + (n / 128) * 64 + n % 64;
      b_wrow[i] = (icol < P.I) ? ((n % 128) / 64) * P.I + icol : -1;
    } else {
      const int ng = col * BN + n;
      b_wrow[i] = (ng < P.N) ? ng : -1;
    }
    // packed block (e, s, t) holds rows 128 t .. of the LDS order above for K step s
    b_pk[i] = 0;
    // (padding rows of a 256-wide tile past the last 128-row tile read tile 0 instead: their
    // block would lie past the expert's region)
    if constexpr (BN % 128 == 0) {
      int tt = col * (BN / 128) + n / 128;
      if (tt >= (kGateUp || MODE == MODE_GATEUP_F32 ? 2 * P.I : P.N) / 128) tt = 0;
      b_pk[i] = (tt * 128 + n % 128) * BK + (cc & 7) * 8;
    }
  }

  // FP8 main-loop chunks: byte offset (row, 16 columns) in the expert's code matrix at K
  // step 0, the two LDS chunk offsets, and the chunk's scale row in s_wsc
  uint32_t b8_lo[W8 ? B8_IT : 1], b8_pk[W8 ? B8_IT : 1];  // row-major / tile-packed codes
  int b8_lds[W8 ? B8_IT : 1], b8_lds2[W8 ? B8_IT : 1], b8_sj[W8 ? B8_IT : 1];
  int b8_raw[W8 ? B8_IT : 1];  // codes kept in LDS: the chunk's offset (16-bit units)
  if constexpr (W8) {
#pragma unroll
    for (int i = 0; i < B8_IT; ++i) {
      const int c = tid + i * NT;
      const int cc = c < B8_CH ? c : c % B8_CH;
      const int n = cc >> 2, c16 = cc & 3;
      int wr;
      if constexpr (kGateUp) {
        const int icol = col * (BN / 2) + (n / 128) * 64 + n % 64;  // see brow()
        wr = icol < P.I ? ((n % 128) / 64) * P.I + icol : 0;
        b8_sj[i] = (n % 128) / 64;
      } else {
        const int ng = col * BN + n;
        wr = ng < P.N ? ng : 0;
        b8_sj[i] = n / 128;
      }
      b8_lo[i] = (uint32_t)wr * (uint32_t)P.K + (uint32_t)c16 * 16u;
      // packed: block (e, s, t) of 128 rows x 64 codes, t = the LDS row's 128-row tile
      int tt = col * (BN / 128) + n / 128;
      if (tt >= P.N / 128) tt = 0;  // padding rows past the last tile (see b_pk)
      b8_pk[i] = (uint32_t)((tt * 128 + n % 128) * 64 + c16 * 16);
      b8_lds[i] = lds_off(n, 2 * c16);
      b8_lds2[i] = lds_off(n, 2 * c16 + 1);
      b8_raw[i] = n * (BK / 2) + ((c16 ^ ((n >> 2) & 3)) << 3);
    }
  }

  u32x4_t ra[PF][A_IT], rb[PF][B_IT];
  f32x4_t acc[FM][FN];
  // FP8 weights with general block scales on tiles of up to 64 rows: the codes enter the
  // MFMAs unscaled (every E4M3 value is exact in bf16), and the sum over each 128-wide K
  // block is scaled into acc8 when the block's second K step has been computed (w8_kb:
  // the next block's index).  The 128-row tiles have no registers for a second set of
  // accumulators and scale each weight before the MFMAs instead.
  constexpr bool kW8Acc = W8 == 1 && BM <= 64;
  f32x4_t acc8[kW8Acc ? FM : 1][kW8Acc ? FN : 1];
  int w8_kb = 0;

  auto zero_acc = [&]() {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // full 64-wide K step, no predicates (see above)
  // (pk: B from the tile-packed layout, where one K step of 128 rows is one contiguous
  // 16 KB block and the blocks of one K step are adjacent)
  auto load_full = [&](int k0, const uint16_t *bbase, int bcount, u32x4_t(&xa)[A_IT],
                       u32x4_t(&xb)[B_IT], auto nt, auto pk) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) xa[i] = *reinterpret_cast<const u32x4_t *>(a_ptr[i] + k0);
    // B through a raw buffer resource on the expert's matrix: a 32-bit per-lane byte
    // offset that does not change along K plus the K step's byte offset in a scalar
    // register.  Plain global loads kept one 64-bit address per lane for every chunk of
    // every register stage (a quarter of the register file on the 16-row tiles).  One
    // expert matrix is < 2 GiB (checked by the host), so both offsets fit 32 bits.
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(bbase), (short)0, 0x7fffffff, 0x00020000);
    if constexpr (W8) {
      // FP8 weights (row-major, bbase = the expert's first code byte): 16 codes per chunk;
      // store_lds converts them into bf16 or, on 16-row tiles, stores the codes
      // (packed: the K step's blocks start k0 * N bytes into the expert's region)
      const int soff8 = decltype(pk)::value ? k0 * P.N : k0;
#pragma unroll
      for (int i = 0; i < B8_IT; ++i)
        xb[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, decltype(pk)::value ? b8_pk[i] : b8_lo[i],
                                                           soff8, decltype(nt)::value ? 2 : 0));
      return;
    }
    const int soff = decltype(pk)::value ? (k0 / BK) * P.N * BK * 2 : k0 * 2;
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      uint32_t lo;
      if constexpr (decltype(pk)::value) {
        lo = (uint32_t)b_pk[i] * 2u;
      } else {
        const int wr = (b_wrow[i] >= 0 && b_wrow[i] < bcount) ? b_wrow[i] : 0;
        lo = ((uint32_t)wr * (uint32_t)P.K + (uint32_t)b_c8[i] * 8u) * 2u;
      }
      // aux 2: non-temporal (the weights are streamed once)
      xb[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              rsrc, lo, soff, decltype(nt)::value ? 2 : 0));
    }
  };
  // ragged K tail and padding rows zeroed (used once, off the steady state)
  auto load_tail = [&](int k0, const uint16_t *bbase, int bcount, u32x4_t(&xa)[A_IT],
                       u32x4_t(&xb)[B_IT]) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      xa[i] = zero_u32x4();
      if (a_ptr[i] && a_row[i] < rows && k0 + a_c8[i] * 8 < P.K)
        xa[i] = *reinterpret_cast<const u32x4_t *>(a_ptr[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      xb[i] = zero_u32x4();
      const int wr = b_wrow[i];
      if (wr >= 0 && wr < bcount && k0 + b_c8[i] * 8 < P.K)
        xb[i] = *reinterpret_cast<const u32x4_t *>(bbase + (size_t)wr * P.K + k0 + b_c8[i] * 8);
    }
  };

  // threads past the chunk count hold a duplicate of another thread's chunk, so every
  // thread stores unconditionally (identical values to the same address)
  // (step: the K step being stored, which picks the FP8 block scale)
  auto store_lds = [&](int buf, const u32x4_t(&xa)[A_IT], const u32x4_t(&xb)[B_IT], int step) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) *reinterpret_cast<u32x4_t *>(&As[buf][a_lds[i]]) = xa[i];
    if constexpr (W8) {
      // 16 E4M3 codes (element j in byte j): kept as codes, or -> bf16
      const int kb = step >> 1, KB = P.K / 128;
      if constexpr (kW8Raw) {
#pragma unroll
        for (int i = 0; i < B8_IT; ++i) *reinterpret_cast<u32x4_t *>(&Bs[buf][b8_raw[i]]) = xb[i];
      } else if constexpr (W8 == 2 || kW8Acc) {
        // one conversion per two codes (exact): scaled by a power-of-two block scale, or
        // unscaled (see acc8)
#pragma unroll
        for (int i = 0; i < B8_IT; ++i) {
          const float sc = W8 == 2 ? s_wsc[b8_sj[i] * KB + kb] : 1.0f;
          u32x4_t o[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int w0 = (int)xb[i][2 * h], w1 = (int)xb[i][2 * h + 1];
            o[h] = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true))};
          }
          *reinterpret_cast<u32x4_t *>(&Bs[buf][b8_lds[i]]) = o[0];
          *reinterpret_cast<u32x4_t *>(&Bs[buf][b8_lds2[i]]) = o[1];
        }
      } else {
        // -> fp32 (exact) * block scale -> bf16
#pragma unroll
        for (int i = 0; i < B8_IT; ++i) {
          const float sc = s_wsc[b8_sj[i] * KB + kb];
          u32x4_t o[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int w0 = (int)xb[i][2 * h], w1 = (int)xb[i][2 * h + 1];
            const f32x2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
            const f32x2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
            const f32x2_t f2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
            const f32x2_t f3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
            o[h] = u32x4_t{pack_bf16x2(f0.x * sc, f0.y * sc), pack_bf16x2(f1.x * sc, f1.y * sc),
                           pack_bf16x2(f2.x * sc, f2.y * sc), pack_bf16x2(f3.x * sc, f3.y * sc)};
          }
          *reinterpret_cast<u32x4_t *>(&Bs[buf][b8_lds[i]]) = o[0];
          *reinterpret_cast<u32x4_t *>(&Bs[buf][b8_lds2[i]]) = o[1];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_IT; ++i) *reinterpret_cast<u32x4_t *>(&Bs[buf][b_lds[i]]) = xb[i];
    }
  };

  // Fragment rows are 16-aligned bases plus (lane & 15), so the swizzle depends on the lane
  // alone: one per-lane offset per 32-wide K chunk, everything else folds into immediates.
  // First LDS row of B fragment fn of this wave.  gate_up tiles keep their B rows in blocks
  // of 128, [64 gate rows | the 64 up rows of the same intermediate columns], so that a
  // 128-row block is one tile of the packed weight layout; fragment fn < FN/2 is a gate
  // fragment and fn + FN/2 the up fragment of the same 16 columns (SwiGLU pairs them in
  // registers).  Other modes keep the natural order.
  static_assert(!kGateUp || (BN % 128 == 0 && (WTN / 2) % 16 == 0), "gate_up tiles pair 64-row blocks");
  static_assert(MODE != MODE_GATEUP_F32 || BN % 128 == 0, "gate_up tiles pair 64-row blocks");
  auto brow = [&](int fn) -> int {
    if constexpr (kGateUp) {
      const int ic = wn * (WTN / 2) + (fn % (FN / 2)) * 16;
      return (ic / 64) * 128 + (fn / (FN / 2)) * 64 + ic % 64;
    } else {
      return wn * WTN + fn * 16;
    }
  };
  int frag_lane[BK / 32];
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) frag_lane[kk] = lds_off(lane & 15, kk * 4 + (lane >> 4));
  // codes in LDS: the lane's 8 codes (K offset kk * 32 + (lane / 16) * 8) of its fragment row
  int raw_lane[BK / 32];
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk)
    raw_lane[kk] = (lane & 15) * (BK / 2) + (((kk * 2 + ((lane >> 5) & 1)) ^ ((lane >> 2) & 3)) << 3) +
                   ((lane >> 4) & 1) * 4;
  // bf16 view of the B buffers for the expand (one buffer over both halves with codes)
  auto bx = [&](int buf) -> uint16_t * { return kW8Raw ? &Bs[0][0] : &Bs[buf][0]; };

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const u32x4_t *>(&As[buf][(wm * WTM + fm * 16) * BK + frag_lane[kk]]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if constexpr (kW8Raw) {
          // 8 codes -> 8 bf16, unscaled (exact; the block scale goes to acc8)
          const u32x2_t w = *reinterpret_cast<const u32x2_t *>(&Bs[buf][brow(fn) * (BK / 2) + raw_lane[kk]]);
          bfr[fn] = u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, false)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[0], 1.0f, true)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, false)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[1], 1.0f, true))};
        } else {
          bfr[fn] = *reinterpret_cast<const u32x4_t *>(&Bs[buf][brow(fn) * BK + frag_lane[kk]]);
        }
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(af[fm], bfr[fn], acc[fm][fn]);
    }
  };
  // FP8 weights, general scales: a 128-wide K block (two K steps) ends, acc8 += block
  // scale * block sum.  Fragment fn's weight rows lie in one 128-row scale block: gate_up,
  // the tile's gate block (fn < FN/2) or up block (see brow()); down, the tile's block
  // holding the fragment's rows
  auto w8_block_end = [&]() {
    if constexpr (kW8Acc) {
      const int KB = P.K / 128;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int j = kGateUp ? fn / (FN / 2) : (wn * WTN + fn * 16) / 128;
        const float sc = s_wsc[j * KB + w8_kb];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          acc8[fm][fn] += sc * acc[fm][fn];
          acc[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
      ++w8_kb;
    }
  };

  // B operand of the LoRA expand for slot a: B_lora[a][e] rows (rank columns)
  auto load_ext_b = [&](int a, u32x4_t(&xb)[B_IT]) {
    const int ra_rank = P.rank[a];
    const uint16_t *bl = P.lora_w[a];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      xb[i] = zero_u32x4();
      const int wr = b_wrow[i];
      const int j0 = b_c8[i] * 8;
      if (wr >= 0 && j0 < ra_rank) {
        const uint16_t *srcb = bl + ((size_t)(P.lora_w_shared ? 0 : e) * P.N + wr) * ra_rank + j0;
        if ((ra_rank & 7) == 0) {
          xb[i] = *reinterpret_cast<const u32x4_t *>(srcb);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (j0 + 2 * q < ra_rank) ? srcb[2 * q] : 0u;
            const uint32_t hi = (j0 + 2 * q + 1 < ra_rank) ? srcb[2 * q + 1] : 0u;
            xb[i][q] = lo | (hi << 16);
          }
        }
      }
    }
  };
  auto store_b = [&](int buf, const u32x4_t(&xb)[B_IT]) {
#pragma unroll
    for (int i = 0; i < B_IT; ++i) *reinterpret_cast<u32x4_t *>(&bx(buf)[b_lds[i]]) = xb[i];
  };
  // one 64-wide K step of the expand: A rows from Xs masked to the rows of slot a
  // (a row's ranks past its own slot's are zero in Xs, so the second 32-wide half is
  // skipped when slot a's rank is at most 32: multi-adapter gate_up 143.4 -> 141.0 us;
  // with one slot in the tile, rows of no slot are zero in Xs and need no mask)
  auto compute_ext = [&](int buf, int a, bool masked) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      if (kk > 0 && (P.rmax <= 32 || P.rank[a] <= 32)) break;
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int r = wm * WTM + fm * 16 + (lane & 15);
        af[fm] = *reinterpret_cast<const u32x4_t *>(&Xs[(wm * WTM + fm * 16) * BK + frag_lane[kk]]);
        if (masked && s_slot[r] != a) af[fm] = zero_u32x4();
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[fn] = *reinterpret_cast<const u32x4_t *>(&bx(buf)[brow(fn) * BK + frag_lane[kk]]);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(af[fm], bfr[fn], acc[fm][fn]);
    }
  };
  // Xs: every row's own-slot LoRA input, reduced over the shrink splits once per tile.
  // Only the chunks below the widest rank are loaded, one (row, chunk) per thread, with
  // the partials of up to G splits loaded together (one memory latency per group) and
  // summed in split order.
  auto build_xs = [&]() {
    // splits loaded per round trip on the taller tiles (8 at a time against 4: 1 % at
    // decode, measured when the 16-row tiles still took this path)
    constexpr int G = 8;
    const int cpr = P.rmax >> 3;  // 8-rank chunks that can hold data (rmax is a multiple of 8)
    // chunks past rmax are zero
    for (int c = tid; c < BM * (8 - cpr); c += NT) {
      const int r = c / (8 - cpr), ch = cpr + c % (8 - cpr);
      *reinterpret_cast<u32x4_t *>(&Xs[lds_off(r, ch)]) = zero_u32x4();
    }
    if (P.part_bf16) {
      for (int c = tid; c < BM * cpr; c += NT) {
        const int r = c / cpr, ch = c % cpr, j0 = ch * 8;
        const int a = s_slot[r];
        u32x4_t v4 = zero_u32x4();
        if (a >= 0 && j0 < s_rank[a])
          v4 = *reinterpret_cast<const u32x4_t *>(P.part_bf16 + (size_t)(row0 + r) * P.rmax + j0);
        *reinterpret_cast<u32x4_t *>(&Xs[lds_off(r, ch)]) = v4;
      }
      return;
    }
    if (BM <= 32 && BM * cpr * 2 <= NT) {
      // all (row, 4-rank) pieces in one pass: each thread holds one f32x4 per split, so
      // up to 16 splits load in one round trip in the registers that 8 splits of 8 ranks
      // take (the decode down expand sums 12; on taller tiles the second code path put
      // more registers in scratch)
      constexpr int G4 = 16;
      if (tid < BM * cpr * 2) {
        const int r = tid / (2 * cpr), j0 = (tid % (2 * cpr)) * 4;
        const int a = s_slot[r];
        u32x2_t v2 = {0u, 0u};
        if (a >= 0 && j0 < s_rank[a]) {
          const f32x4_t *src = reinterpret_cast<const f32x4_t *>(P.part + (size_t)(row0 + r) * P.rmax + j0);
          const size_t split_stride = (size_t)P.R * P.rmax / 4;  // in f32x4 units
          float v[4] = {0.f, 0.f, 0.f, 0.f};
          for (int sp0 = 0; sp0 < P.part_splits; sp0 += G4) {
            f32x4_t x[G4];
#pragma unroll
            for (int q = 0; q < G4; ++q) {
              x[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
              if (sp0 + q < P.part_splits) x[q] = src[(size_t)(sp0 + q) * split_stride];
            }
#pragma unroll
            for (int q = 0; q < G4; ++q)
#pragma unroll
              for (int t = 0; t < 4; ++t) v[t] += x[q][t];
          }
          const int ra_rank = s_rank[a];
          const float sc = s_scal[a];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float lo = (j0 + 2 * q < ra_rank) ? v[2 * q] * sc : 0.f;
            const float hi = (j0 + 2 * q + 1 < ra_rank) ? v[2 * q + 1] * sc : 0.f;
            v2[q] = pack_bf16x2(lo, hi);
          }
        }
        *reinterpret_cast<u32x2_t *>(&Xs[lds_off(r, j0 >> 3) + (j0 & 4)]) = v2;
      }
      return;
    }
    for (int c = tid; c < BM * cpr; c += NT) {
      const int r = c / cpr, ch = c % cpr, j0 = ch * 8;
      const int a = s_slot[r];
      u32x4_t v4 = zero_u32x4();
      // Rank and scaling come from the LDS tables (a is per lane: indexing the argument
      // block with it made the compiler copy the whole block to scratch memory in some
      // instantiations), so the partial loads wait for no other load.
      if (a >= 0 && j0 < s_rank[a]) {
        const f32x4_t *src = reinterpret_cast<const f32x4_t *>(P.part + (size_t)(row0 + r) * P.rmax + j0);
        const size_t split_stride = (size_t)P.R * P.rmax / 4;  // in f32x4 units
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int sp0 = 0; sp0 < P.part_splits; sp0 += G) {
          f32x4_t x[G][2];
#pragma unroll
          for (int q = 0; q < G; ++q) {
            x[q][0] = x[q][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (sp0 + q < P.part_splits) {
              x[q][0] = src[(size_t)(sp0 + q) * split_stride];
              x[q][1] = src[(size_t)(sp0 + q) * split_stride + 1];
            }
          }
#pragma unroll
          for (int q = 0; q < G; ++q)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[t] += x[q][0][t];
              v[4 + t] += x[q][1][t];
            }
        }
        const int ra_rank = s_rank[a];
        const float sc = s_scal[a];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = (j0 + 2 * q < ra_rank) ? v[2 * q] * sc : 0.f;
          const float hi = (j0 + 2 * q + 1 < ra_rank) ? v[2 * q + 1] * sc : 0.f;
          v4[q] = pack_bf16x2(lo, hi);
        }
      }
      *reinterpret_cast<u32x4_t *>(&Xs[lds_off(r, ch)]) = v4;
    }
  };

  // Full K steps [s_begin, s_end): PF register stages in flight, two LDS buffers, one
  // barrier per step.  The steady-state loop has no branches between a load and the use
  // of its registers.  `pre` runs once right after the first loads are issued (so its own
  // memory latency overlaps theirs); `tail_load(u)` runs at each of the last PF steps
  // before its compute, when register stage u has been stored and is free again.
  auto run_full = [&](int s_begin, int s_end, const uint16_t *bbase, int bcount, auto &&pre,
                      auto &&tail_load, auto nt, auto pk) {
    const int n = s_end - s_begin;
    const int n_main = (n / PF) * PF;
    if (n_main > 0) {
#pragma unroll
      for (int u = 0; u < PF; ++u) load_full((s_begin + u) * BK, bbase, bcount, ra[u], rb[u], nt, pk);
      pre();
      store_lds(0, ra[0], rb[0], s_begin);
      __syncthreads();
      for (int i = 0; i < n_main - PF; i += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          load_full((s_begin + i + u + PF) * BK, bbase, bcount, ra[u], rb[u], nt, pk);
          compute(u & 1);
          if (u & 1) w8_block_end();  // (FP8: the main loop starts at K step 0, PF is even)
          store_lds((u + 1) & 1, ra[(u + 1) % PF], rb[(u + 1) % PF], s_begin + i + u + 1);
          __syncthreads();
        }
      }
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        tail_load(u);
        compute(u & 1);
        if (u & 1) w8_block_end();
        if (u + 1 < PF) store_lds((u + 1) & 1, ra[u + 1], rb[u + 1], s_begin + n_main - PF + u + 1);
        __syncthreads();
      }
    } else {
      pre();
    }
    for (int s = s_begin + n_main; s < s_end; ++s) {
      load_full(s * BK, bbase, bcount, ra[0], rb[0], nt, pk);
      store_lds(0, ra[0], rb[0], s);
      __syncthreads();
      compute(0);
      if (s & 1) w8_block_end();
      __syncthreads();
    }
  };

  auto run_single = [&](auto &&loader) {
    loader(ra[0], rb[0]);
    store_lds(0, ra[0], rb[0], 0);  // (K tails: never FP8, whose K is a multiple of 128)
    __syncthreads();
    compute(0);
    __syncthreads();
  };

  if constexpr (MODE == MODE_SHRINK) {
    const int steps_total = (P.K + BK - 1) / BK;
    const int full_total = P.K / BK;
    const int groups = P.slot_groups > 1 ? P.slot_groups : 1;
    const int split = col / groups;
    const int s0 = split * P.k_steps_per_split;
    const int s1 = min(steps_total, s0 + P.k_steps_per_split);
    const int s1f = min(s1, full_total);
    // group g: chunk c of slot a's rank columns [c BN, c BN + BN), the groups enumerating
    // the slots in order with ceil(rank / BN) chunks each
    int a = 0, c = col % groups;
    while (a < P.num_slots && c >= (P.rank[a] + BN - 1) / BN) {
      c -= (P.rank[a] + BN - 1) / BN;
      ++a;
    }
    if (a < P.num_slots && ((slot_mask >> a) & 1)) {
      const int r_a = P.rank[a], c0 = c * BN;
      const int rc = min(BN, r_a - c0);  // rank rows of this chunk
      const uint16_t *bbase = P.lora_w[a] + ((size_t)(P.lora_w_shared ? 0 : e) * r_a + c0) * P.K;
      zero_acc();
      run_full(s0, s1f, bbase, rc, [] {}, [](int) {}, std::false_type{}, std::false_type{});
      if (s1 > s1f) run_single([&](u32x4_t(&xa)[A_IT], u32x4_t(&xb)[B_IT]) {
        load_tail(s1f * BK, bbase, rc, xa, xb);
      });
      // rows of this slot, the chunk's rank columns
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            const int n = wn * WTN + fn * 16 + (lane & 15);
            if (r < rows && n < rc && s_slot[r] == a)
              P.out_f32[((size_t)split * P.R + row0 + r) * P.rmax + c0 + n] = acc[fm][fn][i];
          }
    }
  } else {
    // (FP8 weights: one byte per element, the pointer only carries the byte address)
    const uint16_t *wbase =
        !kHasMain ? nullptr
        : W8 ? reinterpret_cast<const uint16_t *>(reinterpret_cast<const uint8_t *>(P.w) + (size_t)e * P.N * P.K)
             : P.w + (size_t)e * P.N * P.K;
    const int wcount = kGateUp ? 2 * P.I : P.N;
    zero_acc();
    // The expand's first batch of slots (up to PF, ascending).  When the K loop ends on a
    // full pipelined step and those ranks are multiples of 8, their B operands are loaded
    // during the last PF main steps into the register stages those steps free, from
    // clamped addresses (no predicates), and masked when stored.
    int batch0[EB];
    int pending = slot_mask;
    bool r8 = true;
#pragma unroll
    for (int u = 0; u < EB; ++u) {
      batch0[u] = -1;
      if (pending) {
        batch0[u] = __ffs(pending) - 1;
        pending &= pending - 1;
        if (P.rank[batch0[u]] & 7) r8 = false;
      }
    }
    const int full = kHasMain ? P.K / BK : 0;
    constexpr bool kExtEarly = kHasExt && kHasMain;
    const int slot1 = slot_mask ? __ffs(slot_mask) - 1 : 0;
    const bool ext_lds = kExtLds && slot_mask != 0 && (slot_mask & (slot_mask - 1)) == 0 &&
                         (P.rank[slot1] & 7) == 0 && P.rank[slot1] <= kEbRank;
    const bool ext_early = kExtEarly && !ext_lds && slot_mask != 0 && r8 && full >= PF && full % PF == 0 &&
                           full * BK == P.K;
    auto load_ext_b_clamped = [&](int a, u32x4_t(&xb)[B_IT]) {
      const int ra_rank = P.rank[a];
      const uint16_t *bl = P.lora_w[a];
      // an opaque copy of e keeps these addresses from being computed before the K loop
      // (held across it they would spill)
      int e_late = e;
      asm volatile("" : "+s"(e_late));
#pragma unroll
      for (int i = 0; i < B_IT; ++i) {
        const int wr = b_wrow[i] >= 0 ? b_wrow[i] : 0;
        const int j0 = b_c8[i] * 8 < ra_rank ? b_c8[i] * 8 : 0;
        xb[i] = *reinterpret_cast<const u32x4_t *>(
            bl + ((size_t)(P.lora_w_shared ? 0 : e_late) * P.N + wr) * ra_rank + j0);
      }
    };
    // packed row rr of the slot set bmask -> (slot, rank index, slot rank); walks the slots
    // with constant indices (the ranks stay in scalar registers, where a walk over the set
    // bits reloaded them from the argument block on every call: multi-adapter gate_up
    // 173 -> 170 us) and returns the rank, so that no caller indexes P.rank with a
    // per-lane slot (a vector load from the argument block)
    auto locate = [&](int bmask, int rr, int &a, int &j, int &rk) {
      a = -1;
      j = 0;
      rk = 0;
      int off = 0;
#pragma unroll
      for (int s = 0; s < MOE_LORA_MAX_SLOTS; ++s) {
        if (!((bmask >> s) & 1)) continue;
        const int r2 = P.rank[s];
        const int need = (r2 + 15) / 16 * 16;
        if (a < 0 && rr < off + need) {
          a = s;
          j = rr - off;
          rk = r2;
        }
        off += need;
      }
    };
    int a2_rows = 0;
    for (int m = slot_mask; m; m &= m - 1) a2_rows += (P.rank[__ffs(m) - 1] + 15) / 16 * 16;
    const bool a2_pre = kA2Pre && P.down_part != nullptr && slot_mask != 0 && a2_rows <= kA2Rows;
    // A2 rows of every slot in the tile straight into LDS, issued right after the first K
    // steps' loads; nothing waits for them before the epilogue (chunk q of the region is row q / (HC / 8), physical chunk q % (HC / 8); rows past a
    // slot's rank and columns past I read a valid element and are never used)
    auto a2_copy = [&] {
      if constexpr (kA2Pre) {
        if (!a2_pre) return;
        const int icol0 = col * HC;
        const int copies = (a2_rows * (HC / 8) + 63) / 64;
        const uint32_t base = lds_addr(A2p);
        for (int t = wave; t < copies; t += NT / 64) {
          const int q = t * 64 + lane;
          const int rr = q / (HC / 8) < a2_rows ? q / (HC / 8) : 0;
          const int c8 = ((q % (HC / 8)) ^ (rr & (HC / 8 - 1))) * 8;
          // slot of packed row rr, selected per lane over the (uniform) slot bits so that
          // the slot's pointer and rank come from scalar loads
          const uint16_t *src = nullptr;
          int rk = 1, j = 0, off = 0;
          for (int m = slot_mask; m; m &= m - 1) {
            const int s2 = __ffs(m) - 1;
            const int r2 = P.rank[s2];
            const int need = (r2 + 15) / 16 * 16;
            if (!src && rr < off + need) {
              src = P.down_a[s2];
              rk = r2;
              j = rr - off;
            }
            off += need;
          }
          j = j < rk ? j : 0;
          const int icol = icol0 + c8 < P.I ? icol0 + c8 : 0;
          lds_dma16(src + ((size_t)e * rk + j) * P.I + icol,
                    __builtin_amdgcn_readfirstlane(base + (uint32_t)t * 1024u));
        }
      }
    };
    // the single slot's B rows into Eb (LDS row n = B row of output column n of the tile,
    // physical chunk p of a row holds ranks 8 * (p ^ ((n >> 2) & 3)) ..; chunks past the
    // rank read a valid element, which meets zeros in Xs)
    auto eb_copy = [&] {
      if constexpr (kExtLds) {
        if (!ext_lds) return;
        const int rk = P.rank[slot1];
        const uint16_t *bl = P.lora_w[slot1];
        const uint32_t base = lds_addr(Eb);
        for (int t = wave; t < BN * kEbRank / 8 / 64; t += NT / 64) {
          const int n = t * 16 + (lane >> 2);
          const int c8 = ((lane & 3) ^ ((n >> 2) & 3)) * 8;
          int wr;
          if (kGateUp) {
            const int icol = col * (BN / 2) + (n / 128) * 64 + n % 64;  // see brow()
            wr = icol < P.I ? ((n % 128) / 64) * P.I + icol : 0;
          } else {
            const int ng = col * BN + n;
            wr = ng < P.N ? ng : 0;
          }
          lds_dma16(bl + ((size_t)(P.lora_w_shared ? 0 : e) * P.N + wr) * rk + (c8 < rk ? c8 : 0),
                    __builtin_amdgcn_readfirstlane(base + (uint32_t)t * 1024u));
        }
      }
    };
    auto build = [&] {
      eb_copy();
      a2_copy();
      if (kHasExt && slot_mask) build_xs();  // visible after the main loop's first barrier
    };
    auto main_loop = [&](auto nt, auto pk) {
      if (kExtEarly && ext_early) {
        run_full(0, full, wbase, wcount, build, [&](int u) {
          if (u < EB) load_ext_b_clamped(batch0[u] >= 0 ? batch0[u] : batch0[0], rb[u]);
        }, nt, pk);
      } else {
        run_full(0, full, wbase, wcount, build, [](int) {}, nt, pk);
        if (full * BK < P.K) run_single([&](u32x4_t(&xa)[A_IT], u32x4_t(&xb)[B_IT]) {
          load_tail(full * BK, wbase, wcount, xa, xb);
        });
      }
    };
    // the packed layout needs whole 128-row blocks and 64-wide K steps (checked by the host)
    auto main_loop_pk = [&](auto nt) {
      if constexpr (BN % 128 == 0) {
        if (P.w_packed) {
          main_loop(nt, std::true_type{});
          return;
        }
      }
      main_loop(nt, std::false_type{});
    };
    if constexpr (kW8Acc) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc8[fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      w8_kb = 0;
    }
    if (kHasMain) {
      if constexpr (kStreamB) {
        if (single_mtile)
          main_loop_pk(std::true_type{});
        else
          main_loop_pk(std::false_type{});
      } else {
        main_loop_pk(std::false_type{});
      }
    } else {
      build();
    }
    if constexpr (kW8Acc) {
      // (K is a multiple of 128 with FP8 weights: the last block was scaled in)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = acc8[fm][fn];
    }
    if (kExtLds && ext_lds) {
      // one K step over ranks 0-31: A fragments from Xs (rows of other slots or none are
      // zero there), B fragments from Eb
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's B copies landed
      __syncthreads();
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const u32x4_t *>(&Xs[(wm * WTM + fm * 16) * BK + frag_lane[0]]);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = brow(fn) + (lane & 15);
        bfr[fn] = *reinterpret_cast<const u32x4_t *>(&Eb[n * kEbRank + (((lane >> 4) ^ ((n >> 2) & 3)) << 3)]);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_16x16x32(af[fm], bfr[fn], acc[fm][fn]);
    } else if (kHasExt && slot_mask) {
      // B operands of up to PF slots loaded at once into the (now idle) register stages,
      // then one masked K step per slot with A fragments read from Xs
      pending = slot_mask;
      bool first = true;
      while (pending) {
        int batch[EB];
#pragma unroll
        for (int u = 0; u < EB; ++u) {
          batch[u] = -1;
          if (pending) {
            batch[u] = __ffs(pending) - 1;
            pending &= pending - 1;
          }
        }
        if (first && ext_early) {
          // already in rb[]: zero the chunks outside B's rows and the slot's rank
#pragma unroll
          for (int u = 0; u < EB; ++u) {
            if (batch[u] < 0) continue;
            const int ra_rank = P.rank[batch[u]];
#pragma unroll
            for (int i = 0; i < B_IT; ++i)
              if (!(b_wrow[i] >= 0 && b_c8[i] * 8 < ra_rank)) rb[u][i] = zero_u32x4();
          }
        } else {
#pragma unroll
          for (int u = 0; u < EB; ++u)
            if (batch[u] >= 0) load_ext_b(batch[u], rb[u]);
        }
        first = false;
#pragma unroll
        for (int u = 0; u < EB; ++u) {
          if (batch[u] < 0) continue;
          store_b(u & 1, rb[u]);
          __syncthreads();
          compute_ext(u & 1, batch[u], (slot_mask & (slot_mask - 1)) != 0);
          __syncthreads();
        }
      }
    }

    if constexpr (kGateUp) {
      // SwiGLU in registers; the bf16 activation tile goes to LDS (pitch HP), from where it
      // is written out in 16-byte row chunks (the fragment layout would give 2-byte
      // stores) and, with the fused down shrink, contracted with A2 for the tile's share
      // of v = A2 . act.
      static_assert(BM * HP + 64 * HP <= kBsElems, "activation tile and one A2 slice must fit LDS");
      uint16_t *Hs = reinterpret_cast<uint16_t *>(Bs);  // both B buffers are free now: [Hs | A2s]
      uint16_t *A2s = Hs + BM * HP;
      const bool fuse_down = P.down_part != nullptr && slot_mask != 0;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fh = 0; fh < FN / 2; ++fh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            const int c = wn * (WTN / 2) + fh * 16 + (lane & 15);
            const float g = acc[fm][fh][i];
            const float u = acc[fm][fh + FN / 2][i];
            Hs[r * HP + c] = col * HC + c < P.I ? (uint16_t)f32_to_bf16(silu_mul(g, u)) : (uint16_t)0;
          }
      if (a2_pre) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's A2 copies landed
      __syncthreads();
      for (int q = tid; q < BM * (HC / 8); q += NT) {
        const int r = q / (HC / 8), c8 = (q % (HC / 8)) * 8;
        const int icol = col * HC + c8;  // I is a multiple of 8: a chunk is all in or all out
        if (r < rows && icol < P.I)
          *reinterpret_cast<u32x4_t *>(P.out_bf16 + (size_t)(row0 + r) * P.I + icol) =
              *reinterpret_cast<const u32x4_t *>(&Hs[r * HP + c8]);
      }
      // v partials of one batch of slots (set bmask, packed rows in a2src): (row fragment,
      // packed rank fragment) tasks over the waves.  Each row's own-slot values go to Vs
      // (fp32 [BM][64] in the A buffers, free after the K loop; 16-column groups XOR-ed
      // by row / 4), written out once per tile in 16-byte row chunks of the row's own
      // rank (an eighth of the store instructions of 4-byte fragment stores; the time
      // the contraction took was its argument-block loads, see locate()).
      float *Vs = reinterpret_cast<float *>(&As[0][0]);
      static_assert(BM * MOE_LORA_MAX_RANK * 4 <= (int)sizeof(As), "v tile must fit the A buffers");
      auto contract = [&](int bmask, int rows_used, const uint16_t *a2src, bool swizzled) {
        const int nrf = rows_used / 16;
        for (int f = wave; f < (BM / 16) * nrf; f += NT / 64) {
          const int mf = f / nrf, rf = f % nrf;
          int a, j16, rk;
          locate(bmask, rf * 16, a, j16, rk);  // first rank index of this fragment
          f32x4_t v4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < HC / 32; ++kk) {
            const u32x4_t ha = *reinterpret_cast<const u32x4_t *>(
                &Hs[(mf * 16 + (lane & 15)) * HP + kk * 32 + (lane >> 4) * 8]);
            const int ar = rf * 16 + (lane & 15), ac = kk * 4 + (lane >> 4);
            const u32x4_t hb2 = *reinterpret_cast<const u32x4_t *>(
                &a2src[swizzled ? ar * HC + ((ac ^ (ar & (HC / 8 - 1))) << 3) : ar * HP + ac * 8]);
            v4 = mfma_16x16x32(ha, hb2, v4);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mf * 16 + (lane >> 4) * 4 + i;
            const int j = j16 + (lane & 15);
            if (r < rows && j < rk && s_slot[r] == a)
              Vs[r * MOE_LORA_MAX_RANK + (j ^ (((r >> 2) & 3) << 4))] = v4[i];
          }
        }
      };
      if (a2_pre) {
        contract(slot_mask, a2_rows, A2p, true);  // A2 copied in with the first K steps
      } else if (fuse_down) {
        // slots whose A2 rows did not fit the prefetch region: A2 slices packed into A2s,
        // as many slots per batch as fit, one barrier pair per batch
        constexpr int kCapRows = ((kBsElems - BM * HP) / HP) / 16 * 16;
        static_assert(kCapRows >= MOE_LORA_MAX_RANK, "one slot's A2 rows must fit a batch");
        const int icol0 = col * HC;
        int pending = slot_mask;
        while (pending) {
          int bmask = 0, rows_used = 0;
          while (pending) {
            const int a = __ffs(pending) - 1;
            const int need = (P.rank[a] + 15) / 16 * 16;
            if (rows_used + need > kCapRows && bmask != 0) break;
            bmask |= 1 << a;
            rows_used += need;
            pending &= pending - 1;
          }
          __syncthreads();  // previous batch's reads of A2s done
          for (int q = tid; q < rows_used * (HC / 8); q += NT) {
            const int rr = q / (HC / 8), c8 = (q % (HC / 8)) * 8;
            // slot of packed row rr selected over the uniform slot bits (pointer and rank
            // from scalar loads)
            const uint16_t *src = nullptr;
            int rk = 0, j = 0, off = 0;
            for (int m = bmask; m; m &= m - 1) {
              const int s2 = __ffs(m) - 1;
              const int r2 = P.rank[s2];
              const int need = (r2 + 15) / 16 * 16;
              if (!src && rr < off + need) {
                src = P.down_a[s2];
                rk = r2;
                j = rr - off;
              }
              off += need;
            }
            u32x4_t v = zero_u32x4();
            if (src && j < rk && icol0 + c8 < P.I)
              v = *reinterpret_cast<const u32x4_t *>(src + ((size_t)e * rk + j) * P.I + icol0 + c8);
            *reinterpret_cast<u32x4_t *>(&A2s[rr * HP + c8]) = v;
          }
          __syncthreads();
          contract(bmask, rows_used, A2s, false);
        }
      }
      if (fuse_down) {
        __syncthreads();
        // chunks of 4 ranks below the row's own rank (rmax is a multiple of 8)
        for (int q = tid; q < BM * (P.rmax / 4); q += NT) {
          const int r = q / (P.rmax / 4), j = (q % (P.rmax / 4)) * 4;
          const int a = r < rows ? s_slot[r] : -1;
          const int rk = a >= 0 ? s_rank[a] : 0;
          if (j < rk)
            *reinterpret_cast<f32x4_t *>(P.down_part + ((size_t)col * P.R + row0 + r) * P.rmax + j) =
                *reinterpret_cast<const f32x4_t *>(&Vs[r * MOE_LORA_MAX_RANK + (j ^ (((r >> 2) & 3) << 4))]);
        }
      }
    } else if constexpr (MODE == MODE_DOWN) {
      // bf16 output tile through LDS for 16-byte row-chunk stores.  Rows are BN elements
      // apart with the 16-column groups XOR-ed by (row / 4) % 4, so that the four row
      // groups of a fragment store land in different banks without padding, and the whole
      // tile fits the B buffers at once (the padded 128x256 tile went in two halves, one
      // barrier pair each)
      constexpr int OP = BN;
      constexpr int RH = (BM * OP <= kBsElems) ? BM : BM / 2;
      static_assert(RH * OP <= kBsElems && RH % WTM == 0, "output rows must fit the B buffers");
      static_assert(BN % 64 == 0, "the column swizzle permutes 16-column groups within 64");
      uint16_t *Os = reinterpret_cast<uint16_t *>(Bs);
      auto os_col = [](int r, int c) { return c ^ (((r >> 2) & 3) << 4); };
#pragma unroll
      for (int h = 0; h < BM / RH; ++h) {
        if (h) __syncthreads();  // the previous half has been read
        if ((wm * WTM) / RH == h) {
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = wm * WTM - h * RH + fm * 16 + (lane >> 4) * 4 + i;
                const int c = wn * WTN + fn * 16 + (lane & 15);
                Os[r * OP + os_col(r, c)] = (uint16_t)f32_to_bf16(acc[fm][fn][i]);
              }
        }
        __syncthreads();
        for (int q = tid; q < RH * (BN / 8); q += NT) {
          const int r = q / (BN / 8), c8 = (q % (BN / 8)) * 8;
          const int n = col * BN + c8;  // N is a multiple of 8: a chunk is all in or all out
          if (h * RH + r < rows && n < P.N)
            *reinterpret_cast<u32x4_t *>(P.out_bf16 + (size_t)(row0 + h * RH + r) * P.N + n) =
                *reinterpret_cast<const u32x4_t *>(&Os[r * OP + os_col(r, c8)]);
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
            int n = col * BN + wn * WTN + fn * 16 + (lane & 15);
            if constexpr (MODE == MODE_GATEUP_F32) {  // LDS row -> gate/up column
              const int nl = wn * WTN + fn * 16 + (lane & 15);
              const int icol = col * (BN / 2) + (nl / 128) * 64 + nl % 64;
              n = icol < P.I ? ((nl % 128) / 64) * P.I + icol : P.N;
            }
            if (r < rows && n < P.N) P.out_f32[(size_t)(row0 + r) * P.N + n] = acc[fm][fn][i];
          }
    }
  }
  // the next tile's slot mask starts empty (its previous reads ended a tile ago); LDS is
  // reused from here
  if constexpr (!kPersistent) break;
  if (tid == 0) s_mask[parity ^ 1] = 0;
  __syncthreads();
  }  // tile loop
}

// ---------------------------------------------------------------- host side
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int mtile_bound(int R, int E, int BM) {
  const long long nonempty = R < E ? R : E;
  return (int)((R + nonempty * (BM - 1) + BM - 1) / BM);
}

// Tile height from the mean rows per expert (the routed load is only known on device).
// Above 8 rows the 64-row tile keeps most experts in one m-tile, so each weight row is
// streamed from HBM once (16-row tiles re-read the weights of every expert with more
// rows: 1.2x slower at 16 rows per expert, 1.7x on a DeepSeek-V3-sized layer; the GEMMs
// of batches up to 16 rows per expert then run 32-row tiles, see launch_forward).
int pick_bm(int R, int E) {
  const int avg = R / (E > 0 ? E : 1);
  if (avg <= 8) return 16;
  if (avg <= 128) return 64;
  return 128;
}

int shrink_bm(int R, int E) {
  const int avg = R / (E > 0 ? E : 1);
  return avg <= 16 ? 16 : (avg <= 48 ? 32 : 128);
}

// Split K so that the grid has ~512 workgroups, each with at least 4 pipelined K steps
// (against ~1024: multi-adapter T=256 shrink 18.1 -> 15.7 us per launch, DeepSeek-V3-sized
// 27.9 -> 26.0 us, decode even; ~256 was slower at decode and DeepSeek-V3 sizes).
// Each (m-tile, split) gets one block per rank-column chunk of each adapter slot (the
// groups of shrink_groups), so the slots' passes over K run side by side instead of one
// after another in a block.
int shrink_splits(int R, int E, int K, int groups, int &steps_per_split) {
  const int steps = cdiv(K, BK);
  const int tiles = mtile_bound(R, E, shrink_bm(R, E)) * (groups > 1 ? groups : 1);
  int want = cdiv(512, tiles > 0 ? tiles : 1);
  if (want < 1) want = 1;
  steps_per_split = cdiv(steps, want);
  if (steps_per_split < 4) steps_per_split = steps < 4 ? steps : 4;
  return cdiv(steps, steps_per_split);
}

// Rank columns per LoRA shrink tile: 32 on the 16- and 32-row tiles (a slot of higher rank
// takes several column chunks, each its own block), and on the 128-row tiles when every
// rank fits them; else 64
int shrink_bn(int bm, int rmax) { return (bm <= 32 || rmax <= 32) ? 32 : 64; }

// blocks per (m-tile, K split) of the LoRA shrink: one per shrink_bn-wide chunk of each slot
int shrink_groups(const int *rank, int num_slots, int bn) {
  int g = 0;
  for (int s = 0; s < num_slots; ++s) g += (rank[s] + bn - 1) / bn;
  return g > 0 ? g : 1;
}

int rmax8(const moe_lora_adapters *lora) {
  int r = 0;
  for (int s = 0; s < lora->num_slots; ++s) r = lora->rank[s] > r ? lora->rank[s] : r;
  return (r + 7) & ~7;
}

// compute units of the current device (cached per device)
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

template <int BM, int BN, int WM, int WN, int MODE, int PF, int W8 = 0>
int launch_cfg(const GemmParams &P, int n_cols, hipStream_t s) {
  auto kernel = moe_gemm_kernel<BM, BN, WM, WN, MODE, PF, W8>;
  constexpr int threads = WM * WN * 64;
  int tiles = mtile_bound(P.R, P.E, BM);
  long long blocks = (long long)tiles * n_cols;
  blocks = (blocks + 7) & ~7ll;  // the kernels assume a multiple of 8 (one share per XCD)
  if (blocks == 0) return ST_OK;
  if (BM >= 64) {  // persistent blocks: as many as can be resident at once
    static int occ = 0;
    if (occ == 0) {
      int o = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, reinterpret_cast<const void *>(kernel), threads, 0) !=
              hipSuccess || o < 1)
        o = 1;
      occ = o;
    }
    long long resident = ((long long)device_cus() * occ) & ~7ll;
    if (resident < 8) resident = 8;
    if (blocks > resident) blocks = resident;
  }
  GemmParams Q = P;
  Q.n_cols = n_cols;
  kernel<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(Q);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

// n-tiles of the gate_up GEMM (each covers BN/2 intermediate columns)
int gateup_ncols(int bm, int I) { return bm >= 128 ? cdiv(I, 128) : cdiv(I, 64); }

template <int MODE, int W8 = 0>
int launch_gemm(const GemmParams &P, int bm, hipStream_t s) {
  const int BN = 128;
  const int ncols = (MODE == MODE_GATEUP) ? cdiv(P.I, BN / 2) : cdiv(P.N, BN);
  switch (bm) {
    // Register stages of the 16-row tiles: two where three waves share a SIMD (see the
    // kernel's register budget), four on the bf16 gate_up (FP8 gate_up at two waves: four,
    // six and eight stages measured 76, 82 and 80 us)
    case 16:
      if constexpr (W8) return launch_cfg<16, 128, 1, 4, MODE, 2, W8>(P, ncols, s);
      else return launch_cfg<16, 128, 1, 4, MODE, MODE == MODE_DOWN ? 2 : 4>(P, ncols, s);
    case 32: return launch_cfg<32, 128, 2, 2, MODE, 2, W8>(P, ncols, s);
    case 64: return launch_cfg<64, 128, 2, 2, MODE, 2, W8>(P, ncols, s);
    default: return launch_cfg<128, 256, 4, 2, MODE, 2, W8>(P, (MODE == MODE_GATEUP) ? cdiv(P.I, 128) : cdiv(P.N, 256), s);
  }
}

int launch_shrink(const GemmParams &P0, int bm, int splits, hipStream_t s) {
  GemmParams P = P0;
  const int bn = shrink_bn(bm, P.rmax);
  P.slot_groups = shrink_groups(P.rank, P.num_slots, bn);
  const int cols = splits * P.slot_groups;
  // 32 rank columns per block: a 64-wide tile spent most of its B loads on clamped rows
  // past small ranks (decode -0.6 %, prefill -0.4 %), and on the short tiles it stages
  // twice the LDS bytes per K step for the same rows, where the LDS-staged K step (not the
  // loads) bounds the launch; 128-row tiles keep 64 columns for ranks above 32
  if (bm <= 16) return launch_cfg<16, 32, 1, 2, MODE_SHRINK, 2>(P, cols, s);
  if (bm <= 32) return launch_cfg<32, 32, 2, 1, MODE_SHRINK, 2>(P, cols, s);
  if (bn == 32) return launch_cfg<128, 32, 4, 1, MODE_SHRINK, 2>(P, cols, s);
  return launch_cfg<128, 64, 2, 2, MODE_SHRINK, 2>(P, cols, s);
}

// Activation of the decomposed path: act = silu(G_gate + D_gate) * (G_up + D_up), the
// gate_up LoRA delta D joined right before SwiGLU (bf16 PR, Files-changed table,
// activation row: the delta is added before SwiGLU; the activation output feeds the
// down LoRA).  G and D are fp32 [R, 2I] with rows [gate | up]; one thread per 4 columns.
// Split partials of the fused down shrink reduced once per step for the down GEMM's
// expand: out[p][j] = bf16(s_a * sum over splits of part[split][p][j]) for j below the
// rank of row p's slot, zero elsewhere; the splits are summed in ascending order, as the
// down GEMM sums them itself when it reads the partials directly (so both give the same
// bits).  One thread per (row, 8-rank chunk).
struct SlotRanks {
  int rank[MOE_LORA_MAX_SLOTS];
  float scaling[MOE_LORA_MAX_SLOTS];
};

__global__ __launch_bounds__(256) void reduce_part_kernel(const float *__restrict__ part, int splits, int R,
                                                          int rmax, const int32_t *__restrict__ row_slot,
                                                          const SlotRanks sr, uint16_t *__restrict__ out) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int cpr = rmax / 8;
  if (q >= (long long)R * cpr) return;
  const int p = (int)(q / cpr), j0 = (int)(q % cpr) * 8;
  const int a = row_slot[p];
  int rk = 0;
  float sc = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < MOE_LORA_MAX_SLOTS; ++s2)
    if (a == s2) {
      rk = sr.rank[s2];
      sc = sr.scaling[s2];
    }
  u32x4_t v4 = zero_u32x4();
  if (j0 < rk) {
    const f32x4_t *src = reinterpret_cast<const f32x4_t *>(part + (size_t)p * rmax + j0);
    const size_t stride = (size_t)R * rmax / 4;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) {
      const f32x4_t x0 = src[(size_t)sp * stride], x1 = src[(size_t)sp * stride + 1];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] += x0[t];
        v[4 + t] += x1[t];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = (j0 + 2 * c < rk) ? v[2 * c] * sc : 0.f;
      const float hi = (j0 + 2 * c + 1 < rk) ? v[2 * c + 1] * sc : 0.f;
      v4[c] = pack_bf16x2(lo, hi);
    }
  }
  *reinterpret_cast<u32x4_t *>(out + (size_t)p * rmax + j0) = v4;
}

__global__ __launch_bounds__(256) void swiglu_join_kernel(const float *__restrict__ G,
                                                          const float *__restrict__ D,
                                                          uint16_t *__restrict__ act, int R, int I) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = I / 4;
  if (q >= (long long)R * per_row) return;
  const int p = (int)(q / per_row), i = (int)(q % per_row) * 4;
  const float *gr = G + (size_t)p * 2 * I, *dr = D + (size_t)p * 2 * I;
  const f32x4_t g = *reinterpret_cast<const f32x4_t *>(gr + i);
  const f32x4_t u = *reinterpret_cast<const f32x4_t *>(gr + I + i);
  const f32x4_t dg = *reinterpret_cast<const f32x4_t *>(dr + i);
  const f32x4_t du = *reinterpret_cast<const f32x4_t *>(dr + I + i);
  float h[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float gg = g[c] + dg[c], uu = u[c] + du[c];
    h[c] = silu_mul(gg, uu);
  }
  uint2 o;
  o.x = pack_bf16x2(h[0], h[1]);
  o.y = pack_bf16x2(h[2], h[3]);
  *reinterpret_cast<uint2 *>(act + (size_t)p * I + i) = o;
}

// Library-owned fork/join events, created once per device and reused.  They order two
// streams of one device, so they skip the system-scope fence (the release that makes device
// memory visible to the host), which idles the GPU for microseconds at every record.
struct StreamEvents {
  hipEvent_t fork = nullptr, ready = nullptr;
};

int get_events(StreamEvents *&out) {
  static StreamEvents ev[64];
  static int created[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ST_HIP;
  if (!created[dev]) {
    constexpr unsigned kFlags = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&ev[dev].fork, kFlags) != hipSuccess ||
        hipEventCreateWithFlags(&ev[dev].ready, kFlags) != hipSuccess)
      return ST_HIP;
    created[dev] = 1;
  }
  out = &ev[dev];
  return ST_OK;
}

constexpr int kTwoStreamMaxT = 256;  // decomposed-path buffers exist up to this many tokens

struct FwdLayout {
  size_t u_part = 0, act = 0, v_part = 0, v_red = 0, g = 0, dlt = 0, row_slot = 0, total = 0;
  int splits1 = 0, steps1 = 0, splits2 = 0, shrink2_splits = 0, steps2 = 0, rmax = 0;
  bool decomposed = false;
};

// A down expand whose partials come in more than four splits, and whose n-tiles would
// re-read at least kReduceMinBytes of them in all, is fed by one reduction per step
// instead (prefill T=8192: 6 splits, 192 MB of re-reads, step -1.1 %; multi-adapter
// T=256: 12 and 100 MB, -1.1 %; DeepSeek-V3-sized: 32 and 1.9 GB, -1.9 %).  Below that
// the extra launch costs more than it saves (decode T=64: 6 MB, +1.3 %).
constexpr int kReduceMinSplits = 4;
constexpr long long kReduceMinBytes = 32ll << 20;

// fused_only: no room for the decomposed path's fp32 G / delta buffers
FwdLayout layout(const moe_lora_dims &d, const moe_lora_adapters *lora, bool fused_only = false) {
  FwdLayout L;
  const size_t R = (size_t)d.num_tokens * d.top_k;
  const bool has_lora = lora && lora->num_slots > 0;
  size_t off = 0;
  if (has_lora) {
    L.rmax = rmax8(lora);
    const int groups = shrink_groups(lora->rank, lora->num_slots, shrink_bn(shrink_bm((int)R, d.num_experts), L.rmax));
    L.splits1 = shrink_splits((int)R, d.num_experts, d.hidden, groups, L.steps1);
    L.shrink2_splits = shrink_splits((int)R, d.num_experts, d.inter, groups, L.steps2);
    // the fused path writes one down-shrink partial per gate_up n-tile (64 or 128 I columns)
    L.splits2 = L.shrink2_splits > cdiv(d.inter, 64) ? L.shrink2_splits : cdiv(d.inter, 64);
    L.u_part = off;
    off = align256(off + (size_t)L.splits1 * R * L.rmax * sizeof(float));
  }
  L.act = off;
  off = align256(off + R * d.inter * sizeof(uint16_t));
  if (has_lora) {
    L.v_part = off;
    off = align256(off + (size_t)L.splits2 * R * L.rmax * sizeof(float));
    L.row_slot = off;
    off = align256(off + R * sizeof(int32_t));
    L.v_red = off;
    off = align256(off + R * L.rmax * sizeof(uint16_t));
  }
  if (!fused_only && has_lora && d.num_tokens <= kTwoStreamMaxT && (d.inter % 4) == 0) {
    L.decomposed = true;
    L.g = off;
    off = align256(off + R * 2 * d.inter * sizeof(float));
    L.dlt = off;
    off = align256(off + R * 2 * d.inter * sizeof(float));
  }
  L.total = off;
  return L;
}

}  // namespace

size_t forward_workspace_size(const moe_lora_dims &d, const moe_lora_adapters *lora, bool fused_only) {
  return layout(d, lora, fused_only).total;
}

int launch_forward(const moe_lora_dims &d, const uint16_t *x, const uint16_t *x_perm,
                   const int32_t *offsets, const int32_t *p2e, const uint16_t *w1,
                   const uint16_t *w2, const moe_lora_adapters *lora, uint16_t *y_perm, void *ws,
                   size_t ws_bytes, hipStream_t main, hipStream_t side,
                   const moe_lora_options *opts, const float *w1_scale, const float *w2_scale,
                   bool fused_only) {
  const int R = d.num_tokens * d.top_k;
  // FP8 weights (w1/w2 hold E4M3 codes, block scales given): fused path only
  const bool fp8 = w1_scale != nullptr;
  const bool pow2 = fp8 && opts && opts->fp8_pow2_scales;  // power-of-two block scales
  if (R == 0) return ST_OK;
  const FwdLayout L = layout(d, lora, fused_only);
  if (ws_bytes < L.total) return ST_WS_SMALL;
  char *wsb = static_cast<char *>(ws);
  const bool has_lora = lora && lora->num_slots > 0;
  uint16_t *act = reinterpret_cast<uint16_t *>(wsb + L.act);
  float *u_part = has_lora ? reinterpret_cast<float *>(wsb + L.u_part) : nullptr;
  float *v_part = has_lora ? reinterpret_cast<float *>(wsb + L.v_part) : nullptr;
  int32_t *row_slot = has_lora ? reinterpret_cast<int32_t *>(wsb + L.row_slot) : nullptr;

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
  // Batches with up to 16 rows per expert on average run both GEMMs on 32-row tiles (one
  // tile per block, three blocks per CU; an expert rarely has more than 32 rows, so its
  // weights are still read once), where the 64-row tile was three quarters padding; the
  // down-LoRA shrink stays a launch of its own, as for 64-row tiles.  Multi-adapter T=256:
  // gate_up 143.5 -> 130.9 us with LoRA, 129.4 -> 123.0 us without; down 90.8 -> 85.7 us
  // and 74.9 -> 72.6 us.  The decomposed path's fp32 gate_up and LoRA expand take the same
  // tiles (its two-stream step 303 -> 287 us).
  const int bm_gemm = (bm == 64 && R <= 16 * d.num_experts) ? 32 : bm;
  int st;

  hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->gate_up_event_begin) : nullptr;
  hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->gate_up_event_end) : nullptr;
  const int force = opts ? opts->force_path : 0;
  const int packed = opts ? opts->packed_weights : 0;  // bit 0 W1, bit 1 W2 (validated by the API)
  int two_max = (opts && opts->two_stream_max_tokens > 0) ? opts->two_stream_max_tokens : kTwoStreamMaxT;
  if (two_max > kTwoStreamMaxT) two_max = kTwoStreamMaxT;
  // (FP8 weights run the fused path only and leave a side stream unused; a forced
  // decomposed path was rejected by the API)
  const bool decomposed = !fp8 && has_lora && L.decomposed &&
                          (force == 2 || (force == 0 && side && d.num_tokens <= two_max));
  if (force == 2 && has_lora && !L.decomposed) return ST_UNSUPPORTED;
  // the side stream is used only by the decomposed path
  hipStream_t lora_stream = (decomposed && side) ? side : main;
  // The down-LoRA shrink v = A2 . act: contracted in the gate_up epilogue (partials per
  // n-tile) for 16- and 128-row tiles, a separate split-K shrink launch over act for 64-row
  // tiles, whose epilogue contraction cost more than the launch (multi-adapter T=256: step
  // 319 -> 312 us, gate_up 166 -> 145 us; DeepSeek-V3-sized: 3.23 -> 3.18 ms; decode T=64
  // +2 us and prefill even with the launch), and always on the decomposed path.
  const bool sep_down_shrink = decomposed || (has_lora && bm == 64);

  GemmParams shrink1 = base;
  if (has_lora) {  // gate_up LoRA shrink: u_part = A1 . x  (split over H)
    shrink1.a = a_src;
    shrink1.a_gather = a_gather;
    shrink1.K = d.hidden;
    shrink1.N = 0;
    shrink1.k_steps_per_split = L.steps1;
    for (int s = 0; s < lora->num_slots; ++s) shrink1.lora_w[s] = lora->a_gate_up[s];
    shrink1.lora_w_shared = lora->shared_outer;  // shared-outer: one A1 for all experts
    shrink1.out_f32 = u_part;
    shrink1.row_slot_out = row_slot;
  }
  GemmParams gu = base;  // gate_up GEMM
  gu.a = a_src;
  gu.a_gather = a_gather;
  gu.w = w1;
  gu.K = d.hidden;
  gu.N = 2 * d.inter;
  gu.w_packed = packed & 1;
  gu.w_scale = w1_scale;
  // Tile order, per GEMM and tile height, as measured (HBM reads from FETCH_SIZE): m-tile
  // first on the 64-row gate_up tiles (DeepSeek-V3-sized: 13.9 -> 12.3 GB read, 1.92 ->
  // 1.86 ms; multi-adapter even) and the 128-row down tiles (prefill: 0.91 -> 0.73 GB,
  // 380 -> 363 us); column first elsewhere (the 64-row down tiles read 0.9 GB less but took
  // 1.10 -> 1.15 ms; 128-row gate_up 568 -> 575 us)
  gu.mt_fast = (bm_gemm == 64);

  if (!decomposed) {
    // fused: shrink, then the GEMM appends the LoRA expand as extra K steps and applies
    // SwiGLU in its epilogue
    if (has_lora) {
      if ((st = launch_shrink(shrink1, shrink_bm(R, d.num_experts), L.splits1, main)) != ST_OK) return st;
      for (int s = 0; s < lora->num_slots; ++s) gu.lora_w[s] = lora->b_gate_up[s];
      gu.part = u_part;
      gu.part_splits = L.splits1;
      gu.row_slot = row_slot;
    }
    gu.out_bf16 = act;
    if (has_lora && !sep_down_shrink) {  // the down-LoRA shrink rides in the epilogue (partials per I tile)
      for (int s = 0; s < lora->num_slots; ++s) gu.down_a[s] = lora->a_down[s];
      gu.down_part = v_part;
    }
    if (ev0 && hipEventRecord(ev0, main) != hipSuccess) return ST_HIP;
    if ((st = fp8 ? (pow2 ? launch_gemm<MODE_GATEUP, 2>(gu, bm_gemm, main) : launch_gemm<MODE_GATEUP, 1>(gu, bm_gemm, main)) : launch_gemm<MODE_GATEUP>(gu, bm_gemm, main)) !=
        ST_OK)
      return st;
    if (ev1 && hipEventRecord(ev1, main) != hipSuccess) return ST_HIP;
  } else {
    // decomposed: the LoRA shrink and expand (delta D) run on the side stream while main
    // runs the base gate_up GEMM (G); main joins on lora_ready right before the activation,
    // the delta's only consumer (bf16 PR, two-stream flow).
    float *Gb = reinterpret_cast<float *>(wsb + L.g);
    float *Db = reinterpret_cast<float *>(wsb + L.dlt);
    StreamEvents *sev = nullptr;
    if (lora_stream != main) {
      if ((st = get_events(sev)) != ST_OK) return st;
      if (hipEventRecord(sev->fork, main) != hipSuccess) return ST_HIP;
      if (hipStreamWaitEvent(lora_stream, sev->fork, 0) != hipSuccess) return ST_HIP;
    }
    if ((st = launch_shrink(shrink1, shrink_bm(R, d.num_experts), L.splits1, lora_stream)) != ST_OK)
      return st;
    GemmParams ex = base;  // expand: D = s * B1 . bf16(sum u_part), fp32
    ex.N = 2 * d.inter;
    ex.K = 0;
    for (int s = 0; s < lora->num_slots; ++s) ex.lora_w[s] = lora->b_gate_up[s];
    ex.part = u_part;
    ex.part_splits = L.splits1;
    ex.row_slot = row_slot;
    ex.out_f32 = Db;
    if ((st = launch_gemm<MODE_EXPAND_F32>(ex, bm_gemm, lora_stream)) != ST_OK) return st;
    if (lora_stream != main && hipEventRecord(sev->ready, lora_stream) != hipSuccess) return ST_HIP;

    gu.out_f32 = Gb;
    if (ev0 && hipEventRecord(ev0, main) != hipSuccess) return ST_HIP;
    if ((st = launch_gemm<MODE_GATEUP_F32>(gu, bm_gemm, main)) != ST_OK) return st;
    if (ev1 && hipEventRecord(ev1, main) != hipSuccess) return ST_HIP;
    if (lora_stream != main && hipStreamWaitEvent(main, sev->ready, 0) != hipSuccess) return ST_HIP;
    const long long nthr = (long long)R * (d.inter / 4);
    swiglu_join_kernel<<<dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, main>>>(Gb, Db, act, R,
                                                                                    d.inter);
    if (hipGetLastError() != hipSuccess) return ST_HIP;
  }
  // 3) down LoRA shrink: v_part = A2 . act  (split over I); fused into the gate_up
  //    epilogue on the fused path
  if (has_lora && sep_down_shrink) {
    GemmParams P = base;
    P.a = act;
    P.a_gather = 0;
    P.K = d.inter;
    P.N = 0;
    P.k_steps_per_split = L.steps2;
    for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->a_down[s];
    P.out_f32 = v_part;
    P.row_slot = row_slot;
    if ((st = launch_shrink(P, shrink_bm(R, d.num_experts), L.shrink2_splits, main)) != ST_OK)
      return st;
  }
  // 4) down GEMM + down LoRA expand -> y_perm (unweighted)
  {
    GemmParams P = base;
    P.a = act;
    P.a_gather = 0;
    P.w = w2;
    P.K = d.inter;
    P.N = d.hidden;
    P.w_packed = (packed >> 1) & 1;
    P.w_scale = w2_scale;
    P.mt_fast = (bm >= 128);  // (see the gate_up GEMM)
    if (has_lora) {
      for (int s = 0; s < lora->num_slots; ++s) P.lora_w[s] = lora->b_down[s];
      P.lora_w_shared = lora->shared_outer;  // shared-outer: one B2 for all experts
      P.part = v_part;
      P.part_splits = sep_down_shrink ? L.shrink2_splits : gateup_ncols(bm, d.inter);
      P.row_slot = row_slot;
      const long long down_ntiles = cdiv(d.hidden, bm >= 128 ? 256 : 128);
      const long long reread = down_ntiles * P.part_splits * R * L.rmax * (long long)sizeof(float);
      if (P.part_splits > kReduceMinSplits && reread >= kReduceMinBytes) {
        // every down n-tile would re-read all splits: reduce them once
        uint16_t *v_red = reinterpret_cast<uint16_t *>(wsb + L.v_red);
        SlotRanks sr{};
        for (int s = 0; s < lora->num_slots; ++s) {
          sr.rank[s] = lora->rank[s];
          sr.scaling[s] = lora->scaling[s];
        }
        const long long nthr = (long long)R * (L.rmax / 8);
        reduce_part_kernel<<<dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, main>>>(
            v_part, P.part_splits, R, L.rmax, row_slot, sr, v_red);
        if (hipGetLastError() != hipSuccess) return ST_HIP;
        P.part_bf16 = v_red;
      }
    }
    P.out_bf16 = y_perm;
    if ((st = fp8 ? (pow2 ? launch_gemm<MODE_DOWN, 2>(P, bm_gemm, main) : launch_gemm<MODE_DOWN, 1>(P, bm_gemm, main)) : launch_gemm<MODE_DOWN>(P, bm_gemm, main)) != ST_OK)
      return st;
  }
  return ST_OK;
}

}  // namespace moe
