// Tile-packed copies of the expert weights (gfx950).
//
// The grouped GEMMs stream each expert's weights one 64-wide K step at a time for a
// block of 128 output rows.  In the row-major layouts of the vLLM API page's routed op
// (w13 [E, 2I, H], w2 [E, H, I]) such a step gathers 128 segments of 128 bytes that lie
// 4 KB or more apart; in the packed layout it is one contiguous 16 KB block, which a
// streaming probe on MI355X reads at 7.1 TB/s against 6.2 TB/s for the scattered form.
//
// Packed layout of a weight with N rows and K columns per expert: blocks (e, s, t) in
// that order, s over 64-wide K steps and t over 128-row tiles, each block the 128 x 64
// sub-matrix row-major.  Blocks that GEMM tiles running side by side read at the same
// K step are neighbours (one contiguous stream, and no L2 set aliasing between them).  The gate_up tiles are in the GEMM's pairing order: tile t holds
// the 64 gate rows of intermediate columns [64 t, 64 t + 64) and then the 64 up rows of
// the same columns.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// one 16-byte chunk per thread; q indexes the packed buffer's chunks
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src,
                                                   uint16_t *__restrict__ dst, int E, int N, int K,
                                                   int I_gate_up) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int ksteps = K / 64, tiles = N / 128;
  const long long total = (long long)E * N * K / 8;
  if (q >= total) return;
  const int c8 = (int)(q & 7);             // chunk of the 64-wide row piece
  const int r = (int)((q >> 3) & 127);     // row inside the tile
  const long long blk = q >> 10;           // (e, s, t) block
  const int t = (int)(blk % tiles);
  const int s = (int)((blk / tiles) % ksteps);
  const int e = (int)(blk / ((long long)ksteps * tiles));
  int row;
  if (I_gate_up > 0) row = (r / 64) * I_gate_up + t * 64 + r % 64;  // gate rows, then up rows
  else row = t * 128 + r;
  const u32x4_t v =
      *reinterpret_cast<const u32x4_t *>(src + ((size_t)e * N + row) * K + (size_t)s * 64 + c8 * 8);
  *reinterpret_cast<u32x4_t *>(dst + (size_t)q * 8) = v;
}

int launch_pack(const uint16_t *src, uint16_t *dst, int E, int N, int K, int I_gate_up, hipStream_t s) {
  const long long chunks = (long long)E * N * K / 8;
  if (chunks == 0) return ST_OK;
  const long long blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffffll) return ST_UNSUPPORTED;
  pack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(src, dst, E, N, K, I_gate_up);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

// FP8 codes (one byte each): the same (e, s, t) block order, each block 128 rows x 64
// codes = 8 KB, so one K step of a 128-row tile is one contiguous 8 KB read (the row-major
// codes give 64-byte pieces 2 KB or more apart); one 16-byte chunk per thread
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint8_t *__restrict__ src,
                                                       uint8_t *__restrict__ dst, int E, int N, int K,
                                                       int I_gate_up) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int ksteps = K / 64, tiles = N / 128;
  const long long total = (long long)E * N * K / 16;
  if (q >= total) return;
  const int c16 = (int)(q & 3);            // chunk of the 64-code row piece
  const int r = (int)((q >> 2) & 127);     // row inside the tile
  const long long blk = q >> 9;            // (e, s, t) block
  const int t = (int)(blk % tiles);
  const int s = (int)((blk / tiles) % ksteps);
  const int e = (int)(blk / ((long long)ksteps * tiles));
  int row;
  if (I_gate_up > 0) row = (r / 64) * I_gate_up + t * 64 + r % 64;
  else row = t * 128 + r;
  const u32x4_t v =
      *reinterpret_cast<const u32x4_t *>(src + ((size_t)e * N + row) * K + (size_t)s * 64 + c16 * 16);
  *reinterpret_cast<u32x4_t *>(dst + (size_t)q * 16) = v;
}

int launch_pack_fp8(const uint8_t *src, uint8_t *dst, int E, int N, int K, int I_gate_up, hipStream_t s) {
  const long long chunks = (long long)E * N * K / 16;
  if (chunks == 0) return ST_OK;
  const long long blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffffll) return ST_UNSUPPORTED;
  pack_fp8_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(src, dst, E, N, K, I_gate_up);
  return hipGetLastError() == hipSuccess ? ST_OK : ST_HIP;
}

}  // namespace

int launch_pack_weights_fp8(const moe_lora_dims &d, const uint8_t *w1, const uint8_t *w2, uint8_t *w1p,
                            uint8_t *w2p, hipStream_t s) {
  if (w1) {
    const int st = launch_pack_fp8(w1, w1p, d.num_experts, 2 * d.inter, d.hidden, d.inter, s);
    if (st != ST_OK) return st;
  }
  return w2 ? launch_pack_fp8(w2, w2p, d.num_experts, d.hidden, d.inter, 0, s) : ST_OK;
}

int launch_pack_weights(const moe_lora_dims &d, const uint16_t *w1, const uint16_t *w2, uint16_t *w1p,
                        uint16_t *w2p, hipStream_t s) {
  if (w1) {
    const int st = launch_pack(w1, w1p, d.num_experts, 2 * d.inter, d.hidden, d.inter, s);
    if (st != ST_OK) return st;
  }
  return w2 ? launch_pack(w2, w2p, d.num_experts, d.hidden, d.inter, 0, s) : ST_OK;
}

}  // namespace moe
