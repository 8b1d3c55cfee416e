// fa_tiles.h -- tile plumbing shared by the attention kernels: the HBM -> LDS
// row copy, the per-lane LDS operand offsets of the swizzled tiles, output
// staging, and s_waitcnt helpers. All kernels run NWAVES = 4 waves per
// workgroup (one per SIMD) and stream tiles through an NSTAGE-deep LDS ring.
#pragma once

#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace tiles {

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int NSTAGE = 4;     // LDS ring depth
constexpr int PF = 4;         // MFMA operands read ahead

template <int N>
using ic = std::integral_constant<int, N>;

// HBM -> LDS copy of a ROWS x D bf16 tile of a [tokens][stride] tensor into a
// swizzled LDS tile; rows past the sequence end are clamped to its last row.
// All NW waves of the workgroup take part, PER_WAVE 1 KiB instructions each.
template <int D, int ROWS, int NW = NWAVES>
struct RowCopy {
  static constexpr int ROWB = D * 2;
  static constexpr int LPR = ROWB / 16;          // lanes per row
  static constexpr int RPI = 64 / LPR;           // rows per instruction
  static constexpr int NI = ROWS / RPI;          // instructions per tile
  static constexpr int PER_WAVE = NI / NW;
  static_assert(PER_WAVE * NW == NI, "tile copy must split evenly over the waves");
  unsigned off[PER_WAVE];                        // row * stride + swizzled chunk * 16
  int wave, lane;

  __device__ __forceinline__ int row(int u) const { return (wave * PER_WAVE + u) * RPI + lane / LPR; }
  __device__ __forceinline__ unsigned chunk16(int u) const {
    return (unsigned)(((lane % LPR) ^ lds_swz<D>(row(u))) * 16);
  }
  __device__ __forceinline__ void init(int wave_, int lane_, unsigned stride) {
    wave = wave_;
    lane = lane_;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) off[u] = (unsigned)row(u) * stride + chunk16(u);
  }
  // `base` points at token 0 of this head; rows r0 .. r0 + ROWS - 1. The
  // tile's first row is the (scalar) buffer base, so the per-lane offsets stay
  // loop-invariant. UNIFORM passes the base through readfirstlane, for callers
  // whose address arithmetic the compiler places on the vector unit.
  template <bool UNIFORM = false>
  __device__ __forceinline__ void issue(char FA_LDS* tile, const char* base, long stride, int r0, int L) const {
    const char* b = base + (long)r0 * stride;
    if (r0 + ROWS <= L) issue_full<UNIFORM>(tile, b);
    else issue_tail<UNIFORM>(tile, b, stride, L - 1 - r0);
  }
  // A whole tile whose first row is at `b`.
  template <bool UNIFORM = false>
  __device__ __forceinline__ void issue_full(char FA_LDS* tile, const char* b) const {
    const __amdgpu_buffer_rsrc_t rsrc = UNIFORM ? buffer_rsrc_uniform(b) : buffer_rsrc(b);
    char FA_LDS* dst = tile + wave * PER_WAVE * 1024;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) buf2lds16(rsrc, off[u], dst + u * 1024);
  }
  // The last tile of a sequence: rows past `last` (relative to `b`) repeat it.
  template <bool UNIFORM = false>
  __device__ __forceinline__ void issue_tail(char FA_LDS* tile, const char* b, long stride, int last) const {
    const __amdgpu_buffer_rsrc_t rsrc = UNIFORM ? buffer_rsrc_uniform(b) : buffer_rsrc(b);
    char FA_LDS* dst = tile + wave * PER_WAVE * 1024;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int r = min(row(u), last);
      buf2lds16(rsrc, (unsigned)r * (unsigned)stride + chunk16(u), dst + u * 1024);
    }
  }
};

// Per-lane LDS offsets of the MFMA operands in a swizzled [64][D] bf16 tile.
// The swizzle only XORs chunk bits, so other k-steps / d-blocks are an XOR away:
//   row operand (ds_read_b128) of k-step ks, rows 32 qb + l32:  (aoff ^ (ks << 5)) + qb * 32 * ROWB
//   transposed operand (two ds_read_b64_tr_b16) of d-block db, rows 16 t + ...:
//                         (troff[i] ^ (db << 6)) + t * 16 * ROWB, i = 0, 1
template <int D>
struct TileOffsets {
  int aoff;
  int troff[2];
  __device__ __forceinline__ void init(int lane) {
    constexpr int ROWB = D * 2;
    const int hl = lane >> 5, l32 = lane & 31, g16 = lane & 15;
    aoff = l32 * ROWB + ((hl ^ lds_swz<D>(l32)) << 4);
    const int dcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
    const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
    const int r0 = 4 * hl + (g16 >> 2), r1 = r0 + 8;
    troff[0] = r0 * ROWB + ((chunk ^ lds_swz<D>(r0)) * 16) + sub;
    troff[1] = r1 * ROWB + ((chunk ^ lds_swz<D>(r1)) * 16) + sub;
  }
  __device__ __forceinline__ bf16x8 row_operand(const char FA_LDS* tile, int ks, int blk) const {
    return lds_read16(tile + (aoff ^ (ks << 5)) + blk * 32 * D * 2);
  }
  __device__ __forceinline__ bf16x8 tr_operand(const char FA_LDS* tile, int t, int db) const {
    return cat(lds_read_tr(tile + (troff[0] ^ (db << 6)) + t * 16 * D * 2),
               lds_read_tr(tile + (troff[1] ^ (db << 6)) + t * 16 * D * 2));
  }
};

// Per-lane LDS offsets of the 8-bit K operand of the 32x32x64 MFMA in a tile of
// 128-byte rows (E4M3, d = 128), swizzled like a bf16 [rows][64] tile. Lane
// (row l32, half hl) takes bytes 64 ks + 32 hl .. + 31 of its row for k-step ks:
// logical 16-byte chunks 4 ks + 2 hl and 4 ks + 2 hl + 1. The Q^T operand holds
// the same bytes of the query rows, so the contraction pairs them up.
struct TileOffsetsK8 {
  int off[2];
  __device__ __forceinline__ void init(int lane) {
    const int hl = lane >> 5, l32 = lane & 31;
    const int sw = lds_swz<64>(l32);
    off[0] = l32 * 128 + (((2 * hl) ^ sw) << 4);
    off[1] = l32 * 128 + (((2 * hl + 1) ^ sw) << 4);
  }
  __device__ __forceinline__ i32x8 operand(const char FA_LDS* tile, int ks) const {
    const i32x4 lo = __builtin_bit_cast(i32x4, lds_read16(tile + (off[0] ^ (ks << 6))));
    const i32x4 hi = __builtin_bit_cast(i32x4, lds_read16(tile + (off[1] ^ (ks << 6))));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Stage a wave's 32 x D fp32 accumulator (transposed C layout: lane = row
// l32, register r of block db = column db*32 + 8(r/4) + 4(l/32) + r%4) as bf16
// through LDS and write whole 16-byte row segments to global memory.
template <int D>
__device__ __forceinline__ void store_rows_bf16(char FA_LDS* st, const f32x16* acc, float mul, __bf16* gbase,
                                                long row_stride, int row0, int L, int lane) {
  constexpr int OROWB = D * 2 + 16;
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + 8 * g + 4 * hl;
      const bf16x2 a = pack_bf16(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
      const bf16x2 b = pack_bf16(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
      *(bf16x4 FA_LDS*)(st + l32 * OROWB + dcol * 2) = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    }
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = D / 8;
  constexpr int PER_LANE = 32 * CPR / 64;
#pragma unroll
  for (int u = 0; u < PER_LANE; ++u) {
    const int idx = u * 64 + lane;
    const int row = idx / CPR, ch = idx % CPR;
    const int r = row0 + row;
    const bf16x8 v8 = *(const bf16x8 FA_LDS*)(st + row * OROWB + ch * 16);
    if (r < L) *(bf16x8*)(gbase + (long)r * row_stride + ch * 8) = v8;
  }
}

// Rows row0 + l32 (lanes l32 and l32 + 32) of a wave's fp32 accumulators, times
// `mul`, written straight to global memory: lane (l32, hl) holds columns
// db*32 + 8(r/4) + 4 hl + r%4 of its row, four consecutive floats per 16-byte store.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16* acc, float mul, float* gbase, long row_stride,
                                               int row0, int L, int lane) {
  const int l32 = lane & 31, hl = lane >> 5;
  const int r = row0 + l32;
  if (r >= L) return;
  float* rowp = gbase + (long)r * row_stride;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = {acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                       acc[db][4 * g + 3] * mul};
      *(f32x4*)(rowp + db * 32 + 8 * g + 4 * hl) = v;
    }
}

// Wait until at most `n` vector-memory operations of this wave are outstanding
// and no LDS operation is (n must be a compile-time constant after inlining;
// values above 20 wait for everything).
__device__ __forceinline__ void wait_vm(int n) {
#define FA_WAIT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(k)); break;
  switch (n) {
    FA_WAIT_CASE(1) FA_WAIT_CASE(2) FA_WAIT_CASE(3) FA_WAIT_CASE(4) FA_WAIT_CASE(5)
    FA_WAIT_CASE(6) FA_WAIT_CASE(7) FA_WAIT_CASE(8) FA_WAIT_CASE(9) FA_WAIT_CASE(10)
    FA_WAIT_CASE(11) FA_WAIT_CASE(12) FA_WAIT_CASE(13) FA_WAIT_CASE(14) FA_WAIT_CASE(15)
    FA_WAIT_CASE(16) FA_WAIT_CASE(17) FA_WAIT_CASE(18) FA_WAIT_CASE(19) FA_WAIT_CASE(20)
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0)); break;
  }
#undef FA_WAIT_CASE
}

}  // namespace tiles
}  // namespace fa
