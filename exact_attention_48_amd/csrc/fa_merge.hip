// fa_merge.hip -- merge of split-KV partial attention results for gfx950 (MI355X).
//
// Row by row, the combination step of the online softmax (podcast.app episode
// page, description) applied across key chunks:
//   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.
// The kernel is bound by HBM traffic (n_parts fp32 rows in, one bf16 row out),
// so it is laid out for coalescing, not arithmetic: rows are taken in
// (b, h, n) order, so a workgroup's LSE reads are one contiguous run per part;
// D / 8 lanes share a row and each moves 8 columns (two 16-byte loads per part,
// one 16-byte bf16 store). Every lane of a row derives the row's weights from
// the same n_parts LSE values, which the L1 serves after the first lane.
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, __bf16* __restrict__ o,
                                                    float* __restrict__ lse, int n_parts, int B, int H, int N) {
  constexpr int TPR = D / 8;                       // lanes per row
  constexpr int RPB = 256 / TPR;                   // rows per workgroup
  const long rows = (long)B * H * N;
  const long r = (long)blockIdx.x * RPB + threadIdx.x / TPR;   // ((b H + h) N + n): the LSE index
  if (r >= rows) return;
  const int col = (threadIdx.x % TPR) * 8;
  const long bh = r / N;
  const long n = r - bh * N;
  const long b = bh / H;
  const long h = bh - b * H;
  const long orow = (b * N + n) * H + h;           // row of [B, N, H, d]
  // LSE of the first PG parts stays in registers from the max pass, so for
  // up to PG parts every weight is known before any O load goes out and all
  // of a lane's loads are in flight together; more parts run in groups of PG.
  // A part whose weight is 0 (its row saw no key of the chunk) loads nothing.
  constexpr int PG = 16;
  float lv[PG];
  float m = -INFINITY;
#pragma unroll
  for (int g = 0; g < PG; ++g) {
    lv[g] = g < n_parts ? lse_part[g * rows + r] : -INFINITY;
    m = fmaxf(m, lv[g]);
  }
  for (int p = PG; p < n_parts; ++p) m = fmaxf(m, lse_part[p * rows + r]);
  float acc[8] = {};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int p0 = 0; p0 < n_parts; p0 += PG) {
      float w[PG];
      f32x4 a[PG], c[PG];
#pragma unroll
      for (int g = 0; g < PG; ++g) {
        const int p = p0 + g;
        float l = lv[g];
        if (p0 > 0) l = p < n_parts ? lse_part[p * rows + r] : -INFINITY;
        w[g] = expf(l - m);
      }
#pragma unroll
      for (int g = 0; g < PG; ++g) {
        a[g] = f32x4{};
        c[g] = f32x4{};
        if (w[g] > 0.f) {
          const float* src = o_part + ((p0 + g) * rows + orow) * D + col;
          a[g] = *(const f32x4*)src;
          c[g] = *(const f32x4*)(src + 4);
        }
      }
#pragma unroll
      for (int g = 0; g < PG; ++g) {
        tot += w[g];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = __builtin_fmaf(w[g], a[g][e], acc[e]);
          acc[4 + e] = __builtin_fmaf(w[g], c[g][e], acc[4 + e]);
        }
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const bf16x2 o0 = pack_bf16(acc[0] * inv, acc[1] * inv), o1 = pack_bf16(acc[2] * inv, acc[3] * inv);
  const bf16x2 o2 = pack_bf16(acc[4] * inv, acc[5] * inv), o3 = pack_bf16(acc[6] * inv, acc[7] * inv);
  const bf16x4 lo = __builtin_shufflevector(o0, o1, 0, 1, 2, 3), hi = __builtin_shufflevector(o2, o3, 0, 1, 2, 3);
  *(bf16x8*)(o + orow * D + col) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  if (col == 0) lse[r] = (m == -INFINITY) ? -INFINITY : m + logf(tot);
}

hipError_t merge_launch(const float* o_part, const float* lse_part, void* o, float* lse, int n_parts, int B,
                        int H, int N, int d, hipStream_t stream) {
  const long rows = (long)B * H * N;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (d / 8);
  const long grid = (rows + rpb - 1) / rpb;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, o_part, lse_part, (__bf16*)o,
                       lse, n_parts, B, H, N);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, o_part, lse_part, (__bf16*)o,
                       lse, n_parts, B, H, N);
  return hipGetLastError();
}

}  // namespace fa
