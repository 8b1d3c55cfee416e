// probe_dq_atomics.hip -- the HBM atomic traffic a fused dQ would need, alone.
//
// The backward's dQ = scale dS K can be accumulated from the dK/dV kernel with
// fp32 atomic adds (the pages' design cuts such atomic adds; backward pass in
// the co-design list of the phantomic12 summary) or produced by a separate
// Q-major pass that recomputes S and dP (this library's choice). This kernel
// issues exactly the adds a fused kernel would issue, with nothing else: for
// every (sequence, K/V head, 128-key tile) work item of the dK/dV kernel, in
// that kernel's order (fa_order.h), and every 64-row query tile the key tile
// sees, one 64 x d fp32 block added into dq_acc [B, N, H, d], 256 threads per
// workgroup, consecutive lanes on consecutive columns. Its time is a lower
// bound on the fused kernel's, to set against the separate pass. Measurement
// only: libfa_probe.so, not part of the attention library.
#include <hip/hip_runtime.h>

#include "fa_order.h"

namespace {

constexpr int PROBE_BN = 128;   // keys per work item
constexpr int PROBE_TR = 64;    // query rows per tile

__global__ __launch_bounds__(256) void dq_atomics_kernel(float* acc, int B, int H, int N, int d, int causal) {
  fa::TileItem it;
  const int n_kt = (N + PROBE_BN - 1) / PROBE_BN;
  if (!fa::kv_item_level(blockIdx.x, B, H, n_kt, it)) return;
  const int kv0 = it.t * PROBE_BN;
  const int qt0 = causal ? kv0 / PROBE_TR : 0;
  const int n_qt = (N + PROBE_TR - 1) / PROBE_TR;
  const int per = PROBE_TR * d / 256;   // floats per thread and tile
  for (int qt = qt0; qt < n_qt; ++qt) {
    for (int u = 0; u < per; ++u) {
      const int idx = u * 256 + (int)threadIdx.x;
      const int row = idx / d, col = idx - row * d;
      const int q = qt * PROBE_TR + row;
      if (q < N) atomicAdd(acc + (((long)it.s * N + q) * H + it.h) * d + col, 1.0f);
    }
  }
}

}  // namespace

// dq_acc: fp32 [B, N, H, d] on the device; d a multiple of 4 (64 or 128).
// Adds, to element (s, q, h, :), one per key tile of 128 keys that query q's
// tile sees (all of them, or for causal those starting at or before q's 64-row
// tile). Returns the hipError_t of the launch (0 on success); a bad size
// returns hipErrorInvalidValue without launching.
extern "C" int fa_probe_dq_atomics(float* dq_acc, int B, int H, int N, int d, int causal, void* stream) {
  if (!dq_acc || B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return (int)hipErrorInvalidValue;
  const long grid = fa::kv_grid_level(B, H, (N + PROBE_BN - 1) / PROBE_BN);
  if (grid > 0x7fffffffL) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(dq_atomics_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, dq_acc, B, H, N, d,
                     causal);
  return (int)hipGetLastError();
}
