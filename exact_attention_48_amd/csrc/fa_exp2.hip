// fa_exp2.hip -- the softmax's element-wise exponential on its own, for checks.
//
// The attention kernels form P = 2^x with either the hardware v_exp_f32 or the
// FMA-pipe polynomial exp2_poly (the software exponential with range reduction
// of the FlashAttention-4 pages: phantomic12 summary, co-design list; daily.dev
// Summary). This kernel applies exactly those device functions to an array, so
// the values the kernels use can be compared bit for bit with a host emulation
// of the polynomial, and the hardware instruction's error can be measured
// against a float64 reference instead of assumed.
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_exp2.h"

namespace fa {

template <int EXPMODE>
__global__ __launch_bounds__(256) void exp2_eval_kernel(const float* __restrict__ x, float* __restrict__ y, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = exp2_sel<EXPMODE>(x[i]);
}

hipError_t exp2_eval_launch(const float* x, float* y, long n, int exp_mode, hipStream_t stream) {
  const long grid = (n + 255) / 256;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (exp_mode == 1)
    hipLaunchKernelGGL(exp2_eval_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, x, y, n);
  else
    hipLaunchKernelGGL(exp2_eval_kernel<0>, dim3((unsigned)grid), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

}  // namespace fa
