// fa_exp2.h -- launcher of the element-wise exponential check kernel (fa_exp2.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// y[i] = 2^x[i] by the attention kernels' exp2 device function; exp_mode 0 is
// the hardware v_exp_f32, 1 the FMA-pipe polynomial.
hipError_t exp2_eval_launch(const float* x, float* y, long n, int exp_mode, hipStream_t stream);

}  // namespace fa
