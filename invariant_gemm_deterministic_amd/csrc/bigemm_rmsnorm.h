// Internal interface between the C-ABI layer and the RMSNorm kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

// Y[i, :] = X[i, :] / sqrt(mean(X[i, :]^2) + eps) * gamma, one workgroup per row.
// bf16: X, gamma, Y are bf16 bit patterns; otherwise fp32. ldx, ldy in elements.
hipError_t launch_rmsnorm(bool bf16, const void* X, int64_t ldx, const void* gamma, void* Y, int64_t ldy, int64_t M,
                          int64_t D, float eps, hipStream_t stream);

}  // namespace bigemm
