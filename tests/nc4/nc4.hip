// Device negative control for the invariance tests (test infrastructure only):
// a plain bf16 GEMM whose K-split count depends on the batch size M, modelled on
// the batch-dependent split count that the vLLM mHC batch-invariance PR removes
// (section "What": n_sms / cdiv(num_tokens, 64)). Each output element is owned
// by one thread, which sums each K chunk in order (fp32 FMA) and then adds the
// chunk sums in order: deterministic run to run, but not batch invariant.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

__global__ void nc4_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ Y,
                           int M, int N, int K, int64_t ldx, int64_t ldw, int64_t ldy, int splits) {
  const int j = blockIdx.x * 16 + (threadIdx.x & 15);
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (i >= M || j >= N) return;
  float total = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const int k0 = (int)((int64_t)K * s / splits), k1 = (int)((int64_t)K * (s + 1) / splits);
    float part = 0.0f;
    for (int k = k0; k < k1; ++k) part = fmaf(bf16_to_f32(X[i * ldx + k]), bf16_to_f32(W[(int64_t)k * ldw + j]), part);
    total += part;
  }
  Y[i * ldy + j] = total;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int nc4_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* X,
                                                                     int64_t ldx, const void* W, int64_t ldw, void* Y,
                                                                     int64_t ldy, void* stream) {
  if (M < 1 || N < 1 || K < 1 || ldx < K || ldw < N || ldy < N || !X || !W || !Y) return 1;
  if (M > (1 << 20) || N > (1 << 20) || K > (1 << 20)) return 1;
  int splits = 256 / (int)((M + 63) / 64);  // the batch-dependent split count under test
  if (splits < 1) splits = 1;
  if (splits > K) splits = (int)K;
  dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
  hipLaunchKernelGGL(nc4_kernel, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t*)X, (const uint16_t*)W,
                     (float*)Y, (int)M, (int)N, (int)K, ldx, ldw, ldy, splits);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
