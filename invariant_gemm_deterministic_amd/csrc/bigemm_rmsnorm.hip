// Batch-invariant RMSNorm for CDNA4 (gfx950).
//
// The nondeterminism blog, section "batch-invariant RMSNorm", defines
//   RMSNorm(x_i) = x_i / sqrt((1/d) * sum_j x_ij^2 + eps) (.) gamma
// and gives the data-parallel strategy that keeps it batch-invariant: one
// worker per row, the whole reduction of the row inside that worker, and the
// same strategy at every batch size (for small batches it does not switch to
// a split reduction). Here one workgroup of 256 threads handles one row:
//
//   pass 1: thread t accumulates x^2 over the 8-element chunks t, t + 256,
//           t + 512, ... in that order (fp32, fused multiply-add); the 64
//           lanes of a wave are then combined by a butterfly (every lane ends
//           with the same value, since IEEE addition is commutative), and the
//           four wave sums are added in wave order;
//   pass 2: y = (x * r) * gamma with r = 1 / sqrt(sum / d + eps), rounded once
//           to the output type (round to nearest even for bf16).
//
// The reduction tree depends on d only. A thread keeps its first four chunks
// in registers between the passes (all of a row up to d = 8192); chunks past
// them are read again in pass 2, from the caches. The gamma values of those
// four chunks are requested with the row, before pass 1, so that pass 2 does
// not start with a dependent round trip to the cache (bf16 keeps both as raw
// 16-bit pairs and widens them where they are used).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bigemm_rmsnorm.h"

namespace bigemm {

namespace {

constexpr int kNormThreads = 256;
constexpr int kCached = 4;  // chunks of 8 elements a thread keeps in registers (D <= 8192)

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary32 -> bfloat16, round to nearest, ties to even; a NaN keeps its sign
// and top payload bits and gets the quiet bit.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight consecutive elements starting at element 8*c of a row, as fp32.
template <bool kBf16>
__device__ __forceinline__ void load8(const void* row, int c, float (&v)[8]) {
  if (kBf16) {
    const i32x4 q = *((const i32x4*)row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = (uint32_t)q[e];
      v[2 * e] = bf16_to_f32(w & 0xFFFFu);
      v[2 * e + 1] = bf16_to_f32(w >> 16);
    }
  } else {
    const float4 a = *((const float4*)row + 2 * c);
    const float4 b = *((const float4*)row + 2 * c + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Eight consecutive elements of a row held as loaded: four dwords of bf16
// pairs, or eight floats.
template <bool kBf16>
struct Raw8;
template <>
struct Raw8<true> {
  i32x4 q;
  __device__ __forceinline__ void load(const void* row, int c) { q = *((const i32x4*)row + c); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = (uint32_t)q[e];
      v[2 * e] = bf16_to_f32(w & 0xFFFFu);
      v[2 * e + 1] = bf16_to_f32(w >> 16);
    }
  }
};
template <>
struct Raw8<false> {
  float v8[8];
  __device__ __forceinline__ void load(const void* row, int c) { load8<false>(row, c, v8); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v8[e];
  }
};

template <bool kBf16>
__device__ __forceinline__ void store8(void* row, int c, const float (&v)[8]) {
  if (kBf16) {
    i32x4 q;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      q[e] = (int)(f32_to_bf16_rne(__float_as_uint(v[2 * e])) | (f32_to_bf16_rne(__float_as_uint(v[2 * e + 1])) << 16));
    *((i32x4*)row + c) = q;
  } else {
    *((float4*)row + 2 * c) = make_float4(v[0], v[1], v[2], v[3]);
    *((float4*)row + 2 * c + 1) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kNormThreads)
void bigemm_rmsnorm_kernel(const uint8_t* __restrict__ X, int64_t ldx_bytes, const void* __restrict__ gamma,
                           uint8_t* __restrict__ Y, int64_t ldy_bytes, int D, float eps) {
  __shared__ float wave_sum[kNormThreads / 64];
  const int tid = threadIdx.x;
  const uint8_t* x = X + (int64_t)blockIdx.x * ldx_bytes;  // one workgroup per row
  uint8_t* y = Y + (int64_t)blockIdx.x * ldy_bytes;
  const int nchunk = D / 8;

  // The thread's first kCached chunks, and their gamma, stay in registers for
  // pass 2; chunks beyond them (D > 8192) are read again there. The order is
  // the same.
  Raw8<kBf16> xr[kCached], gr[kCached];
#pragma unroll
  for (int i = 0; i < kCached; ++i) {
    const int c = tid + i * kNormThreads;
    if (c < nchunk) {
      xr[i].load(x, c);
      gr[i].load(gamma, c);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kCached; ++i) {
    const int c = tid + i * kNormThreads;
    if (c < nchunk) {
      float v[8];
      xr[i].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    }
  }
  for (int c = tid + kCached * kNormThreads; c < nchunk; c += kNormThreads) {
    float v[8];
    load8<kBf16>(x, c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wave_sum[tid >> 6] = ss;
  __syncthreads();
  const float total = ((wave_sum[0] + wave_sum[1]) + wave_sum[2]) + wave_sum[3];
  const float r = 1.0f / sqrtf(total / (float)D + eps);

#pragma unroll
  for (int i = 0; i < kCached; ++i) {
    const int c = tid + i * kNormThreads;
    if (c < nchunk) {
      float v[8], g[8];
      xr[i].get(v);
      gr[i].get(g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (v[e] * r) * g[e];
      store8<kBf16>(y, c, v);
    }
  }
  for (int c = tid + kCached * kNormThreads; c < nchunk; c += kNormThreads) {
    float v[8], g[8];
    load8<kBf16>(x, c, v);
    load8<kBf16>(gamma, c, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (v[e] * r) * g[e];
    store8<kBf16>(y, c, v);
  }
}

}  // namespace

hipError_t launch_rmsnorm(bool bf16, const void* X, int64_t ldx, const void* gamma, void* Y, int64_t ldy, int64_t M,
                          int64_t D, float eps, hipStream_t stream) {
  const int64_t es = bf16 ? 2 : 4;
  if (bf16)
    hipLaunchKernelGGL(bigemm_rmsnorm_kernel<true>, dim3((unsigned)M), dim3(kNormThreads), 0, stream,
                       (const uint8_t*)X, ldx * es, gamma, (uint8_t*)Y, ldy * es, (int)D, eps);
  else
    hipLaunchKernelGGL(bigemm_rmsnorm_kernel<false>, dim3((unsigned)M), dim3(kNormThreads), 0, stream,
                       (const uint8_t*)X, ldx * es, gamma, (uint8_t*)Y, ldy * es, (int)D, eps);
  return hipGetLastError();
}

}  // namespace bigemm
