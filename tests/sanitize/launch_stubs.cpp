// Host-only stand-ins for the kernel launchers and the static-scratch lookup,
// so that the C-ABI layer (bigemm_api.cpp) links into a CPU program built with
// the address and undefined-behaviour sanitizers. The validators never reach
// them; a call fails loudly.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../invariant_gemm_deterministic_amd/csrc/bigemm_attention.h"
#include "../../invariant_gemm_deterministic_amd/csrc/bigemm_kernels.h"
#include "../../invariant_gemm_deterministic_amd/csrc/bigemm_rmsnorm.h"

static hipError_t unreachable(const char* what) {
  fprintf(stderr, "sanitizer build: %s reached a kernel launch\n", what);
  abort();
}

namespace bigemm {
hipError_t launch_bf16(Op, bool, const void*, const void*, void*, int64_t, int64_t, int64_t, int64_t, int64_t,
                       int64_t, int, hipStream_t) {
  return unreachable("launch_bf16");
}
hipError_t launch_bf16_split(Op, bool, int32_t, const void*, const void*, void*, void*, int64_t, int64_t, int64_t,
                             int64_t, int64_t, int64_t, hipStream_t) {
  return unreachable("launch_bf16_split");
}
hipError_t launch_mxfp8(Op, bool, const void*, const void*, void*, const void*, const void*, int64_t, int64_t,
                        int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
  return unreachable("launch_mxfp8");
}
hipError_t launch_i8(bool, const void*, const void*, void*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                     int, hipStream_t) {
  return unreachable("launch_i8");
}
hipError_t static_scratch_address(int, void**) { return unreachable("static_scratch_address"); }
}  // namespace bigemm

namespace bigemm {
hipError_t launch_rmsnorm(bool, const void*, int64_t, const void*, void*, int64_t, int64_t, int64_t, float,
                          hipStream_t) {
  return unreachable("launch_rmsnorm");
}
hipError_t launch_paged_attention(const AttnParams&, hipStream_t) { return unreachable("launch_paged_attention"); }
hipError_t launch_kv_write(const KvWriteParams&, hipStream_t) { return unreachable("launch_kv_write"); }
}  // namespace bigemm
