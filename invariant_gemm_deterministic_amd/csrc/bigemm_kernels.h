// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

// The one tile configuration of each kernel.
constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kTileKBf16 = 64;   // bf16 and fp16 inputs
constexpr int kTileKMx = 128;    // MXFP8 and int8 inputs

// Input families (the kernel that runs) and the output type (a bigemm_dtype value).
enum { kInBf16 = 1, kInF16 = 2, kInMx = 3, kInI8 = 4 };
struct Op {
  int32_t in;
  int32_t out;
};

// wt (every launcher): W is given as its transpose, [N][ldw] with ldw >= K,
// and for MXFP8 W_scale as [N][ldws] with ldws >= K/32.
// cus (bf16 / fp16, MXFP8, int8): the device's compute units (the grid may be
// padded with prefetch workgroups up to one per CU; see prefetch_grid).
hipError_t launch_bf16(Op op, bool wt, const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                       int64_t ldx, int64_t ldw, int64_t ldy, int cus, hipStream_t stream);

// Opt-in split-K (bf16 / fp16 inputs): chunk sums of k_chunk K values into P
// ([ceil(K/k_chunk)][M][N] fp32, 16-byte aligned), then their ordered sum into Y.
hipError_t launch_bf16_split(Op op, bool wt, int32_t k_chunk, const void* X, const void* W, void* Y, void* P,
                             int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                             hipStream_t stream);

// Size of the static scratch array used by bigemm_run_split_k_static.
constexpr uint64_t kStaticScratchBytes = (uint64_t)64 << 20;

// Device address of the static scratch array on `device`, which must be the
// current device; looked up on the first call per device and cached.
hipError_t static_scratch_address(int device, void** out);

hipError_t launch_mxfp8(Op op, bool wt, const void* X, const void* W, void* Y, const void* XS, const void* WS,
                        int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                        int64_t ldxs, int64_t ldws, int cus, hipStream_t stream);

hipError_t launch_i8(bool wt, const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                     int64_t ldx, int64_t ldw, int64_t ldy, int cus, hipStream_t stream);

}  // namespace bigemm
