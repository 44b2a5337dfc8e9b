// Internal interface between the C-ABI layer and the paged-attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bigemm {

// KV positions per split: fixed, whatever the batch or the context length.
constexpr int kAttnSplit = 256;

struct AttnParams {
  const uint16_t* Q;          // [T][H][D] bf16
  const uint16_t* K;          // [num_blocks][Hkv][block_size][D] bf16
  const uint16_t* V;          // same layout as K
  const int32_t* seq_ids;     // [T]
  const int32_t* positions;   // [T]
  const int32_t* block_table; // [num_seqs][max_blocks]
  void* O;                    // [T][H][D] fp32 or bf16
  float* ws_acc;              // [T][H][nsplit][D]
  float* ws_ml;               // [T][H][nsplit][2]: split maximum, split sum of weights
  int32_t T, H, Hkv, D;
  int32_t bs_log2, num_blocks, num_seqs, max_blocks, max_context, nsplit;
  float scale;
  int32_t out_bf16;
};

struct KvWriteParams {
  const uint16_t* K_new;      // [T][Hkv][D] bf16
  const uint16_t* V_new;
  const int32_t* seq_ids;
  const int32_t* positions;
  const int32_t* block_table;
  uint16_t* K;                // caches, layout as in AttnParams
  uint16_t* V;
  int32_t T, Hkv, D;
  int32_t bs_log2, num_blocks, num_seqs, max_blocks;
};

// Split kernel (one workgroup per token, KV head and split) then the ordered merge.
hipError_t launch_paged_attention(const AttnParams& p, hipStream_t stream);

// Copies each token's K/V rows into the slot its block table gives.
hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream);

}  // namespace bigemm
