// C ABI of the batch-invariant GEMM (declared in include/bigemm.h).
//
// The handle is shape-free: bigemm_create sees no M, N or K, so the one tile
// configuration cannot be chosen per shape — the single-configuration rule of
// the nondeterminism blog's batch-invariant matmul section, enforced by the
// interface. Creation refuses every device but gfx950 and every descriptor
// but those provided, rather than falling back (the fail-closed entry-point
// discipline of the vLLM mHC batch-invariance PR, review follow-up).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>

#include <atomic>

#include "../../include/bigemm.h"
#include "bigemm_kernels.h"
#include "bigemm_attention.h"
#include "bigemm_rmsnorm.h"

struct bigemm_s {
  bigemm::Op op;
  int device;
  int cus;          // the device's compute units
  int32_t k_chunk;  // 0: no split-K
  bool w_trans;     // W given as its transpose, [N, K] (bigemm_create_wt)
};

namespace {

constexpr int64_t kOffsetLimit = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The descriptors provided (include/bigemm.h); in == 0 for anything else.
bigemm::Op desc_op(const bigemm_desc* d) {
  bigemm::Op op{0, 0};
  if (!d || d->x_type != d->w_type) return op;
  const bool fout = d->y_type == BIGEMM_F32 || d->y_type == BIGEMM_BF16;
  if ((d->x_type == BIGEMM_BF16 || d->x_type == BIGEMM_F16) && fout && d->scale_block == 0)
    op = {d->x_type == BIGEMM_BF16 ? bigemm::kInBf16 : bigemm::kInF16, d->y_type};
  else if (d->x_type == BIGEMM_E4M3 && fout && d->scale_block == 32)
    op = {bigemm::kInMx, d->y_type};
  else if (d->x_type == BIGEMM_I8 && d->y_type == BIGEMM_I32 && d->scale_block == 0)
    op = {bigemm::kInI8, d->y_type};
  return op;
}

// wt: W is [N, K] with ldw >= K (and for MXFP8 W_scale [N, K/32] with
// ldws >= K/32) instead of [K, N] with ldw >= N (W_scale [K/32, N], ldws >= N).
bigemm_status check(bigemm::Op op, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                    const void* W, int64_t ldw, const void* Y, int64_t ldy, const void* XS,
                    int64_t ldxs, const void* WS, int64_t ldws, bool wt = false) {
  if (op.in == 0) return BIGEMM_ERR_UNSUPPORTED;
  if (M < 0 || N < 1 || K < 1) return BIGEMM_ERR_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BIGEMM_ERR_ARG;
  if (((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX) return BIGEMM_ERR_ARG;  // grid size
  const bool mx = op.in == bigemm::kInMx;
  const int64_t es = (op.in == bigemm::kInBf16 || op.in == bigemm::kInF16) ? 2 : 1;
  const int64_t eo = op.out == BIGEMM_BF16 ? 2 : 4;
  // bf16 / fp16: any K and N; only whole rows must be 16-byte aligned (below).
  if (mx && (K % 32 != 0 || N % 16 != 0)) return BIGEMM_ERR_ARG;
  if (op.in == bigemm::kInI8 && (K % 16 != 0 || N % 16 != 0)) return BIGEMM_ERR_ARG;
  if (ldx < K || ldw < (wt ? K : N) || ldy < N) return BIGEMM_ERR_ARG;
  // Every row 16-byte aligned (ld times the element size a multiple of 16), and the
  // 128 rows of a tile inside the 32-bit buffer offsets (128 * ld * element size
  // below 2^31); both written without products that could overflow.
  if (ldx % (16 / es) != 0 || ldw % (16 / es) != 0 || ldy % (16 / eo) != 0) return BIGEMM_ERR_ARG;
  if (ldx >= kOffsetLimit / (128 * es) || ldw >= kOffsetLimit / (128 * es) || ldy >= kOffsetLimit / (128 * eo))
    return BIGEMM_ERR_ARG;
  if (!mx) {
    if (XS != nullptr || WS != nullptr) return BIGEMM_ERR_ARG;
  } else {
    if (ldxs < K / 32 || ldws < (wt ? K / 32 : N)) return BIGEMM_ERR_ARG;
    const int64_t wrows = wt ? 128 : K / 32;  // W_scale rows one tile addresses (K >= 32 here)
    if (ldxs >= kOffsetLimit / 128 || ldws >= (kOffsetLimit + wrows - 1) / wrows) return BIGEMM_ERR_ARG;
  }
  if (M == 0) return BIGEMM_OK;
  if (!X || !W || !Y) return BIGEMM_ERR_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return BIGEMM_ERR_ARG;
  if (mx && (!XS || !WS)) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

bigemm_status rmsnorm_check(int32_t dtype, int64_t M, int64_t D, const void* X, int64_t ldx, const void* G,
                            const void* Y, int64_t ldy) {
  if (dtype != BIGEMM_BF16 && dtype != BIGEMM_F32) return BIGEMM_ERR_UNSUPPORTED;
  if (M < 0 || M > INT32_MAX || D < 8 || D > 65536 || D % 8 != 0) return BIGEMM_ERR_ARG;
  const int64_t es = dtype == BIGEMM_BF16 ? 2 : 4;
  if (ldx < D || ldy < D || ldx % (16 / es) != 0 || ldy % (16 / es) != 0) return BIGEMM_ERR_ARG;
  if (M == 0) return BIGEMM_OK;
  if (!X || !G || !Y || !aligned16(X) || !aligned16(G) || !aligned16(Y)) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

// Workspace bytes of a split-K run: ceil(K / k_chunk) chunk sums of M x N fp32,
// or 0 when there is no split (no k_chunk, or a single chunk).
// Saturates at UINT64_MAX (the exact product can need up to 2^90 for sizes that
// other checks reject), so that no size wraps to a small one.
uint64_t split_need(int32_t k_chunk, int64_t M, int64_t N, int64_t K) {
  if (k_chunk <= 0 || K <= k_chunk || M <= 0 || N <= 0) return 0;
  const unsigned __int128 b =
      (unsigned __int128)(uint64_t)((K + k_chunk - 1) / k_chunk) * (uint64_t)M * (uint64_t)N * 4u;
  return b > (unsigned __int128)UINT64_MAX ? UINT64_MAX : (uint64_t)b;
}

// The limits a split-K run adds to check(): the chunk sums are stored through
// the partial kernel's 32-bit tile offsets with row stride N (128 rows of N
// fp32 must stay below 2^31 bytes, whatever the output type), the merge grid
// (at most one thread per output) and the (chunk, tile) grid must fit, and the
// workspace must be present, 16-byte aligned and large enough.
bigemm_status split_check(int32_t k_chunk, int64_t M, int64_t N, int64_t K, const void* ws, uint64_t ws_bytes) {
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BIGEMM_ERR_ARG;
  const uint64_t need = split_need(k_chunk, M, N, K);
  if (need == 0) return BIGEMM_OK;
  if (128 * N * 4 >= kOffsetLimit) return BIGEMM_ERR_ARG;
  if ((__int128)((K + k_chunk - 1) / k_chunk) * ((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX)
    return BIGEMM_ERR_ARG;
  if (M * N > (int64_t)INT32_MAX * 256) return BIGEMM_ERR_ARG;  // merge grid (one thread per output at most)
  if (!ws || !aligned16(ws) || ws_bytes < need) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

// gfx950 check for the current device, done once per device (0 unknown, 1 yes, 2 no).
std::atomic<int> g_arch_ok[64];

bigemm_status current_device_supported() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return BIGEMM_ERR_DEVICE;
  }
  int state = dev >= 0 && dev < 64 ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return BIGEMM_ERR_DEVICE;
    }
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    state = ok ? 1 : 2;
    if (dev >= 0 && dev < 64) g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? BIGEMM_OK : BIGEMM_ERR_UNSUPPORTED;
}

// A handle runs on the device it was created on: the current device must be
// that one (a launch on another device would use the caller's stream and
// buffers of a different GPU).
bigemm_status handle_device_current(const bigemm_s* h) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return BIGEMM_ERR_DEVICE;
  }
  return dev == h->device ? BIGEMM_OK : BIGEMM_ERR_ARG;
}

// The one fixed kernel of the handle's input family (no split).
hipError_t launch_unsplit(const bigemm_s* h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                          const void* W, int64_t ldw, void* Y, int64_t ldy, const void* XS, int64_t ldxs,
                          const void* WS, int64_t ldws, hipStream_t stream) {
  const bigemm::Op op = h->op;
  const bool wt = h->w_trans;
  if (op.in == bigemm::kInMx)
    return bigemm::launch_mxfp8(op, wt, X, W, Y, XS, WS, M, N, K, ldx, ldw, ldy, ldxs, ldws, h->cus, stream);
  if (op.in == bigemm::kInI8) return bigemm::launch_i8(wt, X, W, Y, M, N, K, ldx, ldw, ldy, h->cus, stream);
  return bigemm::launch_bf16(op, wt, X, W, Y, M, N, K, ldx, ldw, ldy, h->cus, stream);
}

// ------------------------------------------------------------------ attention
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int log2_exact(int32_t v) {
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int k = 0;
  while ((1 << k) != v) ++k;
  return k;
}

bigemm_status kv_layout_check(const bigemm_kv_layout* kv) {
  if (!kv) return BIGEMM_ERR_ARG;
  if (kv->num_kv_heads < 1 || (kv->head_dim != 64 && kv->head_dim != 128)) return BIGEMM_ERR_ARG;
  if (kv->block_size > 4096 || log2_exact(kv->block_size) < 0) return BIGEMM_ERR_ARG;
  if (kv->num_blocks < 1 || kv->num_seqs < 1 || kv->max_blocks < 1) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

// Sizes of a paged-attention call; fills nsplit and the workspace bytes.
bigemm_status attn_sizes(const bigemm_kv_layout* kv, int64_t T, int32_t H, int32_t max_context, int32_t* nsplit,
                         uint64_t* need) {
  const bigemm_status st = kv_layout_check(kv);
  if (st != BIGEMM_OK) return st;
  if (T < 0 || H < 1 || H % kv->num_kv_heads != 0) return BIGEMM_ERR_ARG;
  const int32_t G = H / kv->num_kv_heads;
  if (G < 1 || G > 16) return BIGEMM_ERR_ARG;  // the query heads of a group fill one 16-row MFMA tile
  if (max_context < 1 || (int64_t)max_context > (int64_t)kv->max_blocks * kv->block_size) return BIGEMM_ERR_ARG;
  const int64_t ns = ((int64_t)max_context + bigemm::kAttnSplit - 1) / bigemm::kAttnSplit;
  if ((__int128)T * kv->num_kv_heads * ns > INT32_MAX || (__int128)T * H * (kv->head_dim / 32) > INT32_MAX)
    return BIGEMM_ERR_ARG;
  *nsplit = (int32_t)ns;
  *need = (uint64_t)T * (uint64_t)H * (uint64_t)ns * (uint64_t)(kv->head_dim + 2) * 4u;
  return BIGEMM_OK;
}

bigemm_status attn_check(const bigemm_kv_layout* kv, int64_t T, int32_t H, int32_t max_context, int32_t out_dtype,
                         const void* Q, const void* Kc, const void* Vc, const int32_t* seq, const int32_t* pos,
                         const int32_t* bt, const void* O, const void* ws, uint64_t ws_bytes, int32_t* nsplit) {
  if (out_dtype != BIGEMM_F32 && out_dtype != BIGEMM_BF16) return BIGEMM_ERR_UNSUPPORTED;
  uint64_t need = 0;
  const bigemm_status st = attn_sizes(kv, T, H, max_context, nsplit, &need);
  if (st != BIGEMM_OK || T == 0) return st;
  if (!Q || !Kc || !Vc || !seq || !pos || !bt || !O || !ws) return BIGEMM_ERR_ARG;
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O) || !aligned16(ws)) return BIGEMM_ERR_ARG;
  if (!aligned4(seq) || !aligned4(pos) || !aligned4(bt)) return BIGEMM_ERR_ARG;
  if (ws_bytes < need) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

}  // namespace

bigemm_status bigemm_kv_cache_write(const bigemm_kv_layout* kv, int64_t T, const void* K_new, const void* V_new,
                                    const int32_t* seq_ids, const int32_t* positions, const int32_t* block_table,
                                    void* K_cache, void* V_cache, void* stream) {
  const bigemm_status st = kv_layout_check(kv);
  if (st != BIGEMM_OK) return st;
  if (T < 0 || (__int128)T * kv->num_kv_heads * (kv->head_dim / 8) >= (int64_t)INT32_MAX) return BIGEMM_ERR_ARG;
  if (T == 0) return BIGEMM_OK;
  if (!K_new || !V_new || !seq_ids || !positions || !block_table || !K_cache || !V_cache) return BIGEMM_ERR_ARG;
  if (!aligned16(K_new) || !aligned16(V_new) || !aligned16(K_cache) || !aligned16(V_cache)) return BIGEMM_ERR_ARG;
  if (!aligned4(seq_ids) || !aligned4(positions) || !aligned4(block_table)) return BIGEMM_ERR_ARG;
  const bigemm_status dv = current_device_supported();
  if (dv != BIGEMM_OK) return dv;
  bigemm::KvWriteParams p;
  p.K_new = (const uint16_t*)K_new;
  p.V_new = (const uint16_t*)V_new;
  p.seq_ids = seq_ids;
  p.positions = positions;
  p.block_table = block_table;
  p.K = (uint16_t*)K_cache;
  p.V = (uint16_t*)V_cache;
  p.T = (int32_t)T;
  p.Hkv = kv->num_kv_heads;
  p.D = kv->head_dim;
  p.bs_log2 = log2_exact(kv->block_size);
  p.num_blocks = kv->num_blocks;
  p.num_seqs = kv->num_seqs;
  p.max_blocks = kv->max_blocks;
  const hipError_t e = bigemm::launch_kv_write(p, (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}

bigemm_status bigemm_attn_workspace_size(const bigemm_kv_layout* kv, int64_t T, int32_t num_heads,
                                         int32_t max_context, uint64_t* bytes) {
  if (!bytes) return BIGEMM_ERR_ARG;
  int32_t ns = 0;
  uint64_t need = 0;
  const bigemm_status st = attn_sizes(kv, T, num_heads, max_context, &ns, &need);
  if (st != BIGEMM_OK) return st;
  *bytes = need;
  return BIGEMM_OK;
}

bigemm_status bigemm_paged_attention_check_args(const bigemm_kv_layout* kv, int64_t T, int32_t num_heads,
                                                int32_t max_context, int32_t out_dtype, const void* Q,
                                                const void* K_cache, const void* V_cache, const int32_t* seq_ids,
                                                const int32_t* positions, const int32_t* block_table,
                                                const void* O, const void* workspace, uint64_t workspace_bytes) {
  int32_t ns = 0;
  return attn_check(kv, T, num_heads, max_context, out_dtype, Q, K_cache, V_cache, seq_ids, positions,
                    block_table, O, workspace, workspace_bytes, &ns);
}

bigemm_status bigemm_paged_attention(const bigemm_kv_layout* kv, int64_t T, int32_t num_heads, int32_t max_context,
                                     float scale, int32_t out_dtype, const void* Q, const void* K_cache,
                                     const void* V_cache, const int32_t* seq_ids, const int32_t* positions,
                                     const int32_t* block_table, void* O, void* workspace,
                                     uint64_t workspace_bytes, void* stream) {
  int32_t ns = 0;
  const bigemm_status st = attn_check(kv, T, num_heads, max_context, out_dtype, Q, K_cache, V_cache, seq_ids,
                                      positions, block_table, O, workspace, workspace_bytes, &ns);
  if (st != BIGEMM_OK || T == 0) return st;
  const bigemm_status dv = current_device_supported();
  if (dv != BIGEMM_OK) return dv;
  bigemm::AttnParams p;
  p.Q = (const uint16_t*)Q;
  p.K = (const uint16_t*)K_cache;
  p.V = (const uint16_t*)V_cache;
  p.seq_ids = seq_ids;
  p.positions = positions;
  p.block_table = block_table;
  p.O = O;
  p.ws_acc = (float*)workspace;
  p.ws_ml = (float*)workspace + (int64_t)T * num_heads * ns * kv->head_dim;
  p.T = (int32_t)T;
  p.H = num_heads;
  p.Hkv = kv->num_kv_heads;
  p.D = kv->head_dim;
  p.bs_log2 = log2_exact(kv->block_size);
  p.num_blocks = kv->num_blocks;
  p.num_seqs = kv->num_seqs;
  p.max_blocks = kv->max_blocks;
  p.max_context = max_context;
  p.nsplit = ns;
  p.scale = scale;
  p.out_bf16 = out_dtype == BIGEMM_BF16;
  const hipError_t e = bigemm::launch_paged_attention(p, (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}


extern "C" {

int32_t bigemm_abi_version(void) { return BIGEMM_ABI_VERSION; }

const char* bigemm_status_str(bigemm_status s) {
  switch (s) {
    case BIGEMM_OK: return "ok";
    case BIGEMM_ERR_ARG: return "invalid argument";
    case BIGEMM_ERR_UNSUPPORTED: return "unsupported device or descriptor (gfx950; bf16, fp16, MXFP8 or int8)";
    case BIGEMM_ERR_DEVICE: return "HIP device error";
    case BIGEMM_ERR_NOMEM: return "out of host memory";
    case BIGEMM_ERR_SCRATCH:
      return "the split-K chunk sums need more than the static scratch buffer holds (BIGEMM_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

bigemm_status bigemm_check_args(const bigemm_desc* desc, int64_t M, int64_t N, int64_t K,
                                const void* X, int64_t ldx, const void* W, int64_t ldw,
                                const void* Y, int64_t ldy, const void* X_scale, int64_t ldxs,
                                const void* W_scale, int64_t ldws) {
  if (!desc) return BIGEMM_ERR_ARG;
  return check(desc_op(desc), M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs, W_scale, ldws);
}

bigemm_status bigemm_check_args_wt(const bigemm_desc* desc, int64_t M, int64_t N, int64_t K,
                                   const void* X, int64_t ldx, const void* W, int64_t ldw,
                                   const void* Y, int64_t ldy, const void* X_scale, int64_t ldxs,
                                   const void* W_scale, int64_t ldws) {
  if (!desc) return BIGEMM_ERR_ARG;
  return check(desc_op(desc), M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs, W_scale, ldws, true);
}

bigemm_status bigemm_create(const bigemm_desc* desc, bigemm_t* out) {
  if (!out) return BIGEMM_ERR_ARG;
  *out = nullptr;
  if (!desc) return BIGEMM_ERR_ARG;
  const bigemm::Op op = desc_op(desc);
  if (op.in == 0) return BIGEMM_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return BIGEMM_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return BIGEMM_ERR_DEVICE;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0 ||
      (prop.gcnArchName[6] != '\0' && prop.gcnArchName[6] != ':'))
    return BIGEMM_ERR_UNSUPPORTED;
  bigemm_s* h = new (std::nothrow) bigemm_s;
  if (!h) return BIGEMM_ERR_NOMEM;
  h->op = op;
  h->device = dev;
  h->cus = prop.multiProcessorCount;
  h->k_chunk = 0;
  h->w_trans = false;
  *out = h;
  return BIGEMM_OK;
}

bigemm_status bigemm_create_wt(const bigemm_desc* desc, bigemm_t* out) {
  if (!out) return BIGEMM_ERR_ARG;
  *out = nullptr;
  if (!desc) return BIGEMM_ERR_ARG;
  const bigemm_status st = bigemm_create(desc, out);
  if (st != BIGEMM_OK) return st;
  (*out)->w_trans = true;
  return BIGEMM_OK;
}

bigemm_status bigemm_create_split_k(const bigemm_desc* desc, int32_t k_chunk, bigemm_t* out) {
  if (!out) return BIGEMM_ERR_ARG;
  *out = nullptr;
  if (!desc) return BIGEMM_ERR_ARG;
  const bigemm::Op op = desc_op(desc);
  if (op.in != bigemm::kInBf16 && op.in != bigemm::kInF16) return BIGEMM_ERR_UNSUPPORTED;
  if (k_chunk < bigemm::kTileKBf16 || k_chunk % bigemm::kTileKBf16 != 0) return BIGEMM_ERR_ARG;
  const bigemm_status st = bigemm_create(desc, out);
  if (st != BIGEMM_OK) return st;
  (*out)->k_chunk = k_chunk;
  // Set-up of bigemm_run_split_k_static on this device: the static scratch
  // array's device address, looked up once per device.
  void* scratch = nullptr;
  if (bigemm::static_scratch_address((*out)->device, &scratch) != hipSuccess) {
    (void)hipGetLastError();
    delete *out;
    *out = nullptr;
    return BIGEMM_ERR_DEVICE;
  }
  return BIGEMM_OK;
}

bigemm_status bigemm_create_split_k_wt(const bigemm_desc* desc, int32_t k_chunk, bigemm_t* out) {
  const bigemm_status st = bigemm_create_split_k(desc, k_chunk, out);
  if (st != BIGEMM_OK) return st;
  (*out)->w_trans = true;
  return BIGEMM_OK;
}

bigemm_status bigemm_workspace_size(bigemm_t h, int64_t M, int64_t N, int64_t K, uint64_t* bytes) {
  if (!h || !bytes || M < 0 || N < 0 || K < 0) return BIGEMM_ERR_ARG;
  *bytes = split_need(h->k_chunk, M, N, K);
  return BIGEMM_OK;
}

bigemm_status bigemm_check_args_split_k(const bigemm_desc* desc, int32_t k_chunk, int64_t M, int64_t N, int64_t K,
                                        const void* X, int64_t ldx, const void* W, int64_t ldw, const void* Y,
                                        int64_t ldy, const void* workspace, uint64_t workspace_bytes) {
  if (!desc) return BIGEMM_ERR_ARG;
  const bigemm::Op op = desc_op(desc);
  if (op.in != bigemm::kInBf16 && op.in != bigemm::kInF16) return BIGEMM_ERR_UNSUPPORTED;
  if (k_chunk < bigemm::kTileKBf16 || k_chunk % bigemm::kTileKBf16 != 0) return BIGEMM_ERR_ARG;
  const bigemm_status st = check(op, M, N, K, X, ldx, W, ldw, Y, ldy, nullptr, 0, nullptr, 0);
  if (st != BIGEMM_OK || M == 0) return st;
  return split_check(k_chunk, M, N, K, workspace, workspace_bytes);
}

bigemm_status bigemm_run_ws(bigemm_t h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                            const void* W, int64_t ldw, void* Y, int64_t ldy, const void* X_scale,
                            int64_t ldxs, const void* W_scale, int64_t ldws, void* workspace,
                            uint64_t workspace_bytes, void* stream) {
  if (!h) return BIGEMM_ERR_ARG;
  const bigemm_status st = check(h->op, M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs, W_scale, ldws, h->w_trans);
  if (st != BIGEMM_OK || M == 0) return st;
  const bigemm_status sst = split_check(h->k_chunk, M, N, K, workspace, workspace_bytes);
  if (sst != BIGEMM_OK) return sst;
  const bigemm_status dv = handle_device_current(h);
  if (dv != BIGEMM_OK) return dv;
  if (split_need(h->k_chunk, M, N, K) == 0) {  // unsplit handle, or a single chunk: the one fixed kernel
    const hipError_t e = launch_unsplit(h, M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs,
                                        W_scale, ldws, (hipStream_t)stream);
    return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
  }
  const hipError_t e = bigemm::launch_bf16_split(h->op, h->w_trans, h->k_chunk, X, W, Y, workspace, M, N, K, ldx,
                                                 ldw, ldy, (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}

bigemm_status bigemm_run_split_k_static(bigemm_t h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                                        const void* W, int64_t ldw, void* Y, int64_t ldy, void* stream) {
  if (!h) return BIGEMM_ERR_ARG;
  if (h->k_chunk <= 0) return BIGEMM_ERR_ARG;  // a split-K handle only
  const bigemm_status st = check(h->op, M, N, K, X, ldx, W, ldw, Y, ldy, nullptr, 0, nullptr, 0, h->w_trans);
  if (st != BIGEMM_OK || M == 0) return st;
  const uint64_t need = split_need(h->k_chunk, M, N, K);
  if (need > bigemm::kStaticScratchBytes) return BIGEMM_ERR_SCRATCH;
  const bigemm_status dv = handle_device_current(h);
  if (dv != BIGEMM_OK) return dv;
  if (need == 0) {  // a single chunk: the one fixed kernel, no scratch
    const hipError_t e = launch_unsplit(h, M, N, K, X, ldx, W, ldw, Y, ldy, nullptr, 0, nullptr,
                                        0, (hipStream_t)stream);
    return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
  }
  void* scratch = nullptr;
  if (bigemm::static_scratch_address(h->device, &scratch) != hipSuccess) {
    (void)hipGetLastError();
    return BIGEMM_ERR_DEVICE;
  }
  const bigemm_status sst = split_check(h->k_chunk, M, N, K, scratch, bigemm::kStaticScratchBytes);
  if (sst != BIGEMM_OK) return sst;
  const hipError_t e = bigemm::launch_bf16_split(h->op, h->w_trans, h->k_chunk, X, W, Y, scratch, M, N, K, ldx,
                                                 ldw, ldy, (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}

bigemm_status bigemm_rmsnorm_check_args(int32_t dtype, int64_t M, int64_t D, const void* X, int64_t ldx,
                                        const void* gamma, const void* Y, int64_t ldy) {
  return rmsnorm_check(dtype, M, D, X, ldx, gamma, Y, ldy);
}

bigemm_status bigemm_rmsnorm(int32_t dtype, int64_t M, int64_t D, const void* X, int64_t ldx, const void* gamma,
                             void* Y, int64_t ldy, float eps, void* stream) {
  const bigemm_status st = rmsnorm_check(dtype, M, D, X, ldx, gamma, Y, ldy);
  if (st != BIGEMM_OK || M == 0) return st;
  const bigemm_status dv = current_device_supported();
  if (dv != BIGEMM_OK) return dv;
  const hipError_t e = bigemm::launch_rmsnorm(dtype == BIGEMM_BF16, X, ldx, gamma, Y, ldy, M, D, eps,
                                              (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}

bigemm_status bigemm_destroy(bigemm_t h) {
  delete h;
  return BIGEMM_OK;
}

bigemm_status bigemm_get_config(bigemm_t h, int32_t* bm, int32_t* bn, int32_t* bk) {
  if (!h) return BIGEMM_ERR_ARG;
  if (bm) *bm = bigemm::kTileM;
  if (bn) *bn = bigemm::kTileN;
  if (bk) *bk = (h->op.in == bigemm::kInBf16 || h->op.in == bigemm::kInF16) ? bigemm::kTileKBf16 : bigemm::kTileKMx;
  return BIGEMM_OK;
}

bigemm_status bigemm_run(bigemm_t h, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                         const void* W, int64_t ldw, void* Y, int64_t ldy, const void* X_scale,
                         int64_t ldxs, const void* W_scale, int64_t ldws, void* stream) {
  if (!h) return BIGEMM_ERR_ARG;
  if (h->k_chunk > 0) return BIGEMM_ERR_ARG;  // a split-K handle needs bigemm_run_ws
  const bigemm_status st = check(h->op, M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs, W_scale, ldws, h->w_trans);
  if (st != BIGEMM_OK || M == 0) return st;
  const bigemm_status dv = handle_device_current(h);
  if (dv != BIGEMM_OK) return dv;
  const hipError_t e = launch_unsplit(h, M, N, K, X, ldx, W, ldw, Y, ldy, X_scale, ldxs,
                                      W_scale, ldws, (hipStream_t)stream);
  return e == hipSuccess ? BIGEMM_OK : BIGEMM_ERR_DEVICE;
}

}  // extern "C"
