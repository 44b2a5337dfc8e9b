// Drives the C ABI's host-side argument validation over boundary and hostile
// values (sizes up to INT64_MAX, negative sizes, null and misaligned pointers,
// extreme layouts) in a CPU build with the address and undefined-behaviour
// sanitizers: any overflow, out-of-bounds access or invalid shift aborts the
// program. The status of bigemm_check_args is also compared with the
// header's rules restated here in 128-bit arithmetic.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bigemm.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static const int64_t kVals[] = {INT64_MIN, -4096, -1, 0, 1, 7, 8, 12, 15, 16, 31, 32, 48, 64, 100, 127, 128, 129,
                                 160, 4095, 4096, 4099, 4104, (1 << 22) - 8, 1 << 22, (1 << 23) - 8, 1 << 23,
                                 (1 << 24) - 1, 1 << 24, (1 << 26) - 16, INT32_MAX, (int64_t)INT32_MAX + 1,
                                 (int64_t)1 << 40, INT64_MAX / 2, INT64_MAX};
static const int kNV = sizeof(kVals) / sizeof(kVals[0]);
static int64_t pick() { return kVals[next_u64() % kNV]; }
static const uintptr_t kA = (uintptr_t)1 << 20;  // aligned fake device address, never dereferenced
static const void* pick_ptr() {
  switch (next_u64() % 4) {
    case 0: return nullptr;
    case 1: return (const void*)(kA + 2);
    default: return (const void*)kA;
  }
}

typedef __int128 i128;
static bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The header's rules for bigemm_run (W as [K, N]) in 128-bit arithmetic.
static bigemm_status expected(int fam, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, const void* W,
                              int64_t ldw, const void* Y, int64_t ldy, const void* XS, int64_t ldxs,
                              const void* WS, int64_t ldws, int64_t eo) {
  // fam: 0 bf16/fp16, 1 MXFP8, 2 int8
  const i128 es = fam == 0 ? 2 : 1, L = (i128)1 << 31;
  if (M < 0 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return BIGEMM_ERR_ARG;
  if ((i128)((M + 127) / 128) * ((N + 127) / 128) > INT32_MAX) return BIGEMM_ERR_ARG;
  if (fam == 1 && (K % 32 != 0 || N % 16 != 0)) return BIGEMM_ERR_ARG;
  if (fam == 2 && (K % 16 != 0 || N % 16 != 0)) return BIGEMM_ERR_ARG;
  if (ldx < K || ldw < N || ldy < N) return BIGEMM_ERR_ARG;
  if ((i128)ldx * es % 16 != 0 || (i128)ldw * es % 16 != 0 || (i128)ldy * eo % 16 != 0) return BIGEMM_ERR_ARG;
  if (128 * (i128)ldx * es >= L || 128 * (i128)ldw * es >= L || 128 * (i128)ldy * eo >= L) return BIGEMM_ERR_ARG;
  if (fam != 1) {
    if (XS || WS) return BIGEMM_ERR_ARG;
  } else {
    if (ldxs < K / 32 || ldws < N) return BIGEMM_ERR_ARG;
    if (128 * (i128)ldxs >= L || (i128)(K / 32) * ldws >= L) return BIGEMM_ERR_ARG;
  }
  if (M == 0) return BIGEMM_OK;
  if (!X || !W || !Y || !a16(X) || !a16(W) || !a16(Y)) return BIGEMM_ERR_ARG;
  if (fam == 1 && (!XS || !WS)) return BIGEMM_ERR_ARG;
  return BIGEMM_OK;
}

int main() {
  long calls = 0, mismatches = 0;
  const bigemm_desc descs[] = {{BIGEMM_BF16, BIGEMM_BF16, BIGEMM_F32, 0}, {BIGEMM_BF16, BIGEMM_BF16, BIGEMM_BF16, 0},
                               {BIGEMM_F16, BIGEMM_F16, BIGEMM_F32, 0},   {BIGEMM_E4M3, BIGEMM_E4M3, BIGEMM_F32, 32},
                               {BIGEMM_E4M3, BIGEMM_E4M3, BIGEMM_BF16, 32}, {BIGEMM_I8, BIGEMM_I8, BIGEMM_I32, 0},
                               {BIGEMM_BF16, BIGEMM_E4M3, BIGEMM_F32, 0}};
  const int fams[] = {0, 0, 0, 1, 1, 2, -1};
  for (int iter = 0; iter < 300000; ++iter) {
    const int d = (int)(next_u64() % 7);
    const int64_t M = pick(), N = pick(), K = pick(), ldx = pick(), ldw = pick(), ldy = pick();
    const int64_t ldxs = pick(), ldws = pick();
    const void *X = pick_ptr(), *W = pick_ptr(), *Y = pick_ptr();
    const bool scales = (next_u64() & 1) != 0;
    const void* XS = scales ? pick_ptr() : nullptr;
    const void* WS = scales ? pick_ptr() : nullptr;
    const bigemm_status got = bigemm_check_args(&descs[d], M, N, K, X, ldx, W, ldw, Y, ldy, XS, ldxs, WS, ldws);
    const bigemm_status got_wt =
        bigemm_check_args_wt(&descs[d], M, N, K, X, ldx, W, ldw, Y, ldy, XS, ldxs, WS, ldws);
    calls += 2;
    const bigemm_status want = fams[d] < 0 ? BIGEMM_ERR_UNSUPPORTED
                                           : expected(fams[d], M, N, K, X, ldx, W, ldw, Y, ldy, XS, ldxs, WS, ldws,
                                                      descs[d].y_type == BIGEMM_BF16 ? 2 : 4);
    if (got != want) {
      if (mismatches++ < 10)
        fprintf(stderr, "check_args d=%d M=%lld N=%lld K=%lld ldx=%lld ldw=%lld ldy=%lld: got %d want %d\n", d,
                (long long)M, (long long)N, (long long)K, (long long)ldx, (long long)ldw, (long long)ldy, (int)got,
                (int)want);
    }
    if (got_wt < BIGEMM_OK || got_wt > BIGEMM_ERR_UNSUPPORTED) ++mismatches;
    const int32_t kc = (int32_t)pick();
    const uint64_t wsb = (next_u64() & 1) ? UINT64_MAX : (uint64_t)pick();
    const bigemm_status sk =
        bigemm_check_args_split_k(&descs[d], kc, M, N, K, X, ldx, W, ldw, Y, ldy, pick_ptr(), wsb);
    const bigemm_status rn = bigemm_rmsnorm_check_args((int32_t)pick(), M, K, X, ldx, W, Y, ldy);
    calls += 2;
    if (sk < BIGEMM_OK || sk > BIGEMM_ERR_UNSUPPORTED || rn < BIGEMM_OK || rn > BIGEMM_ERR_UNSUPPORTED) ++mismatches;
    bigemm_kv_layout kv = {(int32_t)pick(), (int32_t)pick(), (int32_t)pick(), (int32_t)pick(), (int32_t)pick(),
                           (int32_t)pick()};
    if (next_u64() & 1) kv = {(int32_t)(1 + next_u64() % 16), (next_u64() & 1) ? 64 : 128,
                              (int32_t)(1u << (next_u64() % 13)), (int32_t)pick(), (int32_t)pick(), (int32_t)pick()};
    const int64_t T = pick();
    const int32_t H = (int32_t)pick(), mc = (int32_t)pick();
    uint64_t bytes = 0;
    const bigemm_status ws = bigemm_attn_workspace_size(&kv, T, H, mc, &bytes);
    const bigemm_status pa = bigemm_paged_attention_check_args(&kv, T, H, mc, (int32_t)pick(), X, W, Y,
                                                               (const int32_t*)pick_ptr(), (const int32_t*)pick_ptr(),
                                                               (const int32_t*)pick_ptr(), Y, pick_ptr(), wsb);
    calls += 2;
    if (ws < BIGEMM_OK || ws > BIGEMM_ERR_UNSUPPORTED || pa < BIGEMM_OK || pa > BIGEMM_ERR_UNSUPPORTED) ++mismatches;
    if (ws == BIGEMM_OK && (i128)bytes != (i128)T * H * (((i128)mc + 255) / 256) * (kv.head_dim + 2) * 4) ++mismatches;
  }
  // Null descriptors and handles are rejected, never dereferenced.
  if (bigemm_check_args(nullptr, 1, 8, 8, (void*)kA, 8, (void*)kA, 8, (void*)kA, 8, nullptr, 0, nullptr, 0) !=
          BIGEMM_ERR_ARG ||
      bigemm_run(nullptr, 1, 8, 8, (void*)kA, 8, (void*)kA, 8, (void*)kA, 8, nullptr, 0, nullptr, 0, nullptr) !=
          BIGEMM_ERR_ARG ||
      bigemm_destroy(nullptr) != BIGEMM_OK || bigemm_attn_workspace_size(nullptr, 1, 1, 1, nullptr) != BIGEMM_ERR_ARG)
    ++mismatches;
  for (int s = -2; s < 8; ++s) calls += bigemm_status_str((bigemm_status)s) != nullptr;
  if (mismatches) {
    fprintf(stderr, "%ld mismatches in %ld calls\n", mismatches, calls);
    return 1;
  }
  printf("validators ok: %ld calls\n", calls);
  return 0;
}
