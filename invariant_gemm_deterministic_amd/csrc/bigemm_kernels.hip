// Batch-invariant GEMM kernels for CDNA4 (gfx950).
//
// The method is the one the nondeterminism blog gives in its section on
// batch-invariant matrix multiplication: split the output into 2-D tiles, give
// each tile to one worker that performs the whole K reduction itself, and use
// a single compiled configuration for every shape. The CANN ops-transformer
// issue (background) adds the failure mode to avoid: two kernel classes with
// different K-loop schedules for different rows. So here:
//
//   * one tile shape (128 x 128 outputs) and one MFMA shape per input type,
//     whatever M, N or K;
//   * every output element is produced by one lane of one wave, accumulating in
//     fp32 registers over the K blocks in ascending order, then ascending MFMA
//     steps inside the block — the same chain for interior and edge tiles;
//   * rows >= M, columns >= N and K blocks past K are handled only through
//     addresses: loads use out-of-range buffer offsets (which return zero) and
//     stores use out-of-range offsets (which are dropped). There is no
//     full-tile fast path and no branch on M.
//
// The grid size depends on M (ceil(M/128) * ceil(N/128) workgroups); the
// workgroup -> tile map below only decides placement (which CU and XCD runs a
// tile), never the arithmetic inside a tile.
//
// Data movement: global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging), a ring of LDS buffers (several K blocks in flight), one barrier
// per K block. Operand
// fragments come from LDS with ds_read_b128 (row operand, K contiguous) and
// the transposing ds_read_b64_tr_b16 / ds_read_b64_tr_b8 (the W operand, which
// is N-contiguous in memory). When W is given as [N, K] rows (each kernel's
// kWT flag) its tile is K-contiguous like X's and its fragments are
// ds_read_b128 as well. Both LDS tiles are XOR-swizzled at 16-byte
// granularity so the fragment reads do not collide on LDS banks.
//
// Lane layouts used below (checked with exact small-integer products on the
// device):
//   v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8*(l/32) + 0..7;
//     B lane l holds column l%32, the same k; D register r of lane l is
//     row 8*(r/4) + 4*(l/32) + r%4, column l%32.
//   v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3): lane l holds row (or column)
//     l%32; its bytes 0..15 are k = 16*(l/32) + 0..15 and bytes 16..31 are
//     k = 32 + 16*(l/32) + 0..15; its scale operand is the E8M0 scale of that
//     row (column) for the 32-wide K block l/32. D as above.
//   ds_read_b64_tr_b16: in each 16-lane group, lane i element e is element
//     i%4 of the 8 bytes addressed by lane 4e + i/4.
//   ds_read_b64_tr_b8: in each 16-lane group, lane i byte e is byte i%8 of
//     the 8 bytes addressed by lane 2e + i/8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "bigemm_kernels.h"
#include "bigemm_tilemap.h"

namespace bigemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kThreads = 256;                 // MXFP8 kernel: 4 waves of 64, arranged 2 x 2
constexpr int kTileBytes = 16384;             // one operand tile per stage (both dtypes)
constexpr int kStageBytes = 2 * kTileBytes;   // X tile + W tile
constexpr uint32_t kOob = 0x80000000u;        // buffer offset that is always out of range
constexpr int kNumRecords = 0x7FFFFFFF;       // every in-range offset is below 2^31
constexpr int kRsrcWord3 = 0x00020000;        // raw buffer, 32-bit data format (CDNA)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kNumRecords, kRsrcWord3);
}

// 16-byte-chunk swizzle of a 128-byte-row operand tile (X tiles, and the MXFP8
// W tile): chunk c of row r is stored in slot c ^ swz128(r).
__device__ __forceinline__ int swz_x(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// bf16 W tile rows are 256 bytes (16 chunks).
__device__ __forceinline__ int swz_w16(int k) { return 4 * (k & 3); }
// MXFP8 W tile rows are 128 bytes (8 chunks).
__device__ __forceinline__ int swz_w8(int k) { return k & 7; }

// The pipeline waits are written out explicitly: each thread first waits for
// its own LDS-DMA loads of the stage it is about to read (vmcnt counts them in
// issue order), then the workgroup barrier makes every thread's loads visible.
// A plain __syncthreads() would carry a release fence that waits for every
// outstanding load, including the prefetches that should stay in flight.
// s_waitcnt immediate (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; only vmcnt is constrained here. The builtin (rather than
// inline asm) lets the compiler's own wait insertion see that the wait happened.
#define BIGEMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define BIGEMM_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// binary32 -> bfloat16, round to nearest, ties to even (add half an ulp of the
// 16 dropped bits, plus one when the kept part is odd, then truncate). A NaN
// keeps its sign and top payload bits and gets the quiet bit (bit 6) set.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Store one output element at element index e of the tile-relative buffer
// (out-of-range e is the kOob sentinel and is dropped): the raw 32-bit
// accumulator (fp32 or int32), or its bf16 rounding. kStream: a final output,
// which no kernel of the call reads again, is stored non-temporal (nt), so
// that its lines do not displace in the XCD's L2 the X and W panel lines the
// tiles still running there are reading (the same values are stored either
// way). Split-K chunk sums, which the merge reads next, are stored plainly.
constexpr int kCachePolicyNt = 2;  // the nt bit of the buffer instructions' cache-policy operand
template <bool kOutBf16, bool kStream = true>
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t ry, bool ok, uint32_t e, uint32_t bits) {
  constexpr int aux = kStream ? kCachePolicyNt : 0;
  if (kOutBf16) {
    const uint32_t o = ok ? e * 2 : kOob;
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(bits), ry, o, 0, aux);
  } else {
    const uint32_t o = ok ? e * 4 : kOob;
    __builtin_amdgcn_raw_buffer_store_b32(bits, ry, o, 0, aux);
  }
}

// 32x32x16 MFMA on 16-bit inputs: bf16 or fp16 bit patterns (8 per lane).
template <bool kF16>
__device__ __forceinline__ f32x16 mfma_16bit(i32x4 a, i32x4 b, f32x16 c) {
  if (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// ------------------------------------------------------------------------ bf16
//
// K block 64, MFMA 32x32x16 bf16, fp32 accumulate. 512 threads: 8 waves in a
// 2 x 4 grid, each wave owning a 64 x 32 block of the 128 x 128 output tile
// (two 32 x 32 MFMA fragments stacked along M). Two waves share each SIMD,
// so one can issue while the other waits on LDS. Per stage: X tile 128 x 64
// bf16 (rows of 128 B), W tile 64 x 128 bf16 (rows of 256 B); kStagesBf16
// stages in a ring, kStagesBf16 - 1 K blocks in flight.
constexpr int kBkBf16 = 64;
constexpr int kThreadsBf16 = 512;
#ifndef BIGEMM_BF16_STAGES
#define BIGEMM_BF16_STAGES 4
#endif
constexpr int kStagesBf16 = BIGEMM_BF16_STAGES;
static_assert(kStagesBf16 >= 3 && kStagesBf16 <= 5, "LDS holds 3 to 5 stages of 32 KiB");
// K-loop unroll of the bf16 kernel (steps per loop iteration).
constexpr int kUnrollBf16 = 8 * kStagesBf16;

// A prefetch workgroup of the bf16 / fp16 kernel (prefetch_grid). The
// prefetch workgroups of an XCD share out the K blocks of the distinct X
// panels (tile rows) and W panels (tile columns) of the XCD's tiles
// (prefetch_units): for each of its panel blocks a workgroup reads one dword of
// every 128-byte line the tiles' own loads of that block touch, so that the
// line is in the XCD's L2 when a tile's workgroup asks for it; the dwords go to
// a scratch corner of its LDS and are never read. Waves 0-3 take the X panel
// blocks, lane slot q = tid: row q / 2 (the block's 128 bytes of a row start
// 16-byte aligned, so chunks 0 and 7 cover its one or two lines). Waves 4-7
// take the W panel blocks: rows (q - 256) / 3 of a [K, N] panel (256 bytes of
// columns: chunks 0, 8 and 15 cover two or three lines), or rows (q - 256) / 2
// of a W^T panel (as X). A chunk is touched only where the tiles' own loads
// read it (row, column and K inside the matrix), so every read stays inside
// the bytes the tiles read. One load per wave per panel block.
//
// Pacing: block kb is requested no earlier than (kb - kPrefetchLead) block
// times after the workgroup started (s_memrealtime, 100 MHz), a block time
// being roughly what a tile's workgroup takes per block when its lines come
// from L2 (prefetch_ticks, by the rows the tile multiplies). Running further
// ahead only evicts lines from the L2 before they are used. The wait is on
// the clock alone, so it always ends.
constexpr int kPrefetchLead = 16;
__device__ __forceinline__ int64_t prefetch_ticks(int rows_valid) {
  return rows_valid <= 32 ? 17 : (rows_valid <= 64 ? 21 : 33);
}

// The units of this prefetch workgroup's XCD (the rule of prefetch_units):
// lane i < cx holds the XCD's i-th tile (tmi, tni); bit i of rows (cols) is
// set where that tile is the first of the XCD with its tile row (column).
struct PrefetchUnits {
  int tmi, tni, tm_min;
  uint64_t rows, cols;
};
__device__ __forceinline__ bool prefetch_lane_units(int tiles_m, int tiles_n, int lane, PrefetchUnits& u) {
  const int ntiles = tiles_m * tiles_n;
  const int xcd = blockIdx.x % kXcds;
  const int cx = xcd_tiles(xcd, ntiles);  // at most kPrefetchMaxXcdTiles (prefetch_grid)
  if (cx == 0) return false;
  u.tmi = 0;
  u.tni = 0;
  if (lane < cx) tile_of(xcd + kXcds * lane, ntiles, tiles_m, tiles_n, u.tmi, u.tni);
  bool first_row = lane < cx, first_col = lane < cx;
  u.tm_min = tiles_m;
  for (int j = 0; j < cx; ++j) {
    const int tmj = __builtin_amdgcn_readlane(u.tmi, j), tnj = __builtin_amdgcn_readlane(u.tni, j);
    if (j < lane) {
      first_row = first_row && tmj != u.tmi;
      first_col = first_col && tnj != u.tni;
    }
    u.tm_min = tmj < u.tm_min ? tmj : u.tm_min;
  }
  u.rows = __builtin_amdgcn_ballot_w64(first_row);
  u.cols = __builtin_amdgcn_ballot_w64(first_col);
  return true;
}

// This prefetch workgroup's items of one kind: the K blocks kb of the units in
// `units` (a mask of u's lanes), item kb * (number of units) + unit, dealt
// round-robin over the XCD's prefetch workgroups. For each it waits until
// (kb - kPrefetchLead) * ticks(tm) ticks (s_memrealtime, 100 MHz) after t0,
// then calls touch(kb, tm, tn, j), j counting this workgroup's items. The wait
// is on the clock alone and always ends.
template <class Ticks, class Touch>
__device__ __forceinline__ void prefetch_walk(const PrefetchUnits& u, uint64_t units, int ntiles, int nkb,
                                              uint64_t t0, Ticks ticks, Touch touch) {
  int h, nh;
  prefetch_helper(blockIdx.x, gridDim.x, ntiles, h, nh);
  const int nu = __builtin_popcountll(units);
  int j = 0;
  for (int w = h; w < nkb * nu; w += nh, ++j) {
    const int kb = w / nu;
    uint64_t rest = units;  // the (w % nu)-th set bit: the lane holding this unit
    for (int q = w - kb * nu; q > 0; --q) rest &= rest - 1;
    const int ul = __builtin_ctzll(rest);
    const int tm = __builtin_amdgcn_readlane(u.tmi, ul), tn = __builtin_amdgcn_readlane(u.tni, ul);
    const int64_t due = (int64_t)(kb - kPrefetchLead) * ticks(tm);
    while ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) < due) __builtin_amdgcn_s_sleep(2);
    touch(kb, tm, tn, j);
  }
  BIGEMM_WAIT_VMCNT(0);  // no LDS-DMA load may outlive the workgroup
}

template <bool kWT>
__device__ __forceinline__ void bf16_prefetch(const uint16_t* X, const uint16_t* W, int M, int N, int K,
                                              int64_t ldx, int64_t ldw, int tiles_m, int tiles_n, uint8_t* scratch,
                                              int tid) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  PrefetchUnits u;
  if (!prefetch_lane_units(tiles_m, tiles_n, tid & 63, u)) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const bool isx = wave < 4;  // waves 0-3: the X panels' lines, waves 4-7: the W panels'
  int r, c;   // row of the panel block, 8-element chunk of that row touched by this lane
  if (isx || kWT) {
    r = (tid & 255) >> 1;
    c = (tid & 1) ? 7 : 0;
  } else {
    const int q = tid - 256;
    r = q / 3;
    c = q % 3 == 0 ? 0 : (q % 3 == 1 ? 8 : 15);
  }
  const int nkb = (K + kBkBf16 - 1) / kBkBf16;
  // A row's X panel at that row's tiles' pace; a W panel at the pace of the
  // XCD's fullest tile row, the slowest tiles that read it.
  const int64_t col_ticks = prefetch_ticks(min(128, M - u.tm_min * 128));
  auto ticks = [&](int tm) { return isx ? prefetch_ticks(min(128, M - tm * 128)) : col_ticks; };
  auto touch = [&](int kb, int tm, int tn, int j) {
    const int rows_valid = min(128, M - tm * 128), cols_valid = min(128, N - tn * 128);
    BIGEMM_WAIT_VMCNT(3);  // at most four items' loads in flight (the four LDS corners below)
    const int k0 = kb * kBkBf16;
    uint32_t o = kOob;
    __amdgpu_buffer_rsrc_t rs;
    if (isx) {
      rs = make_rsrc(X + (int64_t)tm * 128 * ldx + k0);
      if (r < rows_valid && k0 + c * 8 < K) o = (uint32_t)((r * ldx + c * 8) * 2);
    } else if constexpr (kWT) {   // W^T panel: 128 rows of K values, touched like X's
      rs = make_rsrc(W + (int64_t)tn * 128 * ldw + k0);
      if (r < cols_valid && k0 + c * 8 < K) o = (uint32_t)((r * ldw + c * 8) * 2);
    } else {                      // W panel: the block's 64 rows of 128 columns
      rs = make_rsrc(W + tn * 128 + (int64_t)k0 * ldw);
      if (r < kBkBf16 && c * 8 < cols_valid && k0 + r < K) o = (uint32_t)((r * ldw + c * 8) * 2);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS(void, scratch + (j & 3) * 2048 + wave * 256), 4, o, 0, 0, 0);
  };
  prefetch_walk(u, isx ? u.rows : u.cols, tiles_m * tiles_n, nkb, t0, ticks, touch);
}

// kSplit: the opt-in split-K variant. The grid is (chunk, tile) pairs; the
// workgroup runs the same chain over the K blocks of its chunk only
// (kb_per_split blocks) and stores the fp32 chunk sum at Y + chunk * split_stride.
// kWT: W is given as its transpose, an [N, K] row-major array (the layout of a
// linear layer's weight), leading dimension ldw >= K. Its tile is then staged
// like the X tile (128 rows of K-contiguous bytes) and the B fragments are
// plain 16-byte reads; the MFMA chain and its operands are the same as for
// W [K, N], so the output bytes are too.
// kKTail: K is not a multiple of 8 (chosen from K alone). The 16-byte chunk of
// an X row (and of a W^T row) that holds the last K values also holds up to 7
// values past K, from the row's padding. W rows past K load as zero, but a
// padding value may be an infinity or a NaN, and 0 * NaN is NaN, so those
// fragment elements are set to +0 before they reach the MFMA. Every element
// then accumulates the same products as with a zero-filled tail.
template <bool kF16, bool kOutBf16, bool kSplit, bool kWT = false, bool kKTail = false>
__global__ __launch_bounds__(kThreadsBf16, 1)
void bigemm_bf16_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                        void* __restrict__ Y, int M, int N, int K,
                        int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n,
                        int kb_per_split, int64_t split_stride) {
  static_assert(!(kSplit && kOutBf16), "chunk sums are stored in fp32");
  // One LDS array per pipeline stage: distinct objects let the compiler see
  // that reads of one stage do not depend on the loads in flight into another.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[kStagesBf16 > 3 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t stage4[kStagesBf16 > 4 ? kStageBytes : 16];
  uint8_t* const stg[5] = {stage0, stage1, stage2, stage3, stage4};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if constexpr (!kSplit) {
    if (__builtin_expect((int)blockIdx.x >= tiles_m * tiles_n, 0)) {  // a prefetch workgroup
      bf16_prefetch<kWT>(X, W, M, N, K, ldx, ldw, tiles_m, tiles_n, stage0, tid);
      return;
    }
  }
  int tm, tn;
  int kb_first = 0;                               // first K block of this workgroup
  int nkb = (K + kBkBf16 - 1) / kBkBf16;          // K blocks this workgroup accumulates
  if (kSplit) {
    const int ntiles = tiles_m * tiles_n;
    const int t = xcd_order(blockIdx.x, gridDim.x);
    const int chunk = t / ntiles;
    tile_coords(t - chunk * ntiles, tiles_m, tiles_n, tm, tn);
    kb_first = chunk * kb_per_split;
    nkb = min(nkb - kb_first, kb_per_split);
    Y = (float*)Y + chunk * split_stride;
  } else {
    tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  }
  const int row0 = tm * 128;
  const int col0 = tn * 128;
  const int rows_valid = min(128, M - row0);
  const int cols_valid = min(128, N - col0);

  // Load assignment: chunk p = i*512 + tid of each tile (i = 0, 1). With
  // buffer_load ... lds a wave's 64 lanes fill 1 KiB of LDS contiguously, so
  // the LDS slot is fixed by p and the swizzle is applied to the global side.
  // xk/wk: the K offset of the chunk inside the block, or a huge value when
  // the chunk's row (column) is outside the matrix, so that one compare with
  // the K remaining in the block decides in-range.
  uint32_t xoff[2], woff[2];
  int xk[2], wk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = i * kThreadsBf16 + tid;
    const int r = p >> 3, s = p & 7, c = s ^ swz_x(r);
    xoff[i] = (uint32_t)((r * ldx + c * 8) * 2);
    xk[i] = r < rows_valid ? c * 8 : 0x7FFFFFFF;
    if constexpr (kWT) {  // W^T tile: 128 columns (rows of W^T) of 128 bytes, swizzled like X
      woff[i] = (uint32_t)((r * ldw + c * 8) * 2);
      wk[i] = r < cols_valid ? c * 8 : 0x7FFFFFFF;
    } else {
      const int kr = p >> 4, sw = p & 15, cw = sw ^ swz_w16(kr);
      woff[i] = (uint32_t)((kr * ldw + cw * 8) * 2);
      wk[i] = cw * 8 < cols_valid ? kr : 0x7FFFFFFF;
    }
  }
  const uint16_t* Xt = X + (int64_t)row0 * ldx + (int64_t)kb_first * kBkBf16;
  const uint16_t* Wt = kWT ? W + (int64_t)col0 * ldw + (int64_t)kb_first * kBkBf16
                           : W + col0 + (int64_t)kb_first * kBkBf16 * ldw;
  const int Kr = K - kb_first * kBkBf16;           // K remaining from this workgroup's first block

  // Issue the 4 LDS-DMA loads of K block kb into `stage`. A block past the
  // end (kb >= nkb) is still issued, entirely out of range: it loads zeros
  // into a stage nobody reads again, and keeps every pipeline step the same
  // instruction sequence (so the number of loads in flight is fixed).
  // kNx: how many of the wave's two X loads are issued. Load i covers tile rows
  // 64 i + 8 wave .. + 7; the loop leaves out those whose rows are all past M
  // (always the last ones). Their LDS rows keep the zeros the prologue's
  // out-of-range loads wrote into every stage, so the fragments read the same
  // values as before; the wait counts follow the wave's number of loads.
  const int wave_s = __builtin_amdgcn_readfirstlane(tid) >> 6;  // the LDS-DMA bases (M0) stay scalar
  auto issue = [&](auto nx, int kb, uint8_t* stage) {
    constexpr int kNx = decltype(nx)::value;
    const bool live = kb < nkb;
    const int k0 = live ? kb * kBkBf16 : 0;
    const int kleft = live ? Kr - k0 : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xt + k0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(kWT ? Wt + k0 : Wt + (int64_t)k0 * ldw);
#pragma unroll
    for (int i = 0; i < kNx; ++i) {
      const uint32_t o = xk[i] < kleft ? xoff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, LDS(void, stage + i * 8192 + wave_s * 1024), 16, o, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = wk[i] < kleft ? woff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, LDS(void, stage + kTileBytes + i * 8192 + wave_s * 1024), 16, o,
                                                0, 0, 0);
    }
  };

  // Fragment addresses (bytes inside a stage): A for the wave's two 32-row
  // fragments, B (transposing reads) for its 32 columns, per 16-wide K step kk.
  const int wm = wave >> 2, wn = wave & 3;
  int a_addr[2][4];     // [fm][kk]
  int b_addr[4][2];     // [kk][half]
  int bt_addr[4];       // kWT: [kk], the 16 bytes of the lane's column
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int r = wm * 64 + f * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      a_addr[f][kk] = r * 128 + ((c ^ swz_x(r)) << 4);
    }
    if constexpr (kWT) {
      const int n = wn * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      bt_addr[kk] = kTileBytes + n * 128 + ((c ^ swz_x(n)) << 4);
    }
    const int g = lane >> 4, j = lane & 15;
    const int col = wn * 32 + (g & 1) * 16 + (j & 3) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kr = kk * 16 + (g >> 1) * 8 + h * 4 + (j >> 2);
      b_addr[kk][h] = kTileBytes + kr * 256 + (((col >> 3) ^ swz_w16(kr)) << 4) + (col & 7) * 2;
    }
  }

  f32x16 acc[2] = {f32x16{}, f32x16{}};

  // One K block: wait for this stage (kStagesBf16 - 2 younger blocks, 2 + kNx
  // loads each, may stay in flight), refill the stage read in the previous block,
  // then run the MFMA chain on this stage: kk ascending, the wave's first kNf
  // fragments per kk (kNf < 2 only where the tile's rows past M cover whole
  // 32-row fragments, which are then neither read nor multiplied; every
  // multiplied fragment runs the same chain as in a full tile).
  auto step = [&](auto nf, auto nx, int kb, const uint8_t* st, uint8_t* refill) {
    constexpr int kNf = decltype(nf)::value;
    constexpr int kNx = decltype(nx)::value;
    BIGEMM_WAIT_VMCNT((2 + kNx) * (kStagesBf16 - 2));
    BIGEMM_BARRIER();
    issue(nx, kb + kStagesBf16 - 1, refill);
    if constexpr (kNf == 0) return;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // kKTail: keep the fragment's K values below K. The lane holds the 8
      // values from K offset kk*16 + 8*(lane/32) of this block; dword d holds
      // values 2d (low half) and 2d + 1. Full blocks keep everything.
      i32x4 kmask = i32x4{-1, -1, -1, -1};
      if constexpr (kKTail) {
        const int n = Kr - kb * kBkBf16 - (kk * 16 + 8 * (lane >> 5));  // values of the 8 below K
#pragma unroll
        for (int d = 0; d < 4; ++d) kmask[d] = n >= 2 * d + 2 ? -1 : (n == 2 * d + 1 ? 0xFFFF : 0);
      }
      i32x4 a[2];
#pragma unroll
      for (int f = 0; f < kNf; ++f) {
        a[f] = *LDS(const i32x4, st + a_addr[f][kk]);
        if constexpr (kKTail) a[f] &= kmask;
      }
      i32x4 b;
      if constexpr (kWT) {
        b = *LDS(const i32x4, st + bt_addr[kk]);
        if constexpr (kKTail) b &= kmask;
      } else {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS(i16x4, st + b_addr[kk][0]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS(i16x4, st + b_addr[kk][1]));
        const i32x2 lo2 = __builtin_bit_cast(i32x2, lo), hi2 = __builtin_bit_cast(i32x2, hi);
        b = i32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      }
#pragma unroll
      for (int f = 0; f < kNf; ++f) acc[f] = mfma_16bit<kF16>(a[f], b, acc[f]);
    }
  };

  // Prologue: a dummy (entirely out-of-range) fill of the last stage, then
  // blocks 0 to kStagesBf16 - 2, all with every load (zeros in the rows past M
  // of every stage). The dummy makes the loads in flight at the loop head
  // target the stages in the same order on entry as on every later iteration.
  // A variant issuing fewer loads per block than the prologue only waits for
  // more than it needs on its first steps.
  issue(std::integral_constant<int, 2>{}, nkb, stg[kStagesBf16 - 1]);
#pragma unroll
  for (int s = 0; s < kStagesBf16 - 1; ++s) issue(std::integral_constant<int, 2>{}, s, stg[s]);
  // Unrolled by kUnrollBf16 steps (a multiple of kStagesBf16) so that each
  // stage is a fixed LDS object in every step. The compiler cannot track which
  // stage the loads in flight target across the loop back-edge, and waits for
  // all of them (vmcnt(0)) before the first step of an iteration; 32 steps
  // make that drain rare (once for K = 2048, twice for K = 4096). The body is
  // about 18 KB of code, inside the instruction cache.
  auto kloop = [&](auto nf, auto nx) {
    for (int kb = 0;;) {
      bool done = false;
#pragma unroll
      for (int u = 0; u < kUnrollBf16; ++u) {
        step(nf, nx, kb, stg[u % kStagesBf16], stg[(u + kStagesBf16 - 1) % kStagesBf16]);
        if (++kb == nkb) {
          done = true;
          break;
        }
      }
      if (done) break;
    }
  };
  // Per wave (uniform: the wave index is read as a scalar): nf fragments hold
  // a row below M, nx of its X loads do. Every wave meets the same barriers;
  // the combinations below are the only ones that occur, and any other would
  // run the full variant, which is correct for every tile.
  const int wave_u = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const int wrow0 = (wave_u >> 2) * 64;
  const int nf = (rows_valid > wrow0) + (rows_valid > wrow0 + 32);
  const int nx = (wave_u * 8 < rows_valid) + (64 + wave_u * 8 < rows_valid);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  const int v = nf * 3 + nx;
  if (__builtin_expect(v == 8 || (v != 7 && v != 4 && v != 3 && v != 1 && v != 0), 1)) {
    kloop(I2{}, I2{});  // full tiles (and any other count: all loads, both fragments)
  } else if (v == 7) {
    kloop(I2{}, I1{});
  } else if (v == 4) {
    kloop(I1{}, I1{});
  } else if (v == 3) {
    kloop(I1{}, I0{});
  } else if (v == 1) {
    kloop(I0{}, I1{});
  } else {
    kloop(I0{}, I0{});
  }
  BIGEMM_WAIT_VMCNT(0);  // no LDS-DMA load may outlive the workgroup

  // Epilogue: plain stores (fp32, or its bf16 rounding), masked through the
  // buffer range check. Fragments never multiplied hold only rows past M.
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc((uint8_t*)Y + ((int64_t)row0 * ldy + col0) * (kOutBf16 ? 2 : 4));
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 64 + f * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const int cl = wn * 32 + (lane & 31);
      // Copy the element out first: bit-casting an ext_vector element
      // expression directly reads element 0 with this compiler.
      const float v = acc[f][r];
      store_out<kOutBf16, !kSplit>(ry, rl < rows_valid && cl < cols_valid, (uint32_t)(rl * ldy + cl),
                                   __builtin_bit_cast(uint32_t, v));
    }
}

// ----------------------------------------------------------------------- MXFP8
//
// K block 128 (four 32-wide scale blocks), MFMA 32x32x64 E4M3 with E8M0 scales
// applied inside the instruction, fp32 accumulate. Per stage: X tile 128 x 128
// bytes, W tile 128 x 128 bytes (both rows of 128 B).
constexpr int kBkMx = 128;

// A prefetch workgroup of the MXFP8 and int8 kernels (prefetch_grid; 256
// threads, K blocks of 128 one-byte values, so 128 bytes of each panel row per
// block): as in bf16_prefetch, the XCD's prefetch workgroups share out the K
// blocks of its distinct X and W panels. Waves 0-1 take the X panel blocks,
// waves 2-3 the W panel blocks, two loads per wave and panel block: lane slot
// q = 64 (2 (wave & 1) + s) + lane for s = 0, 1 touches row q / 2 at chunk 0
// or 7 of its 128 bytes (one or two lines). A [K, N] W panel's rows are the
// block's 128 K rows of the tile's 128 columns, a W^T panel's the tile's 128
// columns of the block's 128 K values. Only bytes the tiles' own loads read are
// touched. kScales (MXFP8): a W panel block also touches its W scales, the
// block's 4 scale rows of the tile's 128 columns ([K/32, N]: wave 2, lanes
// 0-7, chunks 0 and 7 of each row's 128 bytes) or the 4 scale bytes of each of
// the tile's 128 columns ([N, K/32]: waves 2-3, one lane per column). The X
// scales (one row's bytes of 32 blocks share a line) are not touched.
__device__ __forceinline__ int64_t prefetch_ticks_u8(int rows_valid) {
  return rows_valid <= 32 ? 22 : (rows_valid <= 64 ? 34 : 44);
}
template <bool kWT, bool kScales>
__device__ __forceinline__ void u8_prefetch(const uint8_t* X, const uint8_t* W, const uint8_t* WS, int M, int N,
                                            int K, int64_t ldx, int64_t ldw, int64_t ldws, int tiles_m, int tiles_n,
                                            uint8_t* scratch, int tid) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  PrefetchUnits u;
  if (!prefetch_lane_units(tiles_m, tiles_n, tid & 63, u)) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const bool isx = wave < 2;  // waves 0-1: the X panels' lines, waves 2-3: the W panels'
  const int nkb = (K + kBkMx - 1) / kBkMx;
  const int64_t col_ticks = prefetch_ticks_u8(min(128, M - u.tm_min * 128));
  auto ticks = [&](int tm) { return isx ? prefetch_ticks_u8(min(128, M - tm * 128)) : col_ticks; };
  auto touch = [&](int kb, int tm, int tn, int j) {
    const int rows_valid = min(128, M - tm * 128), cols_valid = min(128, N - tn * 128);
    BIGEMM_WAIT_VMCNT(6);  // at most four items' loads (two each) in flight: the four LDS corners below
    const int k0 = kb * kBkMx;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(isx ? X + (int64_t)tm * 128 * ldx + k0
                                                     : (kWT ? W + (int64_t)tn * 128 * ldw + k0
                                                            : W + tn * 128 + (int64_t)k0 * ldw));
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int q = 64 * (2 * (wave & 1) + s2) + (tid & 63);
      const int r = q >> 1, c = (q & 1) ? 7 : 0;
      uint32_t o = kOob;
      if (isx) {
        if (r < rows_valid && k0 + c * 16 < K) o = (uint32_t)(r * ldx + c * 16);
      } else if (kWT) {
        if (r < cols_valid && k0 + c * 16 < K) o = (uint32_t)(r * ldw + c * 16);
      } else {
        if (k0 + r < K && c * 16 < cols_valid) o = (uint32_t)(r * ldw + c * 16);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS(void, scratch + (j & 3) * 2048 + wave * 512 + s2 * 256), 4,
                                                o, 0, 0, 0);
    }
    if constexpr (kScales) {
      if (!isx && (kWT || wave == 2)) {
        const int lane = tid & 63, nsb = K / 32;
        uint32_t o = kOob;
        __amdgpu_buffer_rsrc_t rss;
        if constexpr (kWT) {   // W_scale [N, K/32]: column 64 (wave - 2) + lane, bytes 4 kb .. 4 kb + 3
          const int r = 64 * (wave - 2) + lane;
          rss = make_rsrc(WS + (int64_t)tn * 128 * ldws);
          if (r < cols_valid && 4 * kb < nsb) o = (uint32_t)(r * ldws + 4 * kb);
        } else {               // W_scale [K/32, N]: scale row 4 kb + lane / 2, chunk 0 or 7 of the tile's columns
          const int sr = 4 * kb + (lane >> 1), c = (lane & 1) ? 7 : 0;
          rss = make_rsrc(WS + tn * 128);
          if (lane < 8 && sr < nsb && c * 16 < cols_valid) o = (uint32_t)(sr * ldws + c * 16);
        }
        // one byte (the first scale byte the tiles read there): never past a scale row
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, LDS(void, scratch + 8192 + (j & 3) * 512 + (wave - 2) * 256), 1,
                                                  o, 0, 0, 0);
      }
    }
  };
  prefetch_walk(u, isx ? u.rows : u.cols, tiles_m * tiles_n, nkb, t0, ticks, touch);
}
// Staged scales: the scale bytes of kScaleGroup consecutive K blocks are
// moved to LDS by DMA, once per workgroup (X: 128 rows x 4 kScaleGroup bytes;
// W: 4 kScaleGroup scale rows x 128 bytes, whole lines), into one of two LDS
// buffers, one group ahead, instead of per-lane loads repeated by the waves
// that share a row or column.
#ifndef BIGEMM_MX_SCALE_GROUP
#define BIGEMM_MX_SCALE_GROUP 4
#endif
constexpr int kScaleGroup = BIGEMM_MX_SCALE_GROUP;
static_assert(kScaleGroup == 4 || kScaleGroup == 8, "scale groups of 4 or 8 K blocks");
constexpr int kScaleBufBytes = 128 * 4 * kScaleGroup;  // one operand's scales of one group
#ifndef BIGEMM_MX_STAGES
#define BIGEMM_MX_STAGES 3
#endif
constexpr int kStagesMx = BIGEMM_MX_STAGES;
static_assert(kStagesMx >= 3 && kStagesMx <= 4, "LDS holds 3 or 4 stages of 32 KiB");

// kWT: W is given as its transpose, [N, K] rows with leading dimension
// ldw >= K, and W_scale as [N, K/32] with ldws >= K/32 (the layout X and
// X_scale have). W's tile, fragments and scales are then handled exactly like
// X's; the MFMA operands and scales are the same as for W [K, N].
template <bool kStaged, bool kOutBf16, bool kWT = false>
__global__ __launch_bounds__(kThreads, 1)
void bigemm_mxfp8_kernel(const uint8_t* __restrict__ X, const uint8_t* __restrict__ W,
                         void* __restrict__ Y, const uint8_t* __restrict__ XS,
                         const uint8_t* __restrict__ WS, int M, int N, int K,
                         int64_t ldx, int64_t ldw, int64_t ldy, int64_t ldxs, int64_t ldws,
                         int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[kStagesMx > 3 ? kStageBytes : 16];
  // Staged scales: two buffers (separate objects, so the compiler can tell the
  // DMA into one from reads of the other), each one group of kScaleGroup K
  // blocks: X scales [128 rows][4 * kScaleGroup bytes] then W scales
  // [4 * kScaleGroup rows][128 columns].
  __shared__ __attribute__((aligned(1024))) uint8_t scales0[kStaged ? 2 * kScaleBufBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t scales1[kStaged ? 2 * kScaleBufBytes : 16];
  uint8_t* const stg[4] = {stage0, stage1, stage2, stage3};
  uint8_t* const scl[2] = {scales0, scales1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (__builtin_expect((int)blockIdx.x >= tiles_m * tiles_n, 0)) {  // a prefetch workgroup
    u8_prefetch<kWT, true>(X, W, WS, M, N, K, ldx, ldw, ldws, tiles_m, tiles_n, stage0, tid);
    return;
  }
  int tm, tn;
  tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * 128;
  const int col0 = tn * 128;
  const int rows_valid = min(128, M - row0);
  const int cols_valid = min(128, N - col0);
  const int nkb = (K + kBkMx - 1) / kBkMx;
  const int nsb = K / 32;  // scale blocks along K

  uint32_t xoff[4], woff[4];
  int xk[4], wk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = i * kThreads + tid;
    const int r = p >> 3, s = p & 7, c = s ^ swz_x(r);
    xoff[i] = (uint32_t)(r * ldx + c * 16);
    xk[i] = r < rows_valid ? c * 16 : 0x7FFFFFFF;
    if constexpr (kWT) {  // W^T tile: rows of W^T (output columns), swizzled like X
      woff[i] = (uint32_t)(r * ldw + c * 16);
      wk[i] = r < cols_valid ? c * 16 : 0x7FFFFFFF;
    } else {
      const int kr = p >> 3, cw = s ^ swz_w8(kr);
      woff[i] = (uint32_t)(kr * ldw + cw * 16);
      wk[i] = cw * 16 < cols_valid ? kr : 0x7FFFFFFF;
    }
  }
  const uint8_t* Xt = X + (int64_t)row0 * ldx;
  const uint8_t* Wt = kWT ? W + (int64_t)col0 * ldw : W + col0;

  // The 8 LDS-DMA loads of K block kb into `stage` (a block past the end is
  // issued entirely out of range, as in the bf16 kernel). kNx: how many of the
  // wave's four X loads are issued. Load i covers tile rows 32 i + 8 wave .. + 7;
  // the loop leaves out those whose rows are all past M (always the last ones).
  // Their LDS rows keep the zeros the prologue's out-of-range loads wrote into
  // every stage; the wait counts follow the wave's number of loads.
  auto issue = [&](auto nx, int kb, uint8_t* stage) {
    constexpr int kNx = decltype(nx)::value;
    const bool live = kb < nkb;
    const int k0 = live ? kb * kBkMx : 0;
    const int kleft = live ? K - k0 : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xt + k0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(kWT ? Wt + k0 : Wt + (int64_t)k0 * ldw);
    uint8_t* sx = stage;
    uint8_t* sw = stage + kTileBytes;
#pragma unroll
    for (int i = 0; i < kNx; ++i) {
      const uint32_t o = xk[i] < kleft ? xoff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, LDS(void, sx + i * 4096 + wave * 1024), 16, o, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = wk[i] < kleft ? woff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, LDS(void, sw + i * 4096 + wave * 1024), 16, o, 0, 0, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5;   // which 16-wide K quarter of a 64-wide MFMA step this lane holds
  // A fragment: two 16-byte reads per (fm, kk): k = kk*64 + g*16 and kk*64 + 32 + g*16
  int a_addr[2][2][2];   // [fm][kk][half]
  // B fragment: four 8-byte transposing reads per (fn, kk); for W^T two
  // 16-byte reads addressed like A's (bt_addr)
  int b_addr[2][2][4];   // [fn][kk][read]
  int bt_addr[2][2][2];  // [fn][kk][half]
#pragma unroll
  for (int f = 0; f < 2; ++f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r = wm * 64 + f * 32 + (lane & 31);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = kk * 4 + h * 2 + g;
        a_addr[f][kk][h] = r * 128 + ((c ^ swz_x(r)) << 4);
      }
      if constexpr (kWT) {
        const int n = wn * 64 + f * 32 + (lane & 31);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = kk * 4 + h * 2 + g;
          bt_addr[f][kk][h] = kTileBytes + n * 128 + ((c ^ swz_x(n)) << 4);
        }
      }
      const int G = lane >> 4, j = lane & 15;
      const int col = wn * 64 + f * 32 + (G & 1) * 16 + (j & 1) * 8;
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) {
        const int kr = kk * 64 + (rd >> 1) * 32 + (G >> 1) * 16 + (rd & 1) * 8 + (j >> 1);
        b_addr[f][kk][rd] = kTileBytes + kr * 128 + (((col >> 4) ^ swz_w8(kr)) << 4) + (col & 15);
      }
    }
  }

  // Scale sources: lane holds the scale of its row (column) for K block
  // kb*4 + kk*2 + g. Out-of-range rows, columns or K blocks read as 0 (2^-127,
  // multiplying zero data).
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(XS + (int64_t)row0 * ldxs);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(kWT ? WS + (int64_t)col0 * ldws : WS + col0);
  // xs_base/ws_base: the lane's offset for K block 0; xs_lim/ws_lim: the
  // number of K blocks it may read (0 for rows/columns outside the matrix).
  uint32_t xs_base[2], ws_base[2];
  int xs_lim[2], ws_lim[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int r = wm * 64 + f * 32 + (lane & 31);
    xs_base[f] = (uint32_t)(r * ldxs);
    xs_lim[f] = r < rows_valid ? nsb : 0;
    const int c = wn * 64 + f * 32 + (lane & 31);
    ws_base[f] = kWT ? (uint32_t)(c * ldws) : (uint32_t)c;
    ws_lim[f] = c < cols_valid ? nsb : 0;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // W scales of one K block, [fragment][MFMA step]: one byte per lane and
  // step (32 columns of two scale rows per load). Blocks past K read as out of
  // range (zero).
  auto load_wscales = [&](int kb, int (&sb)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int blk = kb * 4 + kk * 2 + g;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint32_t ob = blk < ws_lim[f] ? ws_base[f] + (uint32_t)(kWT ? blk : blk * ldws) : kOob;
        sb[f][kk] = __builtin_amdgcn_raw_buffer_load_b8(rws, ob, 0, 0);
      }
    }
  };
  // X scales, byte path: one byte per lane, fragment and step, for the first
  // kNf fragments.
  auto load_xscales = [&](auto nf, int kb, int (&sa)[2][2]) {
    constexpr int kNf = decltype(nf)::value;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int blk = kb * 4 + kk * 2 + g;
#pragma unroll
      for (int f = 0; f < kNf; ++f) {
        const uint32_t oa = blk < xs_lim[f] ? xs_base[f] + (uint32_t)blk : kOob;
        sa[f][kk] = __builtin_amdgcn_raw_buffer_load_b8(rxs, oa, 0, 0);
      }
    }
  };
  // Staged path: the scales of group q (K blocks kScaleGroup q ..) into buffer
  // buf, as 1 KiB DMA loads j = 0 .. 2 kXLoads - 1 spread over the waves. X
  // load j: chunk p = 64 j + l is 16 bytes of row p / (kScaleGroup / 4) (its
  // scale bytes 4 kScaleGroup q + 16 (p % (kScaleGroup / 4)) ..), to LDS byte
  // 16 p. W load kXLoads + j: chunk p = 64 j + l is columns 16 (p % 8) .. + 15 of
  // scale row 4 kScaleGroup q + p / 8, to LDS byte kScaleBufBytes + 16 p.
  // Chunks outside the matrix or past K read as zero.
  constexpr int kXLoads = kScaleGroup / 2;
  auto issue_scales = [&](int q, uint8_t* buf) {
    for (int j = wave; j < 2 * kXLoads; j += 4) {
      if (j < kXLoads) {
        const int p = j * 64 + lane;
        const int r = p / (kScaleGroup / 4), cx = q * 4 * kScaleGroup + (p % (kScaleGroup / 4)) * 16;
        const uint32_t ox = (r < rows_valid && cx < nsb) ? (uint32_t)(r * ldxs + cx) : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, LDS(void, buf + j * 1024), 16, ox, 0, 0, 0);
      } else {
        const int p = (j - kXLoads) * 64 + lane;
        uint32_t ow;
        if constexpr (kWT) {  // W^T scales: laid out like the X part
          const int n = p / (kScaleGroup / 4), cx = q * 4 * kScaleGroup + (p % (kScaleGroup / 4)) * 16;
          ow = (n < cols_valid && cx < nsb) ? (uint32_t)(n * ldws + cx) : kOob;
        } else {
          const int kr = q * 4 * kScaleGroup + (p >> 3), cw = (p & 7) * 16;
          ow = (kr < nsb && cw < cols_valid) ? (uint32_t)(kr * ldws + cw) : kOob;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rws, LDS(void, buf + kScaleBufBytes + (j - kXLoads) * 1024), 16, ow,
                                                 0, 0, 0);
      }
    }
  };
  // The scales of block kb (position b in its group) from its group's buffer:
  // the X dword of the lane's row (bytes kk * 2 + g), the W byte of the lane's
  // column in scale row 4 b + kk * 2 + g.
  auto read_scales = [&](int b, const uint8_t* buf, int (&sa_)[2][2], int (&sb_)[2][2]) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int r = wm * 64 + f * 32 + (lane & 31);
      const int d = *LDS(const int, buf + r * 4 * kScaleGroup + b * 4);
      const int c = wn * 64 + f * 32 + (lane & 31);
      int dw = 0;
      if constexpr (kWT) dw = *LDS(const int, buf + kScaleBufBytes + c * 4 * kScaleGroup + b * 4);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        sa_[f][kk] = (d >> (8 * (kk * 2 + g))) & 0xFF;
        if constexpr (kWT)
          sb_[f][kk] = (dw >> (8 * (kk * 2 + g))) & 0xFF;
        else
          sb_[f][kk] = *LDS(const uint8_t, buf + kScaleBufBytes + (b * 4 + kk * 2 + g) * 128 + c);
      }
    }
  };

  // Byte path: scale registers of the K blocks in flight, one ring slot per
  // stage: [slot][fragment][MFMA step].
  int sa[kStagesMx][2][2], sb[kStagesMx][2][2];
  // Unroll length of the K loop: a multiple of the stage count (LDS stages and
  // scale slots) and, on the staged path, of two scale groups, so that every
  // step's stage and scale buffer are fixed objects.
  constexpr int kUnroll = kStaged ? (kStagesMx == 3 ? 6 * kScaleGroup : 2 * kScaleGroup) : 2 * kStagesMx;
  static_assert(!kStaged || (kUnroll % kStagesMx == 0 && kUnroll % (2 * kScaleGroup) == 0), "unroll");

  // One K block. Staged path: the next scale group is requested at the first
  // block of a group (its buffer was last read in the previous block, before
  // this step's barrier). Byte path: each block's scale loads are issued just
  // before its LDS-DMA loads, kStagesMx - 1 blocks ahead, so the wait for this
  // block's DMA also covers its scales. Younger than this block's loads are the
  // next kStagesMx - 2 blocks' loads (4 + kNx DMA loads each, and on the byte
  // path the wave's scale loads); a scale group in flight, or the prologue's
  // full set of loads, only makes the wait cover more than it needs to. Then
  // the stage read in the previous block is refilled and the
  // MFMA chain runs on this stage: kk ascending, the wave's first kNf row
  // fragments (kNf < 2 only where the tile's rows past M cover whole 32-row
  // fragments, which are then neither read nor multiplied; every multiplied
  // fragment runs the same chain as in a full tile). u is the step's position
  // in the unrolled loop.
  auto step = [&](auto nf, auto nx, f32x16 (&acc)[2][2], int kb, int u, const uint8_t* st, uint8_t* refill,
                  int (&sac)[2][2], const int (&sbc)[2][2], int (&san)[2][2],
                  int (&sbn)[2][2]) __attribute__((always_inline)) {
    constexpr int kNf = decltype(nf)::value;
    constexpr int kNx = decltype(nx)::value;
    // Byte path: only the scale loads whose values the wave multiplies are
    // issued (an unused load could be dropped by the compiler, and the count
    // below must be exact): 2 kNf X bytes and 4 W bytes per block, none if
    // kNf = 0.
    constexpr int kScaleLoads = kStaged ? 0 : (kNf > 0 ? 4 + 2 * kNf : 0);
    BIGEMM_WAIT_VMCNT((4 + kNx + kScaleLoads) * (kStagesMx - 2));
    BIGEMM_BARRIER();
    const int nb = kb + kStagesMx - 1;
    // u is a multiple of kScaleGroup exactly where kb is (kUnroll is a multiple
    // of two groups and the loop starts at kb = 0). Every wave issues its share
    // of the scale group, whatever it multiplies.
    if (kStaged) {
      if (u % kScaleGroup == 0) issue_scales(kb / kScaleGroup + 1, scl[(u / kScaleGroup + 1) % 2]);
    } else if constexpr (kNf > 0) {
      load_xscales(nf, nb, san);
      load_wscales(nb, sbn);
    }
    issue(nx, nb, refill);
    if constexpr (kNf == 0) return;
    int sal[2][2], sbl[2][2];
    if (kStaged) read_scales(u % kScaleGroup, scl[(u / kScaleGroup) % 2], sal, sbl);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8 a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (f < kNf) {
          const i32x4 a0 = *LDS(const i32x4, st + a_addr[f][kk][0]);
          const i32x4 a1 = *LDS(const i32x4, st + a_addr[f][kk][1]);
          a[f] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
        if constexpr (kWT) {
          const i32x4 b0 = *LDS(const i32x4, st + bt_addr[f][kk][0]);
          const i32x4 b1 = *LDS(const i32x4, st + bt_addr[f][kk][1]);
          b[f] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        } else {
          i32x2 bv[4];
#pragma unroll
          for (int rd = 0; rd < 4; ++rd)
            bv[rd] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS(i32x2, st + b_addr[f][kk][rd]));
          b[f] = i32x8{bv[0][0], bv[0][1], bv[1][0], bv[1][1], bv[2][0], bv[2][1], bv[3][0], bv[3][1]};
        }
      }
#pragma unroll
      for (int fm = 0; fm < kNf; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[fm], b[fn], acc[fm][fn], 0 /*A: E4M3*/, 0 /*B: E4M3*/, 0, kStaged ? sal[fm][kk] : sac[fm][kk], 0,
              kStaged ? sbl[fn][kk] : sbc[fn][kk]);
    }
  };

  // Prologue: the first scale group (staged path), a dummy (entirely
  // out-of-range) fill of the last stage, then blocks 0 to kStagesMx - 2 with
  // their scales. The dummy makes the loads in
  // flight at the loop head target the stages in the same order on entry as on
  // every later iteration.
  // The prologue issues every load (zeros in the rows past M of every stage); a
  // variant issuing fewer loads per block only waits for more than it needs on
  // its first steps.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (kStaged) issue_scales(0, scl[0]);
  issue(I4{}, nkb, stg[kStagesMx - 1]);
#pragma unroll
  for (int s = 0; s < kStagesMx - 1; ++s) {
    if (!kStaged) {
      load_xscales(I2{}, s, sa[s]);
      load_wscales(s, sb[s]);
    }
    issue(I4{}, s, stg[s]);
  }
  // Unrolled by kUnroll so that each stage and scale slot is fixed in every
  // step. (The compiler cannot track which stage the loads in flight
  // target across the loop back-edge and drains them before the first step of
  // an iteration; a longer body makes that the exception.)
  // Each variant holds its own accumulators and stores its own fragments
  // (plain stores, masked through the buffer range check; a wave with kNf = 0
  // holds only rows past M and stores nothing).
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc((uint8_t*)Y + ((int64_t)row0 * ldy + col0) * (kOutBf16 ? 2 : 4));
  auto kloop = [&](auto nf, auto nx) __attribute__((always_inline)) {
    constexpr int kNf = decltype(nf)::value;
    for (int kb = 0;;) {
      bool done = false;
      // Keep the accumulators in AGPRs across the back edge: with several K
      // loops in the kernel the register allocator otherwise carries them in
      // VGPRs and copies all 64 registers out and back at every iteration.
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = u % kStagesMx, n = (u + kStagesMx - 1) % kStagesMx;
        step(nf, nx, acc, kb, u, stg[c], stg[n], sa[c], sb[c], sa[n], sb[n]);
        if (++kb == nkb) {
          done = true;
          break;
        }
      }
      if (done) break;
    }
    BIGEMM_WAIT_VMCNT(0);  // no LDS-DMA load may outlive the workgroup
#pragma unroll
    for (int fm = 0; fm < kNf; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 64 + fm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int cl = wn * 64 + fn * 32 + (lane & 31);
          // Copy the element out first: bit-casting an ext_vector element
          // expression directly reads element 0 with this compiler.
          const float v = acc[fm][fn][r];
          store_out<kOutBf16>(ry, rl < rows_valid && cl < cols_valid, (uint32_t)(rl * ldy + cl),
                              __builtin_bit_cast(uint32_t, v));
        }
  };
  // Per wave (uniform: the wave index is read as a scalar): nf of its row
  // fragments and nx of its X loads hold a row below M. Only tiles of at most
  // 64 rows get a reduced loop; a wave may run a variant with more fragments or
  // loads than it needs (the extra loads read zeros, the extra fragments are
  // never stored), so six loops cover every count, as in the bf16 kernel.
  const int wave_u = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const int wrow0 = (wave_u >> 1) * 64;
  const int nf = (rows_valid > wrow0) + (rows_valid > wrow0 + 32);
  const int nx = (wave_u * 8 < rows_valid) + (32 + wave_u * 8 < rows_valid);
  if (__builtin_expect(rows_valid > 64, 1)) {
    kloop(I2{}, I4{});  // full tiles (and every tile of more than 64 rows)
  } else if (nf == 2) {
    kloop(I2{}, I2{});
  } else if (nf == 1) {
    kloop(I1{}, I1{});
  } else if (nx == 2) {
    kloop(I0{}, I2{});
  } else if (nx == 1) {
    kloop(I0{}, I1{});
  } else {
    kloop(I0{}, I0{});
  }
}

// ------------------------------------------------------------------------ int8
//
// The MXFP8 skeleton without scales: K block 128, X tile 128 x 128 bytes and W
// tile 128 x 128 bytes per stage, 4 waves of 64 x 64 outputs, three stages.
// MFMA 32x32x32 int8 with int32 accumulate: lane l holds row (column) l%32 and
// the 16 consecutive K values 16*(l/32) .. +15 of a 32-wide step (any K order
// shared by both operands gives the same exact integer sum). Integer addition
// is associative, so the result is independent of the summation order; the
// kernel still walks K in one fixed order like the others.
typedef int i32x16 __attribute__((ext_vector_type(16)));
constexpr int kBkI8 = 128;
constexpr int kStagesI8 = 3;

// kWT: W given as [N, K] rows (ldw >= K); its tile and fragments are then
// handled like X's.
template <bool kWT = false>
__global__ __launch_bounds__(kThreads, 1)
void bigemm_i8_kernel(const uint8_t* __restrict__ X, const uint8_t* __restrict__ W,
                      int32_t* __restrict__ Y, int M, int N, int K,
                      int64_t ldx, int64_t ldw, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kStageBytes];
  uint8_t* const stg[3] = {stage0, stage1, stage2};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (__builtin_expect((int)blockIdx.x >= tiles_m * tiles_n, 0)) {  // a prefetch workgroup
    u8_prefetch<kWT, false>(X, W, nullptr, M, N, K, ldx, ldw, 0, tiles_m, tiles_n, stage0, tid);
    return;
  }
  int tm, tn;
  tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tm, tn);
  const int row0 = tm * 128;
  const int col0 = tn * 128;
  const int rows_valid = min(128, M - row0);
  const int cols_valid = min(128, N - col0);
  const int nkb = (K + kBkI8 - 1) / kBkI8;

  // Load assignment as in the MXFP8 kernel: chunk p = i*256 + tid.
  uint32_t xoff[4], woff[4];
  int xk[4], wk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = i * kThreads + tid;
    const int r = p >> 3, s = p & 7, c = s ^ swz_x(r);
    xoff[i] = (uint32_t)(r * ldx + c * 16);
    xk[i] = r < rows_valid ? c * 16 : 0x7FFFFFFF;
    if constexpr (kWT) {
      woff[i] = (uint32_t)(r * ldw + c * 16);
      wk[i] = r < cols_valid ? c * 16 : 0x7FFFFFFF;
    } else {
      const int kr = p >> 3, cw = s ^ swz_w8(kr);
      woff[i] = (uint32_t)(kr * ldw + cw * 16);
      wk[i] = cw * 16 < cols_valid ? kr : 0x7FFFFFFF;
    }
  }
  const uint8_t* Xt = X + (int64_t)row0 * ldx;
  const uint8_t* Wt = kWT ? W + (int64_t)col0 * ldw : W + col0;

  // The LDS-DMA loads of K block kb (blocks past the end load zeros). kNx: how
  // many of the wave's four X loads are issued; load i covers tile rows
  // 32 i + 8 wave .. + 7, and those whose rows are all past M are left out
  // (their LDS rows keep the zeros the prologue wrote), as in the MXFP8 kernel.
  auto issue = [&](auto nx, int kb, uint8_t* stage) {
    constexpr int kNx = decltype(nx)::value;
    const bool live = kb < nkb;
    const int k0 = live ? kb * kBkI8 : 0;
    const int kleft = live ? K - k0 : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(Xt + k0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(kWT ? Wt + k0 : Wt + (int64_t)k0 * ldw);
#pragma unroll
    for (int i = 0; i < kNx; ++i) {
      const uint32_t o = xk[i] < kleft ? xoff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, LDS(void, stage + i * 4096 + wave * 1024), 16, o, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = wk[i] < kleft ? woff[i] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, LDS(void, stage + kTileBytes + i * 4096 + wave * 1024), 16, o,
                                                0, 0, 0);
    }
  };

  // Fragment addresses per 32-wide K step kk: A one 16-byte read, B two
  // transposing 8-byte reads (K values 0..7 and 8..15 of the lane's 16), or
  // for W^T one 16-byte read addressed like A's.
  const int wm = wave >> 1, wn = wave & 1;
  int a_addr[2][4];      // [f][kk]
  int b_addr[2][4][2];   // [f][kk][half]
  int bt_addr[2][4];     // [f][kk]
#pragma unroll
  for (int f = 0; f < 2; ++f) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int r = wm * 64 + f * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      a_addr[f][kk] = r * 128 + ((c ^ swz_x(r)) << 4);
      if constexpr (kWT) {
        const int n = wn * 64 + f * 32 + (lane & 31);
        bt_addr[f][kk] = kTileBytes + n * 128 + ((c ^ swz_x(n)) << 4);
      }
      const int G = lane >> 4, j = lane & 15;
      const int col = wn * 64 + f * 32 + (G & 1) * 16 + (j & 1) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kr = kk * 32 + (G >> 1) * 16 + h * 8 + (j >> 1);
        b_addr[f][kk][h] = kTileBytes + kr * 128 + (((col >> 4) ^ swz_w8(kr)) << 4) + (col & 15);
      }
    }
  }

  i32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = i32x16{};

  // One K block: wait for this stage (the next blocks' 4 + kNx loads each may
  // stay in flight), refill the stage read in the previous block, MFMA chain kk
  // ascending over the wave's first kNf row fragments (kNf < 2 only where the
  // tile's rows past M cover whole 32-row fragments).
  auto step = [&](auto nf, auto nx, int kb, const uint8_t* st, uint8_t* refill) __attribute__((always_inline)) {
    constexpr int kNf = decltype(nf)::value;
    constexpr int kNx = decltype(nx)::value;
    BIGEMM_WAIT_VMCNT((4 + kNx) * (kStagesI8 - 2));
    BIGEMM_BARRIER();
    issue(nx, kb + kStagesI8 - 1, refill);
    if constexpr (kNf == 0) return;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      i32x4 a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (f < kNf) a[f] = *LDS(const i32x4, st + a_addr[f][kk]);
        if constexpr (kWT) {
          b[f] = *LDS(const i32x4, st + bt_addr[f][kk]);
        } else {
          const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS(i32x2, st + b_addr[f][kk][0]));
          const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS(i32x2, st + b_addr[f][kk][1]));
          b[f] = i32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int fm = 0; fm < kNf; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  };

  // Prologue with every load (zeros in the rows past M of every stage).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  issue(I4{}, nkb, stg[kStagesI8 - 1]);
#pragma unroll
  for (int s2 = 0; s2 < kStagesI8 - 1; ++s2) issue(I4{}, s2, stg[s2]);
  // Unrolled 8 times the stage count, so that the compiler's drain of the loads
  // in flight at the loop head (it cannot tell which stage they target) comes
  // once per 24 blocks. Each variant stores its own fragments.
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(Y + (int64_t)row0 * ldy + col0);
  auto kloop = [&](auto nf, auto nx) __attribute__((always_inline)) {
    constexpr int kNf = decltype(nf)::value;
    for (int kb = 0;;) {
      bool done = false;
      // Keep the accumulators in AGPRs across the back edge (see the MXFP8 kernel).
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
      for (int u = 0; u < 8 * kStagesI8; ++u) {
        step(nf, nx, kb, stg[u % kStagesI8], stg[(u + kStagesI8 - 1) % kStagesI8]);
        if (++kb == nkb) {
          done = true;
          break;
        }
      }
      if (done) break;
    }
    BIGEMM_WAIT_VMCNT(0);  // no LDS-DMA load may outlive the workgroup
#pragma unroll
    for (int fm = 0; fm < kNf; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * 64 + fm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int cl = wn * 64 + fn * 32 + (lane & 31);
          const int v = acc[fm][fn][r];
          store_out<false>(ry, rl < rows_valid && cl < cols_valid, (uint32_t)(rl * ldy + cl), (uint32_t)v);
        }
  };
  // Per wave, as in the MXFP8 kernel: tiles of more than 64 rows run the full
  // loop; in smaller ones each wave runs the smallest of six loops that covers
  // its fragments and X loads holding a row below M.
  const int wave_u = __builtin_amdgcn_readfirstlane(tid) >> 6;
  const int wrow0 = (wave_u >> 1) * 64;
  const int nf = (rows_valid > wrow0) + (rows_valid > wrow0 + 32);
  const int nx = (wave_u * 8 < rows_valid) + (32 + wave_u * 8 < rows_valid);
  if (__builtin_expect(rows_valid > 64, 1)) {
    kloop(I2{}, I4{});
  } else if (nf == 2) {
    kloop(I2{}, I2{});
  } else if (nf == 1) {
    kloop(I1{}, I1{});
  } else if (nx == 2) {
    kloop(I0{}, I2{});
  } else if (nx == 1) {
    kloop(I0{}, I1{});
  } else {
    kloop(I0{}, I0{});
  }
}

// ------------------------------------------------------------- split-K merge
//
// Y[i, j] = P[0][i, j] + P[1][i, j] + ... + P[S-1][i, j], added in ascending
// chunk order in fp32 (then rounded once to bf16 for a bf16 output). P is
// [S][M][N] fp32. kVec4 (N a multiple of 4): one thread per four consecutive
// outputs of a row, 16-byte loads; otherwise one thread per output. The sums
// and their order are the same either way. The chunk sums are loaded up to
// kMergeAhead at a time before they are added (a loop with a run-time count
// otherwise waits for each load before issuing the next); the adds keep
// ascending chunk order.
constexpr int kMergeAhead = 8;
template <bool kOutBf16, bool kVec4>
__global__ __launch_bounds__(256)
void bigemm_split_merge_kernel(const float* __restrict__ P, void* __restrict__ Y, int M, int N, int64_t ldy,
                               int nsplit, int64_t split_stride) {
  if constexpr (kVec4) {
    const int nq = N / 4;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)M * nq) return;
    const int i = (int)(q / nq);
    const int j = (int)(q - (int64_t)i * nq) * 4;
    const float* p = P + (int64_t)i * N + j;
    float4 acc = *(const float4*)p;
    for (int s = 1; s < nsplit; s += kMergeAhead) {
      float4 v[kMergeAhead];
#pragma unroll
      for (int u = 0; u < kMergeAhead; ++u)
        if (s + u < nsplit) v[u] = *(const float4*)(p + (s + u) * split_stride);
#pragma unroll
      for (int u = 0; u < kMergeAhead; ++u)
        if (s + u < nsplit) {
          acc.x += v[u].x;
          acc.y += v[u].y;
          acc.z += v[u].z;
          acc.w += v[u].w;
        }
    }
    if (kOutBf16) {
      const uint32_t b0 = f32_to_bf16_rne(__builtin_bit_cast(uint32_t, acc.x));
      const uint32_t b1 = f32_to_bf16_rne(__builtin_bit_cast(uint32_t, acc.y));
      const uint32_t b2 = f32_to_bf16_rne(__builtin_bit_cast(uint32_t, acc.z));
      const uint32_t b3 = f32_to_bf16_rne(__builtin_bit_cast(uint32_t, acc.w));
      uint2 packed;
      packed.x = b0 | (b1 << 16);
      packed.y = b2 | (b3 << 16);
      *(uint2*)((uint16_t*)Y + (int64_t)i * ldy + j) = packed;
    } else {
      *(float4*)((float*)Y + (int64_t)i * ldy + j) = acc;
    }
  } else {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)M * N) return;
    const int i = (int)(q / N);
    const int j = (int)(q - (int64_t)i * N);
    const float* p = P + (int64_t)i * N + j;
    float acc = *p;
    for (int s = 1; s < nsplit; s += kMergeAhead) {
      float v[kMergeAhead];
#pragma unroll
      for (int u = 0; u < kMergeAhead; ++u)
        if (s + u < nsplit) v[u] = p[(s + u) * split_stride];
#pragma unroll
      for (int u = 0; u < kMergeAhead; ++u)
        if (s + u < nsplit) acc += v[u];
    }
    if (kOutBf16)
      ((uint16_t*)Y)[(int64_t)i * ldy + j] = (uint16_t)f32_to_bf16_rne(__builtin_bit_cast(uint32_t, acc));
    else
      ((float*)Y)[(int64_t)i * ldy + j] = acc;
  }
}

// ------------------------------------------------------------ static scratch
//
// The chunk sums of bigemm_run_split_k_static live in this file-scope device
// array instead of a caller workspace, for callers that cannot allocate. Each
// GPU holds its own copy for the life of the process. Its name is a host-side
// stand-in in host code: the device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that address
// is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch_address(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[device].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != device) return hipErrorInvalidDevice;  // the lookup must run with that device current
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_addr[device].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers

typedef void (*Bf16KernelFn)(const uint16_t*, const uint16_t*, void*, int, int, int, int64_t, int64_t, int64_t, int,
                             int, int, int64_t);

// The bf16 / fp16 kernel instance for W given as [K, N] (wt false) or [N, K],
// and for K a multiple of 8 or not (ktail): choices made from the layout and K,
// never from M.
template <bool kF16, bool kOutBf16, bool kSplit>
Bf16KernelFn bf16_kernel_for(bool wt, bool ktail) {
  if (ktail)
    return wt ? bigemm_bf16_kernel<kF16, kOutBf16, kSplit, true, true>
              : bigemm_bf16_kernel<kF16, kOutBf16, kSplit, false, true>;
  return wt ? bigemm_bf16_kernel<kF16, kOutBf16, kSplit, true> : bigemm_bf16_kernel<kF16, kOutBf16, kSplit, false>;
}

hipError_t launch_bf16(Op op, bool wt, const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                       int64_t ldx, int64_t ldw, int64_t ldy, int cus, hipStream_t stream) {
  const int tiles_m = (int)((M + 127) / 128);
  const int tiles_n = (int)((N + 127) / 128);
  const int ntiles = tiles_m * tiles_n;
  const int grid = prefetch_grid(ntiles, (int)((K + kBkBf16 - 1) / kBkBf16), cus);
  const bool f16 = op.in == kInF16, obf = op.out == 1 /* BIGEMM_BF16 */;
  const bool kt = K % 8 != 0;
  const Bf16KernelFn kern =
      f16 ? (obf ? bf16_kernel_for<true, true, false>(wt, kt) : bf16_kernel_for<true, false, false>(wt, kt))
          : (obf ? bf16_kernel_for<false, true, false>(wt, kt) : bf16_kernel_for<false, false, false>(wt, kt));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreadsBf16), 0, stream, (const uint16_t*)X, (const uint16_t*)W, Y,
                     (int)M, (int)N, (int)K, ldx, ldw, ldy, tiles_m, tiles_n, 0, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_bf16_split(Op op, bool wt, int32_t k_chunk, const void* X, const void* W, void* Y, void* P,
                             int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                             hipStream_t stream) {
  const int tiles_m = (int)((M + 127) / 128);
  const int tiles_n = (int)((N + 127) / 128);
  const int nsplit = (int)((K + k_chunk - 1) / k_chunk);
  const int64_t stride = M * N;
  const bool f16 = op.in == kInF16, obf = op.out == 1 /* BIGEMM_BF16 */;
  const bool kt = K % 8 != 0;
  const Bf16KernelFn kern =
      f16 ? bf16_kernel_for<true, false, true>(wt, kt) : bf16_kernel_for<false, false, true>(wt, kt);
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n * nsplit), dim3(kThreadsBf16), 0, stream, (const uint16_t*)X,
                     (const uint16_t*)W, P, (int)M, (int)N, (int)K, ldx, ldw, N, tiles_m, tiles_n,
                     k_chunk / kBkBf16, stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool vec4 = N % 4 == 0;  // (and then ldy keeps output rows 16-byte aligned)
  const int64_t threads = vec4 ? M * (N / 4) : M * N;
  const int blocks = (int)((threads + 255) / 256);
  auto merge = vec4 ? (obf ? bigemm_split_merge_kernel<true, true> : bigemm_split_merge_kernel<false, true>)
                    : (obf ? bigemm_split_merge_kernel<true, false> : bigemm_split_merge_kernel<false, false>);
  hipLaunchKernelGGL(merge, dim3(blocks), dim3(256), 0, stream, (const float*)P, Y, (int)M, (int)N, ldy, nsplit,
                     stride);
  return hipGetLastError();
}

hipError_t launch_mxfp8(Op op, bool wt, const void* X, const void* W, void* Y, const void* XS, const void* WS,
                        int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldw, int64_t ldy,
                        int64_t ldxs, int64_t ldws, int cus, hipStream_t stream) {
  const int tiles_m = (int)((M + 127) / 128);
  const int tiles_n = (int)((N + 127) / 128);
  // the same padding rule as the bf16 kernel, K counted in 64-deep blocks
  const int grid = prefetch_grid(tiles_m * tiles_n, (int)((K + 63) / 64), cus);
  // The scale load path depends on the scale layout and K only (never on M);
  // both paths read the same scale values.
  const bool staged = K % 512 == 0 && ((uintptr_t)XS & 15) == 0 && ldxs % 16 == 0 && ((uintptr_t)WS & 15) == 0 &&
                      ldws % 16 == 0;
  const bool obf = op.out == 1 /* BIGEMM_BF16 */;
  auto kern = wt ? (staged ? (obf ? bigemm_mxfp8_kernel<true, true, true> : bigemm_mxfp8_kernel<true, false, true>)
                           : (obf ? bigemm_mxfp8_kernel<false, true, true> : bigemm_mxfp8_kernel<false, false, true>))
                 : (staged ? (obf ? bigemm_mxfp8_kernel<true, true> : bigemm_mxfp8_kernel<true, false>)
                           : (obf ? bigemm_mxfp8_kernel<false, true> : bigemm_mxfp8_kernel<false, false>));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, (const uint8_t*)X,
                     (const uint8_t*)W, Y, (const uint8_t*)XS, (const uint8_t*)WS, (int)M, (int)N, (int)K, ldx, ldw,
                     ldy, ldxs, ldws, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_i8(bool wt, const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K, int64_t ldx,
                     int64_t ldw, int64_t ldy, int cus, hipStream_t stream) {
  const int tiles_m = (int)((M + 127) / 128);
  const int tiles_n = (int)((N + 127) / 128);
  const int grid = prefetch_grid(tiles_m * tiles_n, (int)((K + 63) / 64), cus);
  hipLaunchKernelGGL(wt ? bigemm_i8_kernel<true> : bigemm_i8_kernel<false>, dim3(grid), dim3(kThreads), 0,
                     stream, (const uint8_t*)X, (const uint8_t*)W, (int32_t*)Y, (int)M, (int)N, (int)K, ldx, ldw, ldy,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace bigemm
