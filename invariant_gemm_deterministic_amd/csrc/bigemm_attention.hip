// Batch-invariant paged attention for CDNA4 (gfx950).
//
// The nondeterminism blog, section "batch-invariant attention": a query at
// position i of a sequence attends to the keys and values of positions j <= i,
//   o = sum_{j <= i} softmax_j(scale * q . k_j) v_j,
// and the section gives two rules that make it batch-invariant:
//   - the KV cache and its page table are written BEFORE the attention kernel
//     (bigemm_kv_write_kernel below), so the kernel always reads every key and
//     value of positions 0..i from the cache, in the same layout, whether they
//     were cached earlier or arrived in this call;
//   - the KV range is split into chunks of a FIXED SIZE (split-KV with a fixed
//     split size, not a fixed number of splits), so the summation order of a
//     query depends on its own position only, never on the batch.
//
// Split kernel: one workgroup per (query token t, KV head, split s) covers
// positions [256 s, min(256 s + 256, pos + 1)) for the G query heads sharing
// the KV head (G = 1..16, one instantiation each).
//   scores: each wave takes 64 positions as four 16 x 16 tiles of
//           v_mfma_f32_16x16x32_bf16 (query heads as rows, padded with zeros,
//           positions as columns, the head dimension in steps of 32 in a fixed
//           order); K rows are read straight into the B-operand layout;
//   softmax: per head, the split maximum m and p_j = exp(s_j - m) (fp32), and
//           l = sum_j p_j (a fixed DPP tree per wave, then the four waves in
//           order);
//   values: each wave stages its 64 V rows through its own LDS rows, 32 at a
//           time, and reads them back with ds_read_b64_tr_b16 as the B
//           operand of v_mfma_f32_16x16x32_bf16 (no block barrier: one wave's
//           LDS accesses complete in order); the fp32 weights enter as three
//           bf16 parts with an exact sum, positions in a fixed order; then the
//           four waves' outputs are added in order.
// Each split result is a fixed function of that split's inputs.
// Merge kernel: per (token, query head), the splits' (m_s, l_s, acc_s) are
// combined as m = max_s m_s, w_s = exp(m_s - m),
// o = (sum_s w_s acc_s) / (sum_s w_s l_s), the sums in a fixed tree that depends
// on the number of splits only, rounded once to the output type.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bigemm_attention.h"

namespace bigemm {

namespace {

constexpr int kThreads = 256;
static_assert(kAttnSplit == kThreads, "one position of a split per thread after the score reduction");

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Cross-lane moves by DPP: the quad permutations swap neighbours at distance 1
// and 2, row_half_mirror pairs lane i with 7 - i inside each half row,
// row_mirror pairs i with 15 - i inside each 16-lane row; row_bcast:15 /
// row_bcast:31 pass the last lane of a row (of rows 0-1) to the rows that
// row_mask selects.
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppRowMirror = 0x140,
              kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Rows outside kRowMask keep `id`.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows(float x, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), kCtrl, kRowMask, 0xF,
                                                    false));
}

// Max (kMax) or sum of x over the 64 lanes of the wave, valid in lane 63: within
// quads, half rows and rows, then rows 0+1 and 2+3, then the two halves. A
// fixed tree of VALU steps (no LDS round trips). The max ignores NaN, as fmaxf.
template <bool kMax>
__device__ __forceinline__ float wave_reduce63(float x) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  const float id = kMax ? -INFINITY : 0.f;
  x = op(x, dpp<kDppQuadXor1>(x));
  x = op(x, dpp<kDppQuadXor2>(x));
  x = op(x, dpp<kDppHalfMirror>(x));
  x = op(x, dpp<kDppRowMirror>(x));
  x = op(x, dpp_rows<kDppRowBcast15, 0xA>(x, id));
  x = op(x, dpp_rows<kDppRowBcast31, 0xC>(x, id));
  return x;
}

__device__ __forceinline__ int64_t slot_row(int blk, int Hkv, int kvh, int bs_log2, int j) {
  return ((((int64_t)blk * Hkv + kvh) << bs_log2) + (j & ((1 << bs_log2) - 1)));
}

// fp32 -> three bf16 parts whose sum is the value exactly (for values of normal
// bf16 range): hi = RNE(x), mid = RNE(x - hi), lo = x - hi - mid.
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_rne(__float_as_uint(x));
  const float r1 = x - __uint_as_float(hi << 16);
  mid = f32_to_bf16_rne(__float_as_uint(r1));
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_rne(__float_as_uint(r2));
}

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds(const void* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads)
void bigemm_attn_split_kernel(AttnParams p) {
  constexpr int kC = D / 32;      // MFMA steps along the head dimension (scores)
  constexpr int kNT = D / 16;     // 16-column output tiles (values)
  constexpr int kVS = D + 16;     // staged V row stride in elements (D*2 + 32 bytes)
  static_assert(G <= 16, "the query heads of a group are the rows of one 16 x 16 MFMA tile");
  __shared__ __align__(16) float p_s[G][kAttnSplit];        // scores, then weights, by position
  __shared__ __align__(16) uint16_t v_s[4][32][kVS];        // per wave: 32 V rows being consumed
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ int32_t blk_s[kAttnSplit];
  // After the values: per-wave outputs for all 16 rows of the MFMA tile (rows
  // past G hold zeros and are not read). Every row is stored unconditionally:
  // with stores predicated on h < G, this compiler placed one output of the
  // G = 15, D = 64 kernel at a wrong offset when it paired the stores.
  float (*acc_s)[16][D] = (float (*)[16][D])&v_s[0][0][0];
  static_assert(sizeof(v_s) >= sizeof(float) * 4 * 16 * D, "acc_s fits in v_s");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x % p.nsplit;
  const int rest = blockIdx.x / p.nsplit;
  const int kvh = rest % p.Hkv;
  const int t = rest / p.Hkv;
  const int sq = p.seq_ids[t], pos = p.positions[t];
  if (sq < 0 || sq >= p.num_seqs || pos < 0 || pos >= p.max_context) return;  // the merge writes NaN
  const int j0 = s * kAttnSplit;
  if (j0 > pos) return;  // past this token's context
  const int n = min(kAttnSplit, pos + 1 - j0);
  const int b0 = j0 >> p.bs_log2;
  const int nb = ((j0 + n - 1) >> p.bs_log2) - b0 + 1;
  const int32_t* bt = p.block_table + (int64_t)sq * p.max_blocks;
  for (int i = tid; i < nb; i += kThreads) blk_s[i] = bt[b0 + i];

  // Q as the A operand of v_mfma_f32_16x16x32_bf16: lane l supplies head l % 16
  // (zero rows past G), head-dimension elements 32 c + 8 (l / 16) .. + 7.
  const int qh = lane & 15, kq = 8 * (lane >> 4);
  const i32x4 kZero = {0, 0, 0, 0};
  const i32x4 kNaN = {0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0};
  i32x4 qa[kC];
  const uint16_t* qrow = p.Q + ((int64_t)t * p.H + (int64_t)kvh * G + qh) * D + kq;
#pragma unroll
  for (int c = 0; c < kC; ++c) qa[c] = qh < G ? *(const i32x4*)(qrow + 32 * c) : kZero;
  __syncthreads();

  // K and V rows in the B-operand layout: wave w takes positions 64 w + 16 b +
  // (l % 16) of the split, lane l elements 32 c + 8 (l / 16) .. + 7 of the row.
  // Rows past the context are zero (their weights are zero), rows whose block
  // id is invalid are NaN.
  // Row offsets of this lane's four positions (-1: past the context or an
  // invalid block id).
  int64_t roff[4];
  bool past[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int jj = 64 * wave + 16 * b + qh;
    past[b] = jj >= n;
    roff[b] = -1;
    if (!past[b]) {
      const int j = j0 + jj;
      const int blk = blk_s[(j >> p.bs_log2) - b0];
      if (blk >= 0 && blk < p.num_blocks) roff[b] = slot_row(blk, p.Hkv, kvh, p.bs_log2, j) * D + kq;
    }
  }
  auto load_rows = [&](const uint16_t* base, i32x4 (&dst)[4][kC]) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < kC; ++c)
        dst[b][c] = past[b] ? kZero : roff[b] < 0 ? kNaN : *(const i32x4*)(base + roff[b] + 32 * c);
  };
  i32x4 kb[4][kC];
  load_rows(p.K, kb);

  // Scores: D[head][position] of each 16-position block; lane l holds position
  // l % 16 for heads 4 (l / 16) + r. The V rows of a block are requested once
  // its K rows are consumed (so K and V are not both held in registers).
  i32x4 vb[4][kC];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kC; ++c)
      acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[c]),
                                                     __builtin_bit_cast(bf16x8, kb[b][c]), acc4, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kC; ++c)
      vb[b][c] = past[b] ? kZero : roff[b] < 0 ? kNaN : *(const i32x4*)(p.V + roff[b] + 32 * c);
    const int jj = 64 * wave + 16 * b + qh;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * (lane >> 4) + r;
      if (h < G) p_s[h][jj] = jj < n ? acc4[r] * p.scale : -INFINITY;
    }
  }
  __syncthreads();

  // softmax statistics of the split, per head; thread tid owns position tid
  float sh[G], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    sh[h] = p_s[h][tid];
    const float x = wave_reduce63<true>(sh[h]);
    if (lane == 63) red_m[wave][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    const float w = expf(sh[h] - m[h]);
    p_s[h][tid] = w;
    const float x = wave_reduce63<false>(w);
    if (lane == 63) red_l[wave][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = ((red_l[0][h] + red_l[1][h]) + red_l[2][h]) + red_l[3][h];

  // Values: O[head][d] += P[head][position] V[position][d] by 16 x 16 x 32 MFMA
  // tiles, positions in two steps of 32 per wave. The fp32 weights enter as
  // three bf16 parts (exact sum), V through LDS with the transposing read.
  f32x4 o[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // ds_read_b64_tr_b16: in each 16-lane group, lane i element e is element i % 4
  // of the 8 bytes lane 4 e + i / 4 addresses. Lane j of group g addresses row
  // 8 g + j / 4 (+ 4), columns 16 nt + 4 (j % 4): lane i then holds column
  // 16 nt + i, rows 8 g .. 8 g + 7 — the B operand.
  const int tr_row = kq + ((lane & 15) >> 2), tr_col = 4 * (lane & 3);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int c = 0; c < kC; ++c) *(i32x4*)&v_s[wave][16 * bb + qh][32 * c + kq] = vb[2 * ks + bb][c];
    // weights of positions 64 w + 32 ks + 8 (l / 16) .. + 7 for head l % 16
    i32x4 ph = kZero, pm = kZero, pl = kZero;
    if (qh < G) {
      const float4 w0 = *(const float4*)&p_s[qh][64 * wave + 32 * ks + kq];
      const float4 w1 = *(const float4*)&p_s[qh][64 * wave + 32 * ks + kq + 4];
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t h0, m0, l0, h1, m1, l1;
        split3(wv[2 * e2], h0, m0, l0);
        split3(wv[2 * e2 + 1], h1, m1, l1);
        ph[e2] = (int)(h0 | (h1 << 16));
        pm[e2] = (int)(m0 | (m1 << 16));
        pl[e2] = (int)(l0 | (l1 << 16));
      }
    }
    // v_s[wave] is this wave's own: its LDS writes and reads complete in order,
    // so only the compiler must keep them in order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4>(&v_s[wave][tr_row][16 * nt + tr_col]));
      const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4>(&v_s[wave][tr_row + 4][16 * nt + tr_col]));
      const i32x2 r0d = __builtin_bit_cast(i32x2, r0), r1d = __builtin_bit_cast(i32x2, r1);
      const i32x4 vbop = {r0d[0], r0d[1], r1d[0], r1d[1]};
      const bf16x8 vop = __builtin_bit_cast(bf16x8, vbop);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph), vop, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pm), vop, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl), vop, o[nt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();  // acc_s overlaps every wave's staging rows

  // per-wave outputs (lane l: column 16 nt + l % 16, heads 4 (l / 16) + r), then
  // the four waves added in order
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_s[wave][4 * (lane >> 4) + r][16 * nt + qh] = o[nt][r];
  __syncthreads();

  const int64_t base = ((int64_t)t * p.H + (int64_t)kvh * G) * p.nsplit + s;  // (t, head kvh*G, s)
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    const float v = ((acc_s[0][h][d] + acc_s[1][h][d]) + acc_s[2][h][d]) + acc_s[3][h][d];
    p.ws_acc[(base + (int64_t)h * p.nsplit) * D + d] = v;
  }
  if (tid == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p.ws_ml[(base + (int64_t)h * p.nsplit) * 2] = m[h];
      p.ws_ml[(base + (int64_t)h * p.nsplit) * 2 + 1] = l[h];
    }
  }
}

// Merge: one workgroup per (token, query head, slice of output elements), so
// that long contexts (many splits) still spread over the chip.
//   m = max_s m_s (exact in any order), then per chunk of 256 splits the weights
//   w_s = exp(m_s - m) and l_s go to LDS.
//   Each output element has kLanes = 32 fp32 accumulator lanes: lane a takes
//   the splits s = a, a + 32, a + 64, ... in ascending order (one fma chain for
//   the weight sum, one for the weighted values). The lanes are then added in
//   a fixed tree: P_r = (lane r + lane r+8) + (lane r+16 + lane r+24) for
//   r = 0..7, and P_0 + P_1 + ... + P_7 in ascending r.
// The arithmetic depends on the number of splits only. kRt threads share an
// element (each holding 32 / kRt lanes): 8 when there are many (token, head)
// pairs, 32 when there are few and each has many splits. Both give the same
// bytes; the choice only sets how many workgroups the merge spreads over.
constexpr int kMergeLanes = 32;

template <int D, bool kBf16, int kRt>
__global__ __launch_bounds__(kThreads)
void bigemm_attn_merge_kernel(AttnParams p) {
  constexpr int E = kThreads / kRt;        // output elements per workgroup
  constexpr int kLpt = kMergeLanes / kRt;  // accumulator lanes per thread
  constexpr int kChunk = kThreads;
  static_assert(kChunk % kMergeLanes == 0, "chunks keep the lane of every split");
  static_assert(D % E == 0, "slices tile the head");
  __shared__ float w_s[kChunk];
  __shared__ float l_s[kChunk];
  __shared__ float red[4];
  __shared__ float part_a[kMergeLanes][E];
  __shared__ float part_l[kMergeLanes][E];
  constexpr int kSlices = D / E;
  // Placement only: workgroups are dispatched round-robin over the 8 XCDs.
  // When slices are narrower than a 128-byte line of the partials (E < 32),
  // renumbering them so that consecutive numbers share an XCD keeps the
  // slices of one (token, head) on one L2.
  const int nwg = (int)gridDim.x, per = nwg / 8, bid = (int)blockIdx.x;
  const int vb = (E < 32 && bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
  const int th = vb / kSlices;  // t * H + h
  const int ei = threadIdx.x % E;
  const int e = (vb % kSlices) * E + ei;
  const int rt = threadIdx.x / E;       // this thread's lanes: rt + kRt * q
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = th / p.H;
  const int sq = p.seq_ids[t], pos = p.positions[t];
  const bool valid = !(sq < 0 || sq >= p.num_seqs || pos < 0 || pos >= p.max_context);
  const int ns = valid ? pos / kAttnSplit + 1 : 0;
  const float* ml = p.ws_ml + (int64_t)th * p.nsplit * 2;
  const float* ac = p.ws_acc + (int64_t)th * p.nsplit * D + e;

  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kThreads) mloc = fmaxf(mloc, ml[2 * s]);
  mloc = wave_reduce63<true>(mloc);
  if (lane == 63) red[wave] = mloc;
  __syncthreads();
  const float mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float la[kLpt], aa[kLpt];
#pragma unroll
  for (int q = 0; q < kLpt; ++q) la[q] = aa[q] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += kChunk) {
    if (c0 + tid < ns) {
      w_s[tid] = expf(ml[2 * (c0 + tid)] - mx);
      l_s[tid] = ml[2 * (c0 + tid) + 1];
    }
    __syncthreads();
    const int cn = min(kChunk, ns - c0);
#pragma unroll 4
    for (int j0 = 0; j0 < cn; j0 += kMergeLanes) {
#pragma unroll
      for (int q = 0; q < kLpt; ++q) {
        const int j = j0 + rt + kRt * q;
        if (j < cn) {
          la[q] = fmaf(w_s[j], l_s[j], la[q]);
          aa[q] = fmaf(w_s[j], ac[(int64_t)(c0 + j) * D], aa[q]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < kLpt; ++q) {
    part_l[rt + kRt * q][ei] = la[q];
    part_a[rt + kRt * q][ei] = aa[q];
  }
  __syncthreads();
  if (threadIdx.x >= E) return;
  float l = 0.f, a = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float pl = (part_l[r][ei] + part_l[r + 8][ei]) + (part_l[r + 16][ei] + part_l[r + 24][ei]);
    const float pa = (part_a[r][ei] + part_a[r + 8][ei]) + (part_a[r + 16][ei] + part_a[r + 24][ei]);
    l = r == 0 ? pl : l + pl;
    a = r == 0 ? pa : a + pa;
  }
  const float o = valid ? a / l : __builtin_nanf("");
  if (kBf16)
    ((uint16_t*)p.O)[(int64_t)th * D + e] = (uint16_t)f32_to_bf16_rne(__float_as_uint(o));
  else
    ((float*)p.O)[(int64_t)th * D + e] = o;
}

__global__ __launch_bounds__(256)
void bigemm_kv_write_kernel(KvWriteParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = p.D / 8;  // 16-byte chunks per row
  if (idx >= (int64_t)p.T * p.Hkv * cpr) return;
  const int c = (int)(idx % cpr);
  const int64_t r = idx / cpr;  // t * Hkv + kvh
  const int kvh = (int)(r % p.Hkv);
  const int t = (int)(r / p.Hkv);
  const int sq = p.seq_ids[t], pos = p.positions[t];
  if (sq < 0 || sq >= p.num_seqs || pos < 0 || (int64_t)pos >= ((int64_t)p.max_blocks << p.bs_log2)) return;
  const int blk = p.block_table[(int64_t)sq * p.max_blocks + (pos >> p.bs_log2)];
  if (blk < 0 || blk >= p.num_blocks) return;
  const int64_t dst = slot_row(blk, p.Hkv, kvh, p.bs_log2, pos) * p.D + c * 8;
  const int64_t src = r * p.D + c * 8;
  *(i32x4*)(p.K + dst) = *(const i32x4*)(p.K_new + src);
  *(i32x4*)(p.V + dst) = *(const i32x4*)(p.V_new + src);
}

// One instantiation per group size G = H / Hkv in 1..16 (the callers check the range).
template <int D, int G>
void launch_split_g(const AttnParams& p, hipStream_t stream, dim3 grid) {
  if (p.H / p.Hkv == G) {
    hipLaunchKernelGGL((bigemm_attn_split_kernel<D, G>), grid, dim3(kThreads), 0, stream, p);
  } else if constexpr (G < 16) {
    launch_split_g<D, G + 1>(p, stream, grid);
  }
}

template <int D>
void launch_split(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.T * p.Hkv * p.nsplit));
  launch_split_g<D, 1>(p, stream, grid);
}

// Eight threads per element (32 elements per workgroup) unless that leaves
// fewer than 2048 workgroups; then 32 threads per element (8 per workgroup).
// The output bytes are the same either way.
constexpr int64_t kMergeWideBelow = 2048;

template <int D, int kRt>
void launch_merge_rt(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.T * p.H * (D / (kThreads / kRt))));
  if (p.out_bf16)
    hipLaunchKernelGGL((bigemm_attn_merge_kernel<D, true, kRt>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((bigemm_attn_merge_kernel<D, false, kRt>), grid, dim3(kThreads), 0, stream, p);
}

template <int D>
void launch_merge(const AttnParams& p, hipStream_t stream) {
  if ((int64_t)p.T * p.H * (D / 32) < kMergeWideBelow) launch_merge_rt<D, 32>(p, stream);
  else launch_merge_rt<D, 8>(p, stream);
}

}  // namespace

hipError_t launch_paged_attention(const AttnParams& p, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  if (p.D == 64) launch_split<64>(p, stream);
  else launch_split<128>(p, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 64) launch_merge<64>(p, stream);
  else launch_merge<128>(p, stream);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.T * p.Hkv * (p.D / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bigemm_kv_write_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bigemm
