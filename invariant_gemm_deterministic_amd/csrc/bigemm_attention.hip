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
// the KV head. Thread layout: groups of D/8 lanes; lane gl of a group holds
// elements [8 gl, 8 gl + 8) of a row, and group g reads positions
// g, g + 256/(D/8), ... of the split (16 B per lane, a row per group).
//   scores: each lane forms 8-element partial dot products (v_dot2_f32_bf16 in
//           a fixed order) for its group's positions, then a reduce-scatter
//           butterfly over the group's lanes leaves every thread with the full
//           dot product of exactly one position;
//   softmax: per head, the split maximum m and p_j = exp(s_j - m) (fp32), and
//           l = sum_j p_j (wave butterfly, then the four waves in order);
//   values: each lane accumulates p_j * v_j over its group's positions in
//           ascending order (fp32 FMA), a reduce-scatter butterfly over the
//           groups of a wave, then the four waves in order.
// Every butterfly step adds two partial sums of fixed, disjoint position sets,
// so each split result is a fixed function of that split's inputs.
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The elements are copied to scalars before the bit cast: a cast of the vector
// element expression itself reinterprets element 0.
__device__ __forceinline__ float dot8(const i32x4 a, const i32x4 b) {
  float d = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ac = a[c], bc = b[c];
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ac), __builtin_bit_cast(bf16x2, bc), d, false);
  }
  return d;
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Cross-lane moves. DPP: row_mirror pairs lane i of a 16-lane row with 15 - i,
// row_half_mirror pairs i with 7 - i inside each half row, the two quad
// permutations swap neighbours at distance 2 and 1, row_ror:8 pairs i with i ^ 8.
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141, kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1,
              kDppRor8 = 0x128;

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// One reduce-scatter step between partner lanes (partner differs in the bit
// `hi` tests and agrees on the bits already reduced): lanes with hi clear keep
// index k (own a + partner's a), lanes with hi set keep index k + half (own b +
// partner's b). Each kept sum is formed by exactly one lane.
template <int kCtrl>
__device__ __forceinline__ float rs_pair(float a, float b, bool hi) {
  const float sa = a + dpp<kCtrl>(a);
  const float sb = b + dpp<kCtrl>(b);
  return hi ? sb : sa;
}

// v[0..N) of every lane of an aligned group of N lanes (N = 16 or 8, a row or
// half row) are partial sums over disjoint sets; afterwards v[0] of lane i
// holds the total of index i (the lane keeps, at each step, the half its own
// bit selects).
template <int N>
__device__ __forceinline__ void reduce_scatter(float (&v)[N], int lane) {
  static_assert(N == 16 || N == 8, "a row or half row of lanes");
  if constexpr (N == 16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = rs_pair<kDppRowMirror>(v[k], v[k + 8], (lane & 8) != 0);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = rs_pair<kDppHalfMirror>(v[k], v[k + 4], (lane & 4) != 0);
#pragma unroll
  for (int k = 0; k < 2; ++k) v[k] = rs_pair<kDppQuadXor2>(v[k], v[k + 2], (lane & 2) != 0);
  v[0] = rs_pair<kDppQuadXor1>(v[0], v[1], (lane & 1) != 0);
}

// The same over the groups of a wave (lane bits 32, 16 and, for 8-lane groups,
// 8): v_permlane32_swap / v_permlane16_swap exchange the halves directly, so
// that a' + b' is own + partner for the kept index. Afterwards lane l holds
// indices [off, off + N >> steps) where off adds N/2 for lane bit 32, N/4 for
// bit 16 (and N/8 for bit 8).
template <int N, int kL>
__device__ __forceinline__ int reduce_scatter_groups(float (&v)[N], int lane) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + N / 2]), false,
                                                    false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + N / 4]), false,
                                                    false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  int off = ((lane & 32) ? N / 2 : 0) + ((lane & 16) ? N / 4 : 0);
  if constexpr (kL == 8) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) v[k] = rs_pair<kDppRor8>(v[k], v[k + N / 8], (lane & 8) != 0);
    off += (lane & 8) ? N / 8 : 0;
  }
  return off;
}

__device__ __forceinline__ int64_t slot_row(int blk, int Hkv, int kvh, int bs_log2, int j) {
  return ((((int64_t)blk * Hkv + kvh) << bs_log2) + (j & ((1 << bs_log2) - 1)));
}

template <int D, int G>
__global__ __launch_bounds__(kThreads)
void bigemm_attn_split_kernel(AttnParams p) {
  constexpr int kL = D / 8;                 // lanes per row
  constexpr int kGroups = kThreads / kL;    // rows read at once
  constexpr int kPer = kAttnSplit / kGroups;  // positions per lane
  static_assert(kPer == kL, "the score reduce-scatter leaves one position per lane");
  constexpr int kAcc = G * 8;
  __shared__ __align__(16) float p_s[G][kAttnSplit];
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ float acc_s[4][G][D];
  __shared__ int32_t blk_s[kAttnSplit];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = tid / kL, gl = tid % kL;
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

  i32x4 q[G];
  const uint16_t* qrow = p.Q + ((int64_t)t * p.H + (int64_t)kvh * G) * D + gl * 8;
#pragma unroll
  for (int h = 0; h < G; ++h) q[h] = *(const i32x4*)(qrow + h * D);
  __syncthreads();

  // Rows of this split: zero past the context, NaN where the block id is invalid.
  const i32x4 kZero = {0, 0, 0, 0};
  const i32x4 kNaN = {0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0, 0x7FC07FC0};
  i32x4 kr[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int jj = grp + kGroups * i;
    kr[i] = kZero;
    if (jj < n) {
      const int j = j0 + jj;
      const int blk = blk_s[(j >> p.bs_log2) - b0];
      kr[i] = kNaN;
      if (blk >= 0 && blk < p.num_blocks)
        kr[i] = *(const i32x4*)(p.K + slot_row(blk, p.Hkv, kvh, p.bs_log2, j) * D + gl * 8);
    }
  }

  i32x4 vr[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int jj = grp + kGroups * i;
    vr[i] = kZero;
    if (jj < n) {
      const int j = j0 + jj;
      const int blk = blk_s[(j >> p.bs_log2) - b0];
      vr[i] = kNaN;
      if (blk >= 0 && blk < p.num_blocks)
        vr[i] = *(const i32x4*)(p.V + slot_row(blk, p.Hkv, kvh, p.bs_log2, j) * D + gl * 8);
    }
  }

  const int own = grp + kGroups * gl;  // the position whose score this thread ends with
  float sh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) sc[i] = dot8(q[h], kr[i]);
    reduce_scatter<kPer>(sc, gl);
    sh[h] = own < n ? sc[0] * p.scale : -INFINITY;
  }

  // softmax statistics of the split, per head
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x = sh[h];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if (lane == 0) red_m[wave][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    const float w = expf(sh[h] - m[h]);
    p_s[h][tid] = w;
    float x = w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) red_l[wave][h] = x;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = ((red_l[0][h] + red_l[1][h]) + red_l[2][h]) + red_l[3][h];

  // p * v over this group's positions, ascending; weight of position grp + kGroups*i
  // sits at p_s[h][grp * kPer + i] (the thread that owned its score)
  float acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.f;
#pragma unroll
  for (int i4 = 0; i4 < kPer / 4; ++i4) {
    float4 w4[G];
#pragma unroll
    for (int h = 0; h < G; ++h) w4[h] = *(const float4*)&p_s[h][grp * kPer + 4 * i4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const i32x4 vv = vr[4 * i4 + ii];
      float v[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[2 * c] = __uint_as_float((uint32_t)vv[c] << 16);
        v[2 * c + 1] = __uint_as_float((uint32_t)vv[c] & 0xFFFF0000u);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = ii == 0 ? w4[h].x : ii == 1 ? w4[h].y : ii == 2 ? w4[h].z : w4[h].w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h * 8 + e] = fmaf(w, v[e], acc[h * 8 + e]);
      }
    }
  }

  // reduce-scatter over the groups of this wave
  const int off = reduce_scatter_groups<kAcc, kL>(acc, lane);
  constexpr int kOwn = kAcc * kL / 64;  // values each lane owns afterwards
#pragma unroll
  for (int k = 0; k < kOwn; ++k) {
    const int f = off + k;
    acc_s[wave][f >> 3][gl * 8 + (f & 7)] = acc[k];
  }
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

// Merge: one workgroup per (token, query head, slice of kMergeE output
// elements), so that long contexts (many splits) still spread over the chip.
//   m = max_s m_s (exact in any order), then per chunk of 256 splits the weights
//   w_s = exp(m_s - m) and l_s go to LDS;
//   thread (e, r), r < R = 256 / kMergeE, takes splits s = r + R j in ascending
//   order into kU interleaved fp32 accumulators (split s to accumulator
//   (s / R) % kU), adds them in a fixed tree, then the R partials in ascending r.
// The tree depends on the number of splits only.
constexpr int kMergeE = 32;

template <int D, bool kBf16>
__global__ __launch_bounds__(kThreads)
void bigemm_attn_merge_kernel(AttnParams p) {
  constexpr int R = kThreads / kMergeE;
  constexpr int kU = 4;
  constexpr int kChunk = kThreads;
  static_assert(kChunk % (R * kU) == 0, "chunks keep the accumulator of every split");
  __shared__ float w_s[kChunk];
  __shared__ float l_s[kChunk];
  __shared__ float red[4];
  __shared__ float part_a[R][kMergeE];
  __shared__ float part_l[R][kMergeE];
  constexpr int kSlices = D / kMergeE;
  const int th = blockIdx.x / kSlices;  // t * H + h
  const int e = (blockIdx.x % kSlices) * kMergeE + threadIdx.x % kMergeE;
  const int r = threadIdx.x / kMergeE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = th / p.H;
  const int sq = p.seq_ids[t], pos = p.positions[t];
  const bool valid = !(sq < 0 || sq >= p.num_seqs || pos < 0 || pos >= p.max_context);
  const int ns = valid ? pos / kAttnSplit + 1 : 0;
  const float* ml = p.ws_ml + (int64_t)th * p.nsplit * 2;
  const float* ac = p.ws_acc + (int64_t)th * p.nsplit * D + e;

  float mloc = -INFINITY;
  for (int s = tid; s < ns; s += kThreads) mloc = fmaxf(mloc, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float la[kU], aa[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) la[u] = aa[u] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += kChunk) {
    if (c0 + tid < ns) {
      w_s[tid] = expf(ml[2 * (c0 + tid)] - mx);
      l_s[tid] = ml[2 * (c0 + tid) + 1];
    }
    __syncthreads();
    const int cn = min(kChunk, ns - c0);
    for (int j0 = r; j0 < cn; j0 += R * kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = j0 + u * R;
        if (j < cn) {
          la[u] = fmaf(w_s[j], l_s[j], la[u]);
          aa[u] = fmaf(w_s[j], ac[(int64_t)(c0 + j) * D], aa[u]);
        }
      }
    }
    __syncthreads();
  }
  part_l[r][threadIdx.x % kMergeE] = (la[0] + la[1]) + (la[2] + la[3]);
  part_a[r][threadIdx.x % kMergeE] = (aa[0] + aa[1]) + (aa[2] + aa[3]);
  __syncthreads();
  if (r != 0) return;
  const int ei = threadIdx.x;
  float l = part_l[0][ei], a = part_a[0][ei];
#pragma unroll
  for (int i = 1; i < R; ++i) {
    l += part_l[i][ei];
    a += part_a[i][ei];
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

template <int D>
void launch_split(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.T * p.Hkv * p.nsplit));
  switch (p.H / p.Hkv) {
    case 1: hipLaunchKernelGGL((bigemm_attn_split_kernel<D, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((bigemm_attn_split_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((bigemm_attn_split_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    default: hipLaunchKernelGGL((bigemm_attn_split_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p); break;
  }
}

template <int D>
void launch_merge(const AttnParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.T * p.H * (D / kMergeE)));
  if (p.out_bf16)
    hipLaunchKernelGGL((bigemm_attn_merge_kernel<D, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((bigemm_attn_merge_kernel<D, false>), grid, dim3(kThreads), 0, stream, p);
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
