/*
 * bigemm — batch-invariant matrix multiply Y = X * W for AMD Instinct MI355X (gfx950).
 *
 * Batch invariance is the property the CANN ops-transformer issue defines in
 * its problem statement: output row i is a function of input row i and the
 * shared weight only, y[i] = f(x[i], W), never of the other rows. The
 * nondeterminism blog (section "batch-invariant matrix multiplication")
 * gives the recipe: keep the whole K reduction of each output tile inside one
 * worker, never split K, and compile exactly one kernel configuration that
 * every shape uses. This library is that recipe on CDNA4: one fixed tile
 * configuration per input type, the K blocks walked in ascending order by a
 * single workgroup, one MFMA shape at every M, no atomics, no workspace.
 * (When a product has few tiles and a long K, otherwise idle CUs also run
 * workgroups that only read the tiles' next K blocks into the L2 cache; they
 * store nothing and change no output byte.)
 * The same rules give the other entry points below: handles that take W as
 * [N, K] rows (a linear layer's weight layout) with the same output bytes, an
 * opt-in split-K whose split count follows K only, a batch-invariant RMSNorm,
 * and batch-invariant paged decode attention (a KV-cache write plus attention
 * with a fixed split size); each states its own invariance guarantee.
 *
 * Consequences the caller can rely on for the matrix multiply (per handle,
 * device and library build):
 *   - the bytes of Y[i, :] depend only on the bytes of X[i, :] (and of
 *     X_scale[i, :] for MXFP8), on W (and W_scale), on N, K and the
 *     leading dimensions' validity — not on M, not on the contents of other
 *     rows, not on i itself (the row's position in the batch);
 *   - repeated calls on the same inputs give identical bytes.
 *
 * All functions are C ABI, never throw, and return a bigemm_status.
 */
#ifndef BIGEMM_H
#define BIGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BIGEMM_ABI_VERSION 8

/* Exported entry points (the library is built with hidden visibility by default). */
#if defined(__GNUC__)
#define BIGEMM_API __attribute__((visibility("default")))
#else
#define BIGEMM_API
#endif

typedef struct bigemm_s* bigemm_t;

typedef enum {
  BIGEMM_OK = 0,
  BIGEMM_ERR_ARG = 1,          /* invalid argument; nothing was launched                    */
  BIGEMM_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or dtype combination not provided   */
  BIGEMM_ERR_DEVICE = 3,       /* a HIP call or the kernel launch failed                     */
  BIGEMM_ERR_NOMEM = 4,        /* host allocation of the handle failed                       */
  BIGEMM_ERR_SCRATCH = 5       /* bigemm_run_split_k_static: more scratch than the static
                                  buffer holds (BIGEMM_STATIC_SCRATCH_BYTES); nothing launched */
} bigemm_status;

typedef enum {
  BIGEMM_BF16 = 1,  /* bfloat16: the top 16 bits of an IEEE binary32                            */
  BIGEMM_F32 = 2,   /* IEEE binary32                                                           */
  BIGEMM_E4M3 = 3,  /* OCP E4M3FN (bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN)    */
  BIGEMM_E8M0 = 4,  /* OCP E8M0 block scale, 2^(byte - 127), 0xFF = NaN                         */
  BIGEMM_F16 = 5,   /* IEEE binary16                                                           */
  BIGEMM_I8 = 6,    /* two's-complement signed 8-bit integer                                   */
  BIGEMM_I32 = 7    /* two's-complement signed 32-bit integer                                  */
} bigemm_dtype;

/*
 * Operation descriptor. The combinations provided:
 *   bf16:  x_type = w_type = BIGEMM_BF16, y_type = BIGEMM_F32 or BIGEMM_BF16, scale_block = 0
 *   fp16:  x_type = w_type = BIGEMM_F16,  y_type = BIGEMM_F32 or BIGEMM_BF16, scale_block = 0
 *   MXFP8: x_type = w_type = BIGEMM_E4M3, y_type = BIGEMM_F32 or BIGEMM_BF16, scale_block = 32
 *          (one E8M0 scale per 32 consecutive K elements — the MXFP8 path with a
 *          K-varying scale named in the CANN issue's background and grid)
 *   int8:  x_type = w_type = BIGEMM_I8,   y_type = BIGEMM_I32, scale_block = 0
 *          (exact integer products and sums; integer addition is associative, so
 *          the result does not depend on the order at all — barring overflow,
 *          which cannot occur for K < 2^31 / 128^2 = 131072)
 * Floating-point inputs accumulate in fp32 in the one fixed order. A BIGEMM_BF16
 * output is that fp32 accumulator rounded once, to nearest even (a NaN becomes
 * a quiet NaN of the same sign: the top 16 bits with bit 6 set); it is
 * therefore exactly the rounding of the BIGEMM_F32 result of the same call.
 * The BI, fixed-order and fail-closed rules the blog and the CANN issue state
 * for the matmul hold for every combination. Fields are int32_t (holding
 * bigemm_dtype values) to keep the struct layout fixed.
 */
typedef struct {
  int32_t x_type;
  int32_t w_type;
  int32_t y_type;
  int32_t scale_block;
} bigemm_desc;

/*
 * Create a handle for the current HIP device.
 * Takes no M, N or K: the configuration cannot depend on the problem shape.
 * Returns BIGEMM_ERR_UNSUPPORTED on any device other than gfx950 and for any
 * descriptor other than those above — it never falls back to another path.
 * Ownership: the handle owns only immutable configuration; free it with
 * bigemm_destroy. *out is set to NULL on failure.
 */
BIGEMM_API bigemm_status bigemm_create(const bigemm_desc* desc, bigemm_t* out);

/*
 * Enqueue Y = X * W on `stream` (a hipStream_t; NULL = the null stream) and
 * return without synchronising.
 *
 * Shapes and layouts (row-major, leading dimensions in ELEMENTS):
 *   X [M, K], leading dimension ldx >= K     (bf16 / fp16 bits, E4M3 or int8 bytes)
 *   W [K, N], leading dimension ldw >= N     (same type as X)
 *   Y [M, N], leading dimension ldy >= N     (float32, bf16 or int32; written, never read)
 *   MXFP8 only:
 *   X_scale [M, K/32], leading dimension ldxs >= K/32   (E8M0 bytes)
 *   W_scale [K/32, N], leading dimension ldws >= N      (E8M0 bytes)
 * Each X element at [i, k] is multiplied by 2^(X_scale[i, k/32] - 127) and
 * each W element at [k, j] by 2^(W_scale[k/32, j] - 127).
 *
 * Requirements (violations return BIGEMM_ERR_ARG synchronously; nothing is
 * launched and Y is untouched):
 *   M >= 0, N >= 1, K >= 1; M == 0 is a successful no-op;
 *   bf16, fp16: any K and N;  MXFP8: K % 32 == 0, N % 16 == 0;
 *   int8: K % 16 == 0, N % 16 == 0;
 *   X, W, Y non-NULL when M > 0, 16-byte aligned; ldx, ldw, ldy such that
 *   every row starts 16-byte aligned (ldx, ldw, ldy times the element size
 *   multiples of 16). The operand tiles move in 16-byte pieces, and this
 *   alignment is the one rule that keeps every piece inside its row; a
 *   caller whose K (or N) leaves rows of another length pads the rows (the
 *   padding values are never used) rather than the library picking a second
 *   load path by layout;
 *   bf16, fp16 with K % 8 != 0 (or N % 8 != 0): the last 16-byte piece of a
 *   row of X (of W) also covers up to 7 padding elements past K (past N).
 *   Those are read, so the padding must be readable memory (it always is
 *   within a row of ld elements), and never used: X values past K are set to
 *   zero before the multiply (W rows past K are never read), and W columns
 *   past N reach only output columns that are not stored;
 *   MXFP8: X_scale, W_scale non-NULL (no alignment requirement);
 *   other types: X_scale and W_scale NULL;
 *   128 * ldx, 128 * ldw, 128 * ldy times the element size below 2^31.
 * Y must not overlap X, W or the scales (not checked).
 *
 * Memory: all buffers are device memory owned by the caller. The library
 * allocates nothing per call (this path has no split-K and hence no workspace).
 * Y is written with non-temporal stores (a finished tile's output does not
 * stay in the L2 that the other tiles' operands use), so a kernel reading Y
 * right after the call finds it past the L2.
 * Device: the current HIP device must be the one the handle was created on
 * (BIGEMM_ERR_ARG otherwise, checked on the host before anything is launched).
 * Errors: BIGEMM_ERR_ARG as above; BIGEMM_ERR_DEVICE if the launch fails (the
 * HIP error is consumed). Concurrent calls on different streams are safe;
 * bigemm_destroy must not race with calls in flight.
 */
BIGEMM_API bigemm_status bigemm_run(bigemm_t h, int64_t M, int64_t N, int64_t K,
                         const void* X, int64_t ldx,
                         const void* W, int64_t ldw,
                         void* Y, int64_t ldy,
                         const void* X_scale, int64_t ldxs,
                         const void* W_scale, int64_t ldws,
                         void* stream);

/*
 * Opt-in split-K handle (bf16 and fp16 inputs; fp32 or bf16 output): the
 * pinned-split, ordered-merge deterministic split-K that the vLLM mHC pull
 * request ("What") pins and that the nondeterminism blog (section on
 * batch-invariant matmul) names as what breaks invariance when the split
 * count follows the batch. Here the split count follows K only:
 *   - the K range of every output tile is cut into ceil(K / k_chunk) chunks of
 *     k_chunk values (k_chunk a positive multiple of 64, fixed per handle);
 *   - one workgroup per (tile, chunk) accumulates its chunk in fp32 in the
 *     same fixed order as bigemm_run and stores the chunk sum to the workspace;
 *   - a second kernel adds the chunk sums in ascending chunk order (fp32),
 *     then rounds once to bf16 for a bf16 output.
 * Rows stay batch-invariant (nothing depends on M or on other rows), and the
 * same call repeated gives the same bytes. The bytes differ from those of an
 * unsplit handle whenever K > k_chunk (another fixed summation tree); with
 * K <= k_chunk they are identical. The point is occupancy: at small M the
 * unsplit kernel has ceil(M/128)*ceil(N/128) tiles, each reduced by one
 * workgroup, this one that many workgroups times the chunk count.
 * Returns BIGEMM_ERR_ARG for a bad k_chunk, BIGEMM_ERR_UNSUPPORTED for other
 * descriptors or devices. Run it with bigemm_run_ws (bigemm_run returns
 * BIGEMM_ERR_ARG on such a handle: it needs a workspace).
 */
BIGEMM_API bigemm_status bigemm_create_split_k(const bigemm_desc* desc, int32_t k_chunk, bigemm_t* out);

/*
 * The split-K handle above with W given as [N, K] rows (ldw >= K), as for
 * bigemm_create_wt: the same chunks, chunk sums and ordered merge, with W's
 * tile staged from the transposed layout, so the bytes equal those of a
 * bigemm_create_split_k handle with the same k_chunk given W as [K, N].
 * bf16 and fp16 inputs; errors as bigemm_create_split_k. Run with
 * bigemm_run_ws.
 */
BIGEMM_API bigemm_status bigemm_create_split_k_wt(const bigemm_desc* desc, int32_t k_chunk, bigemm_t* out);

/*
 * Handle whose W is given as its transpose: an [N, K] row-major array with
 * leading dimension ldw >= K (the layout in which a linear layer keeps its
 * weight), so such a weight needs no copy. For MXFP8, W_scale is then
 * [N, K/32] with ldws >= K/32 (W's E8M0 scales next to its rows, as X_scale
 * is for X). Every descriptor of bigemm_create is accepted.
 * It is the same multiply, Y = X * W with W[k, j] read from element [j, k]
 * of that array (and its scale from W_scale[j, k/32]), under the same fixed
 * recipe as bigemm_run: one tile configuration, the whole K in one
 * workgroup, ascending K blocks, one MFMA shape. The MFMA chain sees the
 * same operands and scales in the same order, so Y has exactly the bytes of
 * a bigemm_create handle given the same logical W as [K, N]. Only the staging
 * of W's tile and scales differs.
 * Run it with bigemm_run or bigemm_run_ws (no workspace). The requirements of
 * bigemm_run hold with ldw >= K in place of ldw >= N (for bf16 / fp16 with
 * K % 8 != 0 the padding past K of W's rows is read and zeroed like X's) and, for MXFP8,
 * ldws >= K/32 in place of ldws >= N and 128 * ldws below 2^31. Devices other
 * than gfx950 return BIGEMM_ERR_UNSUPPORTED. bigemm_create_split_k_wt is its
 * split-K form (bf16 and fp16).
 * *out is NULL on failure.
 */
BIGEMM_API bigemm_status bigemm_create_wt(const bigemm_desc* desc, bigemm_t* out);

/*
 * The argument checks of a bigemm_create_wt handle's bigemm_run, as a pure
 * host function (no HIP call): W [N, K] with ldw >= K, MXFP8 W_scale
 * [N, K/32] with ldws >= K/32; otherwise as bigemm_check_args.
 */
BIGEMM_API bigemm_status bigemm_check_args_wt(const bigemm_desc* desc, int64_t M, int64_t N, int64_t K,
                                   const void* X, int64_t ldx, const void* W, int64_t ldw,
                                   const void* Y, int64_t ldy, const void* X_scale, int64_t ldxs,
                                   const void* W_scale, int64_t ldws);

/*
 * Device workspace, in bytes, that bigemm_run_ws needs for this shape:
 * ceil(K / k_chunk) * M * N * 4 for a split-K handle when K > k_chunk, 0
 * otherwise (an unsplit handle, or a single chunk). Pure host function.
 * BIGEMM_ERR_ARG for a NULL handle or output, or negative sizes.
 */
BIGEMM_API bigemm_status bigemm_workspace_size(bigemm_t h, int64_t M, int64_t N, int64_t K, uint64_t* bytes);

/*
 * bigemm_run with a caller-provided device workspace (16-byte aligned, at least
 * bigemm_workspace_size bytes; it may be NULL when that size is 0). The
 * library allocates nothing. The workspace is scratch for the duration of the
 * call on `stream`: calls that share a workspace must be ordered (same stream)
 * or they race. For a handle without split-K this is bigemm_run. Errors as
 * bigemm_run, plus BIGEMM_ERR_ARG when the run splits K (K > k_chunk) and
 *   - the workspace is missing, misaligned or short, or
 *   - 128 * N * 4 >= 2^31 (the chunk sums are fp32 rows of N values, addressed
 *     through 32-bit offsets within a 128-row tile, whatever the output type).
 */
BIGEMM_API bigemm_status bigemm_run_ws(bigemm_t h, int64_t M, int64_t N, int64_t K,
                            const void* X, int64_t ldx,
                            const void* W, int64_t ldw,
                            void* Y, int64_t ldy,
                            const void* X_scale, int64_t ldxs,
                            const void* W_scale, int64_t ldws,
                            void* workspace, uint64_t workspace_bytes,
                            void* stream);

/* Size of the static device scratch buffer of bigemm_run_split_k_static. */
#define BIGEMM_STATIC_SCRATCH_BYTES (64ull << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * bigemm_run_ws call of a split-K handle (bigemm_create_split_k or
 * bigemm_create_split_k_wt) with the chunk sums kept in the library's own
 * static device buffer instead of a caller workspace. Same kernels, so Y has
 * the bytes of bigemm_run_ws on the same handle and inputs.
 *   - The buffer is a file-scope device array of BIGEMM_STATIC_SCRATCH_BYTES
 *     (64 MiB); every GPU the library runs on holds its own copy until the
 *     process ends. Its device address is looked up once per device when a
 *     split-K handle is created there. This call allocates nothing (no
 *     hipMalloc, no allocating library routine).
 *   - The chunk sums need ceil(K / k_chunk) * M * N * 4 bytes (0 when
 *     K <= k_chunk: then the unsplit kernel runs and the buffer is unused).
 *     More than BIGEMM_STATIC_SCRATCH_BYTES returns BIGEMM_ERR_SCRATCH and
 *     launches nothing; use bigemm_run_ws with a workspace for such shapes.
 *   - Every element the merge reads is written by the same call first, so the
 *     buffer needs no clearing and the previous call's contents never reach Y.
 *   - All calls on one GPU share that GPU's buffer: calls that overlap on one
 *     GPU (different streams, or host threads without ordering) race and may
 *     return wrong results. Order them on one stream.
 * Errors as bigemm_run_ws (BIGEMM_ERR_ARG also for a handle without split-K).
 */
BIGEMM_API bigemm_status bigemm_run_split_k_static(bigemm_t h, int64_t M, int64_t N, int64_t K,
                                                   const void* X, int64_t ldx,
                                                   const void* W, int64_t ldw,
                                                   void* Y, int64_t ldy,
                                                   void* stream);

/*
 * The argument checks of bigemm_run_ws on a split-K handle created from
 * (desc, k_chunk), W given as [K, N], as a pure host function (no HIP call):
 * those of bigemm_check_args plus the workspace and size limits listed under
 * bigemm_run_ws. BIGEMM_ERR_UNSUPPORTED for descriptors that have no split-K
 * form, BIGEMM_ERR_ARG for a bad k_chunk.
 */
BIGEMM_API bigemm_status bigemm_check_args_split_k(const bigemm_desc* desc, int32_t k_chunk,
                                                   int64_t M, int64_t N, int64_t K,
                                                   const void* X, int64_t ldx,
                                                   const void* W, int64_t ldw,
                                                   const void* Y, int64_t ldy,
                                                   const void* workspace, uint64_t workspace_bytes);

/*
 * Batch-invariant RMSNorm, the blog's section "batch-invariant RMSNorm":
 *   Y[i, j] = X[i, j] / sqrt((1/D) * sum_k X[i, k]^2 + eps) * gamma[j]
 * with the data-parallel strategy it recommends and no small-batch switch: one
 * workgroup per row at every M, the row's sum of squares accumulated in fp32 in
 * an order fixed by D alone, then rounded once to the output type. Each output
 * row depends only on its input row, gamma, D and eps.
 *   dtype: BIGEMM_BF16 (X, gamma, Y bf16) or BIGEMM_F32 (all fp32)
 *   X [M, D] (ldx >= D), gamma [D], Y [M, D] (ldy >= D), row-major, elements.
 * Requirements (else BIGEMM_ERR_ARG, nothing launched): M >= 0 (M == 0 is a
 * no-op), 8 <= D <= 65536, D % 8 == 0; X, gamma, Y non-NULL and 16-byte aligned
 * with every row 16-byte aligned; M <= 2^31 - 1. Y may equal X (in place) but
 * must not otherwise overlap X or gamma. BIGEMM_ERR_UNSUPPORTED on a device
 * other than gfx950 (checked once per device, never a fallback). Enqueued on
 * `stream` without synchronising; allocates nothing.
 */
BIGEMM_API bigemm_status bigemm_rmsnorm(int32_t dtype, int64_t M, int64_t D,
                             const void* X, int64_t ldx,
                             const void* gamma,
                             void* Y, int64_t ldy,
                             float eps, void* stream);

/* The argument checks of bigemm_rmsnorm as a pure host function (no HIP call). */
BIGEMM_API bigemm_status bigemm_rmsnorm_check_args(int32_t dtype, int64_t M, int64_t D,
                                        const void* X, int64_t ldx, const void* gamma,
                                        const void* Y, int64_t ldy);

/*
 * ---------------------------------------------------------------------------
 * Batch-invariant paged attention (the nondeterminism blog, section
 * "batch-invariant attention").
 *
 * A query token t of sequence seq_ids[t] at position positions[t] = i attends
 * to the keys and values of that sequence at positions 0..i (the causal mask):
 *   O[t, h] = sum_{j <= i} softmax_j(scale * Q[t, h] . K_j) V_j,
 * with query head h reading key/value head h / (num_heads / num_kv_heads)
 * (grouped-query attention). Decode is one token per sequence at its last
 * position; a chunk of prefill is several tokens of one sequence at consecutive
 * positions. The section's two rules are the interface:
 *   - the KV cache and the page table are updated BEFORE attention:
 *     bigemm_kv_cache_write puts the new tokens' keys and values into the
 *     cache, then bigemm_paged_attention reads every position 0..i from the
 *     cache in the same layout, whether it was cached by an earlier call or
 *     written just now — so splitting a sequence into chunks, or processing
 *     it all at once, does not change a token's result;
 *   - the KV range is cut into splits of a FIXED SIZE, BIGEMM_ATTN_SPLIT
 *     positions (never a fixed number of splits). Each split is reduced by one
 *     workgroup in a fixed order (fp32), and the splits are merged in a
 *     fixed tree that depends only on their number; the merge is rounded once
 *     to the output type.
 * So the bytes of O[t, :, :] depend only on Q[t], on the keys and values of
 * positions 0..i of its sequence, on i and on scale — not on T, on the other
 * tokens, on the token's index t, on which physical blocks hold the positions,
 * on max_context or on the workspace. Repeated calls give identical bytes.
 */
#define BIGEMM_ATTN_SPLIT 256

/*
 * The paged KV cache. K and V are separate device arrays of bf16, each
 *   [num_blocks][num_kv_heads][block_size][head_dim], row-major,
 * and the block table is a device array of int32 [num_seqs][max_blocks]:
 * position j of sequence s lives in block block_table[s][j / block_size] at
 * row j % block_size. The caller owns the cache, assigns the blocks (the page
 * table) and keeps each table row's entries for positions 0..i valid.
 */
typedef struct {
  int32_t num_kv_heads;  /* >= 1                                          */
  int32_t head_dim;      /* 64 or 128                                     */
  int32_t block_size;    /* positions per block: a power of two, 1..4096  */
  int32_t num_blocks;    /* blocks in each of K and V, >= 1               */
  int32_t num_seqs;      /* rows of the block table, >= 1                 */
  int32_t max_blocks;    /* entries per block-table row, >= 1             */
} bigemm_kv_layout;

/*
 * Write the keys and values of T new tokens into the cache:
 *   K_cache[slot(t, kvh)] = K_new[t, kvh, :], same for V, for every KV head,
 * where slot is the row of position positions[t] of sequence seq_ids[t].
 *   K_new, V_new [T][num_kv_heads][head_dim] bf16; seq_ids, positions [T] int32.
 * A token whose sequence, position (< max_blocks * block_size) or block id
 * (< num_blocks) is out of range is skipped; nothing outside the caches is
 * written. Two tokens with the same slot race (the caller's error).
 * Requirements (else BIGEMM_ERR_ARG, nothing launched): the layout as above,
 * T >= 0 (0 is a no-op), T * num_kv_heads * head_dim / 8 < 2^31; pointers
 * non-NULL when T > 0, the bf16 arrays 16-byte aligned, the int32 arrays
 * 4-byte aligned. BIGEMM_ERR_UNSUPPORTED on a device other than gfx950.
 * Enqueued on `stream`; allocates nothing.
 */
BIGEMM_API bigemm_status bigemm_kv_cache_write(const bigemm_kv_layout* kv, int64_t T,
                                    const void* K_new, const void* V_new,
                                    const int32_t* seq_ids, const int32_t* positions,
                                    const int32_t* block_table,
                                    void* K_cache, void* V_cache, void* stream);

/*
 * Device workspace, in bytes, for bigemm_paged_attention:
 *   T * num_heads * ceil(max_context / BIGEMM_ATTN_SPLIT) * (head_dim + 2) * 4.
 * Pure host function; BIGEMM_ERR_ARG for arguments bigemm_paged_attention
 * would reject (other than pointers).
 */
BIGEMM_API bigemm_status bigemm_attn_workspace_size(const bigemm_kv_layout* kv, int64_t T, int32_t num_heads,
                                         int32_t max_context, uint64_t* bytes);

/*
 * Enqueue the attention of T query tokens over the cache on `stream`.
 *   Q [T][num_heads][head_dim] bf16; O [T][num_heads][head_dim], out_dtype
 *   BIGEMM_F32 or BIGEMM_BF16; seq_ids, positions [T] int32 (device);
 *   max_context: an upper bound on positions[t] + 1, at most
 *   max_blocks * block_size (it sizes the grid and the workspace only);
 *   scale: the score scale, normally 1/sqrt(head_dim) rounded to float.
 * num_heads must be num_kv_heads times G, 1 <= G <= 16 (a group's query heads
 * are the rows of one 16-row MFMA tile).
 * Data-dependent cases, handled on the device without faulting: a token whose
 * sequence or position is out of range (position >= max_context included)
 * gets an all-NaN output; a block-table entry outside [0, num_blocks) reached
 * by a token's positions makes that token's output NaN. Scores beyond the fp32
 * range give inf or NaN.
 * Requirements (else BIGEMM_ERR_ARG, nothing launched): the layout as above;
 * T >= 0 (0 is a no-op); 1 <= max_context <= max_blocks * block_size; the
 * grids T * num_kv_heads * splits and T * num_heads * head_dim / 32 below 2^31; pointers
 * non-NULL when T > 0, Q, the caches, O and the workspace 16-byte aligned, the
 * int32 arrays 4-byte aligned; workspace_bytes >= bigemm_attn_workspace_size.
 * O must not overlap the inputs or the workspace. The workspace is scratch for
 * the call: calls sharing one must be ordered on one stream.
 * BIGEMM_ERR_UNSUPPORTED on a device other than gfx950. Allocates nothing.
 */
BIGEMM_API bigemm_status bigemm_paged_attention(const bigemm_kv_layout* kv, int64_t T, int32_t num_heads,
                                     int32_t max_context, float scale, int32_t out_dtype,
                                     const void* Q, const void* K_cache, const void* V_cache,
                                     const int32_t* seq_ids, const int32_t* positions,
                                     const int32_t* block_table, void* O,
                                     void* workspace, uint64_t workspace_bytes, void* stream);

/* The argument checks of bigemm_paged_attention as a pure host function (no HIP call). */
BIGEMM_API bigemm_status bigemm_paged_attention_check_args(const bigemm_kv_layout* kv, int64_t T,
                                                int32_t num_heads, int32_t max_context,
                                                int32_t out_dtype, const void* Q,
                                                const void* K_cache, const void* V_cache,
                                                const int32_t* seq_ids, const int32_t* positions,
                                                const int32_t* block_table, const void* O,
                                                const void* workspace, uint64_t workspace_bytes);

/* Release a handle. NULL is accepted. */
BIGEMM_API bigemm_status bigemm_destroy(bigemm_t h);

/* Static, NUL-terminated description of a status code. */
BIGEMM_API const char* bigemm_status_str(bigemm_status s);

/*
 * The one compiled tile configuration behind a handle (evidence that it is
 * fixed): output tile bm x bn and K-block bk. Any output pointer may be NULL.
 */
BIGEMM_API bigemm_status bigemm_get_config(bigemm_t h, int32_t* bm, int32_t* bn, int32_t* bk);

/*
 * The argument checks bigemm_run performs, as a pure host function: no HIP
 * call, no device access, pointers are only tested for NULL and alignment.
 */
BIGEMM_API bigemm_status bigemm_check_args(const bigemm_desc* desc, int64_t M, int64_t N, int64_t K,
                                const void* X, int64_t ldx,
                                const void* W, int64_t ldw,
                                const void* Y, int64_t ldy,
                                const void* X_scale, int64_t ldxs,
                                const void* W_scale, int64_t ldws);

/* BIGEMM_ABI_VERSION of the loaded library. */
BIGEMM_API int32_t bigemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BIGEMM_H */
