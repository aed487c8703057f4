/*
 * mla.h - absorbed Multi-head Latent Attention (MLA) decode on AMD MI355X (gfx950).
 *
 * One decode step for a batch of sequences is five operations that run in
 * stream order (the fused calls below run the same step in three launches):
 *
 *   mla_absorb_q      q~ = W_UK^T q_nope per head (the content query folded into
 *                     the latent space)
 *   mla_rope_append   rotate q_rope and the new token's shared RoPE key; write
 *                     the new cache row [c_kv_new | RoPE(k_rope_new)]
 *   mla_decode_latent split-KV attention over the latent cache: scores
 *                     q~.c_kv + q_rope.k_rope, online softmax, softmax-weighted
 *                     sum of the latents, one partial result per split
 *   mla_combine       log-sum-exp merge of the splits into o_lat
 *   mla_up_v          out = W_UV o_lat per head
 *   mla_absorb_rope   mla_absorb_q and mla_rope_append in one call (one launch
 *                     for bf16)
 *   mla_kv_down       the appended row's latent and RoPE key from the hidden
 *                     state (the step before the path)
 *   mla_*_paged       the calls that touch the cache, for a cache kept in
 *                     fixed-size pages behind a block table
 *   mla_combine_up_v  mla_combine and mla_up_v in one call: the merge is
 *                     formed where W_UV consumes it and o_lat never goes to
 *                     memory
 *   mla_*_fp8         the calls that touch the cache, for a cache whose
 *                     latents are stored in 8-bit floating point
 *   mla_fold_*        the up-projections multiplied into the query and output
 *                     weights ahead of time; mla_absorb_q_folded and
 *                     mla_out_folded use them in place of mla_absorb_q and
 *                     mla_up_v + the output projection
 *
 * Sources (page title, section):
 *   [P1] "DeepSeek MLA, Built From the Paper": section 1 (the cache holds
 *        r_kv + d_rope values per token and layer), section 2 (a decoupled
 *        RoPE key shared by all heads), section 3 (matrix absorption:
 *        q^T (W_UK c) equals (W_UK^T q)^T c, so keys are never rebuilt).
 *   [P2] "MLA from scratch" (DeepSeek 3.2 series): module structure and
 *        MLAAttention (weight shapes, latent cache), KV cache management
 *        during decode (the new latent is written at the current position and
 *        the cache grows by one row), absorbing projections (attention weights
 *        applied to the latents directly, W_UV after).
 *   [P3] "Build a DeepSeek Model (From Scratch)", chapter 3: figure captions
 *        on RoPE (dimensions rotated in pairs by a position-dependent angle)
 *        and on the decoupled architecture (content score + position score).
 *   [P5] "Multi-head latent attention" (octlm blog): the cache holds the
 *        latent and one RoPE key of width d_rope shared across heads.
 *
 * Conventions (readings where the pages leave a step open):
 *   - RoPE pairs adjacent dimensions (2i, 2i+1); pair i is turned by the angle
 *     pos * rope_base^(-2i/d_rope).  Angles and rotations are evaluated in
 *     double precision and rounded once to the storage dtype.
 *   - The new token is appended first and then attended to: a sequence with
 *     L cached tokens attends over L + 1 rows and its query sits at position L.
 *   - Cached RoPE keys are stored already rotated by their own positions.
 *   - softmax_scale <= 0 selects 1/sqrt(d_head + d_rope).
 *
 * Data layout (all row-major, contiguous, little-endian):
 *   q_nope   [B][H][d_head]          storage dtype
 *   q_rope   [B][H][d_rope]          storage dtype (not yet rotated)
 *   w_uk     [H][d_head][r]          storage dtype; the weight of a
 *                                    Linear(r -> H*d_head) reshaped per head
 *   w_uv     [H][d_v][r]             storage dtype; same for values
 *   q_lat    [B][H][r + d_rope]      storage dtype; [q~ | RoPE(q_rope)]
 *   kv_cache [total_rows][r + d_rope] storage dtype; row = [c_kv | rotated k_rope]
 *   c_kv_new [B][r], k_rope_new [B][d_rope]   storage dtype
 *   positions   [B] int32    L_b: cached tokens before the step = the new
 *                            token's position and its row index in the sequence
 *   row_offsets [B] int64    first cache row of sequence b
 *   seq_lens    [B] int32    rows attended = L_b + 1 (after the append)
 *   o_part   [B][num_splits][H][r] in the storage dtype (float32 for
 *            MLA_F32, bf16 for MLA_BF16): the partial of split s of
 *            sequence b for head h is the contiguous row (b*num_splits + s)*H
 *            + h.  A bf16 partial is the fp32 result rounded once to nearest
 *            even.
 *   lse_part [B][num_splits][H] float32
 *   o_lat    [B][H][r] float32, lse [B][H] float32, out [B][H][d_v] float32
 *   Sequence b owns cache rows [row_offsets[b], row_offsets[b] + seq_lens[b]).
 *
 * Splits: with chunk = ceil(max_seq_len / num_splits) rounded up to a
 * multiple of 32 (the kernel's row tile), split s of sequence b covers
 * in-sequence rows [s*chunk, min((s+1)*chunk, seq_lens[b])).  A split with no
 * rows writes lse_part = -inf and leaves its o_part untouched; mla_combine
 * skips it.
 *
 * Ownership and execution: the caller allocates every buffer (device memory,
 * 16-byte aligned) and owns it; the library allocates nothing, keeps no state
 * between calls and is safe to call from several host threads.  Every call
 * validates its arguments on the host, then only enqueues work on `stream`
 * (a hipStream_t; NULL = the default stream) and returns; the caller
 * synchronises.  On any error nothing is enqueued and a status code is
 * returned; nothing is thrown and nothing aborts.  Device-side metadata
 * (row_offsets, seq_lens, positions) cannot be checked on the host: rows are
 * clamped into [0, total_rows) so that inconsistent metadata gives wrong
 * numbers, never an out-of-bounds access.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, odd d_rope, bad split count */
  MLA_ERR_UNSUPPORTED = 2,  /* no kernel instantiation for these dims/dtype */
  MLA_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned */
  MLA_ERR_WORKSPACE = 4,    /* num_splits exceeds what the kernels support */
  MLA_ERR_HIP = 5           /* the HIP runtime reported an error (see mla_last_error) */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

typedef struct {
  int32_t batch;        /* B: sequences in the step */
  int32_t heads;        /* H */
  int32_t d_head;       /* content query/key width per head */
  int32_t d_v;          /* value width per head */
  int32_t rank;         /* r: latent width (c_kv) */
  int32_t d_rope;       /* width of the shared RoPE key, even */
  int32_t dtype;        /* mla_dtype: storage dtype of q, weights, q_lat, cache */
  float softmax_scale;  /* <= 0: 1/sqrt(d_head + d_rope) */
  float rope_base;      /* <= 0: 10000 */
} mla_dims;

/* Supported shapes: (dtype, H, r, d_rope) in
 *   (F32, 8, 64, 16), (F32, 16, 64, 32), (BF16, 128, 512, 64),
 * with d_head in {32, 64, 128, 256} and d_v a multiple of 32, at most 1024. */

/* Fold W_UK into the query ([P1] section 3): for every b, h, j
 *   q_lat[b][h][j] = sum_d w_uk[h][d][j] * q_nope[b][h][d],   j < r,
 * accumulated in fp32 and rounded once to the storage dtype.  Columns
 * [r, r + d_rope) of q_lat are not touched. */
mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk,
                        void* q_lat, void* stream);

/* Rotate the query's RoPE part and append the new token ([P2] cache
 * management, [P5], [P1] section 2): for every b,
 *   q_lat[b][h][r + k]           = RoPE(q_rope[b][h], positions[b])[k]
 *   kv_cache[row_offsets[b] + positions[b]] = [c_kv_new[b] | RoPE(k_rope_new[b], positions[b])]
 * c_kv_new is copied bit for bit.  total_rows bounds the cache. */
mla_status mla_rope_append(const mla_dims* dims, const void* q_rope, const void* c_kv_new,
                           const void* k_rope_new, const int32_t* positions,
                           const int64_t* row_offsets, int64_t total_rows, void* q_lat,
                           void* kv_cache, void* stream);

/* mla_absorb_q followed by mla_rope_append, with the arguments of both
 * ([P1] section 3, [P2] cache management, [P5]): the two write disjoint
 * columns of q_lat, so with bf16 storage they run as one kernel launch (fp32
 * storage enqueues the two launches).  Results are those of the two calls. */
mla_status mla_absorb_rope(const mla_dims* dims, const void* q_nope, const void* w_uk,
                           const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                           const int32_t* positions, const int64_t* row_offsets, int64_t total_rows,
                           void* q_lat, void* kv_cache, void* stream);

/* Attention in the latent space ([P1] section 3, [P2] absorbing projections,
 * [P3] content score + position score): for every b, h and split s with rows
 * t in the split,
 *   score_t = softmax_scale * (q_lat[b][h][0:r] . c_kv_t + q_lat[b][h][r:] . k_rope_t)
 *   o_part(b, s, h, :) = sum_t softmax(score)_t * c_kv_t    (softmax within the split)
 *   lse_part[b][s][h]  = ln sum_t exp(score_t)
 * fp32 accumulation; bf16 storage computes the products in bf16 with fp32
 * sums.  max_seq_len must be >= every seq_lens[b]; rows beyond
 * num_splits * chunk are not read.  1 <= num_splits <= 4096. */
mla_status mla_decode_latent(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                             const int64_t* row_offsets, const int32_t* seq_lens,
                             int64_t total_rows, int32_t max_seq_len, int32_t num_splits,
                             void* o_part, float* lse_part, void* stream);

/* Merge the splits (softmax over the union of the splits' rows):
 *   m = max_s lse_part[b][s][h];  w_s = exp(lse_part[b][s][h] - m)
 *   o_lat[b][h] = sum_s w_s o_part(b, s, h, :) / sum_s w_s
 *   lse[b][h]   = m + ln sum_s w_s                (lse may be NULL)
 * Splits whose lse_part is -inf are skipped and their o_part rows are not
 * read (mla_decode_latent writes none for a split past its sequence's rows),
 * here and in mla_combine_up_v. */
mla_status mla_combine(const mla_dims* dims, const void* o_part, const float* lse_part,
                       int32_t num_splits, float* o_lat, float* lse, void* stream);

/* Apply W_UV after the weighted sum ([P2] absorbing projections):
 *   out[b][h][d] = sum_j w_uv[h][d][j] * o_lat[b][h][j]
 * fp32 accumulation; with bf16 weights, o_lat enters the product as the sum
 * of two bf16 terms (high and low part), which keeps it exact to ~2^-16. */
mla_status mla_up_v(const mla_dims* dims, const float* o_lat, const void* w_uv, float* out,
                    void* stream);

/* mla_combine followed by mla_up_v, without o_lat ([P2] absorbing
 * projections: the weighted sum of the latents, then W_UV):
 *   out[b][h][d] = sum_j w_uv[h][d][j] * o_lat[b][h][j]
 * with o_lat[b][h] the merge of the splits defined under mla_combine, and
 * lse[b][h] as there (lse may be NULL).  The merged row is formed in fp32 and,
 * with bf16 weights, enters the product as the sum of two bf16 terms (as in
 * mla_up_v).  A sequence whose splits are all empty gets out = 0 and
 * lse = -inf. */
mla_status mla_combine_up_v(const mla_dims* dims, const void* o_part, const float* lse_part,
                            int32_t num_splits, const void* w_uv, float* out, float* lse,
                            void* stream);

/* Paged cache ([P2] mentions vLLM-style page management for variable-length
 * batches; this is the plainest form of it).  The cache is total_pages pages
 * of page_rows rows (a power of two from 32 to 65536), row layout as above;
 * in-sequence row t of sequence b is row t % page_rows of page
 * block_table[b * bt_stride + t / page_rows] (int32 page ids, bt_stride >= 1
 * entries per sequence).  The paging changes where rows live, not what is
 * computed: each call below gives the same result as its packed counterpart
 * on the same rows.  Page ids and page indices are clamped into range on the
 * device (wrong numbers, never a stray access, for inconsistent tables). */
mla_status mla_decode_latent_paged(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                   const int32_t* block_table, int32_t bt_stride, int32_t page_rows,
                                   int64_t total_pages, const int32_t* seq_lens, int32_t max_seq_len,
                                   int32_t num_splits, void* o_part, float* lse_part, void* stream);

mla_status mla_rope_append_paged(const mla_dims* dims, const void* q_rope, const void* c_kv_new,
                                 const void* k_rope_new, const int32_t* positions,
                                 const int32_t* block_table, int32_t bt_stride, int32_t page_rows,
                                 int64_t total_pages, void* q_lat, void* kv_cache, void* stream);

mla_status mla_absorb_rope_paged(const mla_dims* dims, const void* q_nope, const void* w_uk,
                                 const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                                 const int32_t* positions, const int32_t* block_table,
                                 int32_t bt_stride, int32_t page_rows, int64_t total_pages,
                                 void* q_lat, void* kv_cache, void* stream);

/* FP8 latent cache ([P2] names FP8 quantisation of the latent cache among
 * what a production implementation adds, and fixes no format; the one below
 * is this library's).  Row layout, 640 bytes per cached token:
 *   bytes [0, 512)   c_kv as OCP E4M3FN codes of c_kv / s (sign, 4 exponent
 *                    bits with bias 7, 3 mantissa bits; 448 the largest value;
 *                    code 0x7f/0xff is NaN and is never written)
 *   bytes [512, 640) the rotated RoPE key, 64 bf16 values (as in the bf16 row)
 * with s = kv_scale[row] (fp32 [rows], 16-byte aligned base), a power of two:
 * the smallest 2^e, e an integer in [-116, 63], with max|c_kv| <= 448 * 2^e.
 * The cached latent is the dequantised value code * s (exact in bf16).  Only
 * the bf16 instance (heads 128, rank 512, d_rope 64); other dims give
 * MLA_ERR_UNSUPPORTED.
 *
 * mla_decode_latent_fp8: mla_decode_latent over the dequantised cache, same
 * q_lat, o_part and lse_part (so mla_combine / mla_combine_up_v apply
 * unchanged).  kv_cache: device [total_rows][640] bytes; rows as for
 * mla_decode_latent (row_offsets) or mla_decode_latent_paged (block table).
 *
 * mla_absorb_rope_fp8: mla_absorb_rope, except that the appended row is
 * written in the fp8 layout: c_kv_new (bf16) is quantised with its own row
 * exponent (nearest code, ties to even; magnitudes above 448 * s, possible
 * only at the exponent clamp, saturate to 448), the rotated key is written as
 * in the bf16 row, and kv_scale[row] = s.  Inputs must be finite. */
mla_status mla_decode_latent_fp8(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                 const float* kv_scale, const int64_t* row_offsets,
                                 const int32_t* seq_lens, int64_t total_rows, int32_t max_seq_len,
                                 int32_t num_splits, void* o_part, float* lse_part, void* stream);

mla_status mla_decode_latent_fp8_paged(const mla_dims* dims, const void* q_lat, const void* kv_cache,
                                       const float* kv_scale, const int32_t* block_table,
                                       int32_t bt_stride, int32_t page_rows, int64_t total_pages,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t num_splits, void* o_part, float* lse_part,
                                       void* stream);

mla_status mla_absorb_rope_fp8(const mla_dims* dims, const void* q_nope, const void* w_uk,
                               const void* q_rope, const void* c_kv_new, const void* k_rope_new,
                               const int32_t* positions, const int64_t* row_offsets,
                               int64_t total_rows, void* q_lat, void* kv_cache, float* kv_scale,
                               void* stream);

mla_status mla_absorb_rope_fp8_paged(const mla_dims* dims, const void* q_nope, const void* w_uk,
                                     const void* q_rope, const void* c_kv_new,
                                     const void* k_rope_new, const int32_t* positions,
                                     const int32_t* block_table, int32_t bt_stride,
                                     int32_t page_rows, int64_t total_pages, void* q_lat,
                                     void* kv_cache, float* kv_scale, void* stream);

/* Latent KV production from the hidden state, the step before the append
 * ([P2] module structure: W_DKV, then the RMSNorm norm_kv over the latent;
 * [P1] section 2, [P5]: W_KR gives the one RoPE key shared by the heads):
 *   x             = w_dkv h[b]                       w_dkv [r][d_model]
 *   c_kv_new[b]   = norm_w * x / sqrt(mean(x^2) + eps)   norm_w [r]
 *   k_rope_new[b] = w_kr h[b]                        w_kr [d_rope][d_model]
 * h [B][d_model]; weights are Linear weights (out, in); outputs are the
 * inputs of mla_rope_append / mla_absorb_rope (RoPE is applied there).  fp32
 * accumulation, summed over d_model in a fixed order, each output rounded
 * once.  bf16 storage only; d_model a multiple of 512; eps >= 0.  workspace:
 * device memory of mla_kv_down_workspace_size bytes (fp32 partial sums),
 * owned by the caller; calls that share one workspace must not overlap. */
mla_status mla_kv_down(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv,
                       const void* w_kr, const void* norm_w, float eps, void* workspace,
                       void* c_kv_new, void* k_rope_new, void* stream);

mla_status mla_kv_down_workspace_size(const mla_dims* dims, int32_t d_model, size_t* bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_kv_down with its fp32 partial sums in a fixed 4 MiB device array of
 * the library instead of a caller workspace.  Same arguments and results as
 * mla_kv_down without `workspace`; calls whose partial sums
 * (mla_kv_down_workspace_size) exceed 4 MiB return MLA_ERR_WORKSPACE.  It
 * allocates nothing: the array is part of the library's code object, one
 * copy per device, found on the first call on that device.  Every call on a
 * device shares that device's array, so calls that overlap on one device
 * (on different streams, or from several host threads) race; calls in one
 * stream's order do not.  The kernels write every partial sum before they
 * read any, so nothing carried over from an earlier call is used. */
mla_status mla_kv_down_noalloc(const mla_dims* dims, int32_t d_model, const void* h, const void* w_dkv,
                               const void* w_kr, const void* norm_w, float eps, void* c_kv_new,
                               void* k_rope_new, void* stream);

/* Folded projections ([P2] absorbing projections: W_O absorbs W_UV, a
 * product of fixed weights computed once, after which the attention-weighted
 * latents go straight to the output space, and the query side absorbs the
 * key up-projection the same way; [P5] "What we didn't build, and why": at
 * decode time the up-projection is folded into the query and output
 * matrices).  Readings: [P2]'s forward pass has an RMSNorm between W_DQ and
 * W_UQ, so the exact query fold is W_UK into W_UQ per head; [P2]'s single
 * (d_model, d_c) output matrix would sum the heads' latent outputs, so the
 * output fold is per head and the output sums over heads.
 *
 * Shapes: c_q [B][d_c_q] the normalised query latent (RMSNorm(W_DQ x)),
 * w_uq [H*d_head][d_c_q] (the Linear(d_c_q -> H*d_head) weight; rows
 * h*d_head.. are head h's), w_o [d_model][H*d_v] (the Linear(H*d_v -> d_model)
 * weight), w_qk [H][r][d_c_q], w_ov [d_model][H*r], y [B][d_model] float32.
 * bf16 storage only (other dtypes: MLA_ERR_UNSUPPORTED); d_c_q a multiple of
 * 256, d_model a multiple of 64, both at most 65536; rank a multiple of 64.
 *
 * mla_fold_query:  w_qk[h][j][i] = sum_d w_uk[h][d][j] * w_uq[h*d_head + d][i]
 * mla_fold_output: w_ov[m][h*r + j] = sum_d w_o[m][h*d_v + d] * w_uv[h][d][j]
 *   (fp32 accumulation, each folded weight rounded once to bf16; done once
 *   per set of weights, not per step)
 * mla_absorb_q_folded: q_lat[b][h][j] = sum_i w_qk[h][j][i] * c_q[b][i], j < r
 *   (fp32 accumulation, one rounding; replaces mla_absorb_q, columns
 *   [r, r + d_rope) untouched)
 * mla_out_folded: y[b][m] = sum_h sum_j w_ov[m][h*r + j] * o_lat[b][h][j]
 *   (replaces mla_up_v followed by W_O; o_lat from mla_combine enters the
 *   bf16 product as a high and a low bf16 part; fp32 accumulation summed over
 *   a fixed split of the k range, so repeated calls give the same bits).
 *   workspace: device memory of mla_out_folded_workspace_size bytes (fp32
 *   partial sums), owned by the caller; calls that share one workspace must
 *   not overlap. */
mla_status mla_fold_query(const mla_dims* dims, int32_t d_c_q, const void* w_uq, const void* w_uk,
                          void* w_qk, void* stream);

mla_status mla_fold_output(const mla_dims* dims, int32_t d_model, const void* w_o, const void* w_uv,
                           void* w_ov, void* stream);

mla_status mla_absorb_q_folded(const mla_dims* dims, int32_t d_c_q, const void* c_q, const void* w_qk,
                               void* q_lat, void* stream);

mla_status mla_out_folded(const mla_dims* dims, int32_t d_model, const float* o_lat, const void* w_ov,
                          void* workspace, float* y, void* stream);

mla_status mla_out_folded_workspace_size(const mla_dims* dims, int32_t d_model, size_t* bytes);

/* Bytes of o_part and lse_part for `num_splits` splits. */
mla_status mla_partials_size(const mla_dims* dims, int32_t num_splits, size_t* o_part_bytes,
                             size_t* lse_part_bytes);

/* Split count the library would choose: enough work-groups to cover the
 * device's compute units with splits of at least a few hundred rows.
 * Returns a value >= 1, or <= 0 on invalid arguments.  num_cus <= 0 queries
 * the current device. */
int32_t mla_plan_splits(const mla_dims* dims, int32_t max_seq_len, int64_t total_rows,
                        int32_t num_cus);

/* The same choice when the caller knows the lengths on the host (seq_lens:
 * host memory, dims->batch values, each >= 1): every chunk of whole 32-row
 * tiles is a candidate, with the exact number of non-empty splits it makes
 * (so that a batch of mixed lengths can fill the compute units in one
 * round).  Returns the split count S (>= 1; 0 on invalid arguments) and, in
 * *plan_max_seq_len, the max_seq_len to pass with it to the decode calls:
 * chunk * S, at least every length, for which ceil(max_seq_len / S) rounded
 * up to whole tiles is the planned chunk. */
int32_t mla_plan_splits_for_lengths(const mla_dims* dims, const int32_t* seq_lens, int32_t num_cus,
                                    int32_t* plan_max_seq_len);

/* MLA_OK if the dims are valid and have a kernel instantiation. */
mla_status mla_check_dims(const mla_dims* dims);

const char* mla_status_string(mla_status status);

/* Text of the last error on the calling host thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
