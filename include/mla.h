/*
 * mla.h — C ABI of libmla.so: Multi-head Latent Attention (MLA) decode on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed.  For every sequence b of a batch, one query token (the
 * newest one) attends over the sequence's cached tokens j = 0..T_b-1 with n_h
 * heads.  The cache keeps per token only the joint KV latent c^KV_j (width d_c)
 * and the shared, already rotated RoPE key k^R_j (width d_h^R)
 * [DeepSeek-V2 explainer (一文通透DeepSeek-V2) §2.2.1 and §2.2.2].  Keys and
 * values of head i are W^UK_i c^KV_j and W^UV_i c^KV_j, and the score is
 *     s_{i,j} = ([q^C_i; q^R_i] . [W^UK_i c^KV_j; k^R_j]) * softmax_scale,
 * softmax_scale = 1/sqrt(d_h + d_h^R)  [deepseek(2)——deepseek 關鍵技術, §1 MLA].
 * By associativity W^UK_i moves to the query side and W^UV_i past the softmax
 * [DeepSeek-V2 explainer §2.2.2; V3 interview notes (Deepseek系列从v3到R易背面经版),
 * section MLA]:
 *     q_lat_i = (W^UK_i)^T q^C_i                                   mla_absorb_q
 *     o_lat_i = sum_j softmax_j(s_{i,.}) c^KV_j, with
 *               s_{i,j} = (q_lat_i . c^KV_j + q^R_i . k^R_j) * scale  mla_decode (+ mla_merge_splits)
 *     o_i     = W^UV_i o_lat_i                                     mla_out_proj
 * and [o_1; ...; o_nh] is the input of the output projection W^O.
 *
 * Conventions for every entry point.
 *  - Tensor pointers are DEVICE pointers owned by the caller; dense, row-major,
 *    16-byte aligned.  The library allocates no device memory.  Pointers to
 *    mla_dims_t / mla_paged_cache_t / mla_partition_t structs are HOST pointers,
 *    read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    enqueue kernels and return; they do not synchronise.
 *  - Validation happens before anything is enqueued: on MLA_ERR_* nothing was
 *    launched and no device memory was touched.  A failed launch returns
 *    MLA_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Heads are stacked in order: head i of a [.., n_h*d_h] matrix owns rows
 *    i*d_h .. (i+1)*d_h-1 ([deepseek(2) 關鍵技術] §1 stacked notation).
 *  - LSE values are natural-log sum-exp of the scaled scores.
 *
 * Fast paths (MFMA kernels): n_h = 128, d_c = 512, d_h^R = 64, d_h = 128,
 * page_size = 64, bf16 queries/weights, bf16 or fp8 cache.  Other shapes and
 * dtypes (e.g. the fp32 tiny case) run on generic VALU kernels with fp32
 * arithmetic, limited to d_c <= 1024, d_h^R <= 256, d_h <= 1024.
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
  MLA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, inconsistent sizes */
  MLA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype combination, size limit) */
  MLA_ERR_ALIGNMENT = 3,     /* a tensor pointer is not 16-byte aligned */
  MLA_ERR_WORKSPACE = 4,     /* workspace missing or smaller than mla_decode_workspace_size */
  MLA_ERR_HIP = 5            /* the HIP runtime reported an error (launch or device query) */
} mla_status_t;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2           /* OCP E4M3FN (finite max 448); cache only */
} mla_dtype_t;

/* n_h, d_h, d_h^R, d_c. */
typedef struct {
  int32_t n_heads;
  int32_t d_head;
  int32_t d_rope;
  int32_t d_latent;
} mla_dims_t;

/*
 * Paged latent cache [DeepSeek-V2 explainer §2.2.2: only c^KV and k^R are cached;
 * §2.1.1 names paged KV memory].  Token t of sequence b sits in page
 * block_table[b * max_pages_per_seq + t / page_size], slot t % page_size, as
 * the row [c^KV_t (d_latent) | k^R_t (d_rope)].
 *   kv:      [num_pages, page_size, d_latent + d_rope] elements of `dtype`.
 *   scales:  fp8 only: [num_pages, page_size, ceil((d_latent + d_rope)/128)] fp32,
 *            one per token per 128-channel group; a stored value is code * scale
 *            (the 1x128 per-token-group FP8 format of the V3 notes, section
 *            F8量化策略).  NULL for other dtypes.
 *   block_table: [batch, max_pages_per_seq] int32; only the first
 *            ceil(seq_lens[b]/page_size) entries of a row are read, each must be
 *            in [0, num_pages).
 *   seq_lens: [batch] int32, 0 <= seq_lens[b] <= max_pages_per_seq * page_size.
 * Slots past a sequence's length are never read (they may hold NaN).
 * Input that breaks these rules does not make a kernel read or write outside
 * the arrays: lengths are clamped to [0, max_pages_per_seq * page_size], and a
 * page id outside [0, num_pages) reads as a page of zero rows (decode) or is
 * skipped (cache store).  mla_validate_cache_host checks the rules on the host.
 */
typedef struct {
  const void* kv;
  const float* scales;
  mla_dtype_t dtype;
  int32_t page_size;
  int32_t num_pages;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
  const int32_t* seq_lens;
} mla_paged_cache_t;

/*
 * How mla_decode divides the tokens of the batch into work items.
 *   split_tokens > 0: sequence b is cut into ceil(T_b / split_tokens) chunks
 *       [s*split_tokens, min((s+1)*split_tokens, T_b)); split_tokens must be a
 *       multiple of page_size.  Chunk s of sequence b uses workspace slot
 *       b * S + s, S = ceil(max_pages_per_seq * page_size / split_tokens).
 *   split_tokens == 0, num_parts == 0: one work item per sequence, no workspace.
 *   split_tokens == 0, num_parts > 0: a cost stream made of the pages of all
 *       non-empty sequences in sequence order, with 2 extra units between
 *       consecutive sequences (the fixed cost of a further sequence in one work
 *       item: its query loads and output write), C units in all, is divided
 *       into W = min(num_parts, total pages) contiguous parts; part w takes the
 *       pages among units [floor(w*C/W), floor((w+1)*C/W)).  A single
 *       sequence is thus cut into equal (+-1 page) parts.  Part w's share of
 *       sequence b uses workspace slot w + b.  num_parts < 0 means "chosen by
 *       the library to fill the current device once": its compute-unit count.
 * A sequence covered by a single work item receives its final o_lat / lse
 * directly from mla_decode; the others (and empty sequences) receive them from
 * mla_merge_splits.
 */
typedef struct {
  int32_t split_tokens;
  int32_t num_parts;
} mla_partition_t;

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(mla_status_t status);

/* Build description: target, kernels compiled in. */
const char* mla_build_info(void);

/*
 * q_lat[b, i, :] = (W^UK_i)^T q_nope[b, i, :]   ([DeepSeek-V2 explainer §2.2.2]
 * absorption of W^UK into the query side).
 *   q_nope: [batch, n_h, d_h] (q_dt);  w_uk: [n_h * d_h, d_c] (w_dt) = W^UK as on
 *   the pages;  q_lat: [batch, n_h, d_c] (out_dt).  fp32 accumulation.
 *   q_dt, w_dt, out_dt in {MLA_F32, MLA_BF16}.
 */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch,
                          const void* q_nope, mla_dtype_t q_dt,
                          const void* w_uk, mla_dtype_t w_dt,
                          void* q_lat, mla_dtype_t out_dt, void* stream);

/*
 * Workspace needed by mla_decode / mla_merge_splits for a partition: split
 * partials o_part [num_slots, n_h, d_c] at offset 0, stored in the o_dt of the
 * mla_decode call (bf16 or fp32; the area is sized for fp32), then fp32
 * lse_part [num_slots, n_h] at offset mla_lse_part_offset(...).  *bytes = 0 when
 * the partition never splits.  num_parts < 0 needs a current HIP device.
 */
mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch,
                                       int32_t max_pages_per_seq, int32_t page_size,
                                       const mla_partition_t* part,
                                       size_t* bytes, int32_t* num_slots);

/* Byte offset of lse_part inside the workspace for num_slots slots. */
size_t mla_lse_part_offset(const mla_dims_t* dims, int32_t num_slots);

/*
 * Attention of each sequence's query over its paged cache, absorbed form
 * (scores against c^KV and k^R, output in latent space; [deepseek(2) 關鍵技術] §1
 * with [DeepSeek-V2 explainer] §2.2.2 absorption).
 *   q_lat: [batch, n_h, d_c], q_pe: [batch, n_h, d_rope] (RoPE already applied),
 *       both q_dt (MLA_F32, or MLA_BF16).
 *   softmax_scale: multiplies every score, normally 1/sqrt(d_h + d_rope).
 *   o_lat: [batch, n_h, d_c] (o_dt in {MLA_F32, MLA_BF16}); lse: [batch, n_h]
 *       fp32 or NULL.  Written for sequences covered by one work item.
 *   workspace: see mla_decode_workspace_size; may be NULL when it is 0 bytes.
 * The cache must be f32 with f32 queries, or bf16 / fp8 with bf16 queries.
 */
mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch,
                        const void* q_lat, const void* q_pe, mla_dtype_t q_dt,
                        const mla_paged_cache_t* cache, float softmax_scale,
                        const mla_partition_t* part,
                        void* workspace, size_t workspace_bytes,
                        void* o_lat, mla_dtype_t o_dt, float* lse, void* stream);

/*
 * Log-sum-exp merge of split partials: for each sequence split over several
 * work items, lse = log sum_s exp(lse_s) and o_lat = sum_s exp(lse_s - lse) o_s.
 * Sequences with no tokens get o_lat = 0 and lse = -inf.  Sequences covered by
 * one work item are left untouched.  Arguments must match the mla_decode call
 * whose partials are merged (o_dt included: it is also the partials' dtype);
 * seq_lens is the cache's device array.
 */
mla_status_t mla_merge_splits(const mla_dims_t* dims, int32_t batch,
                              const int32_t* seq_lens, int32_t page_size,
                              int32_t max_pages_per_seq, const mla_partition_t* part,
                              const void* workspace, size_t workspace_bytes,
                              void* o_lat, mla_dtype_t o_dt, float* lse, void* stream);

/*
 * Several new query tokens per sequence, causal within them ([deepseek(2)
 * 關鍵技術] §1: each query attends to the tokens up to its own position; §2.2:
 * the multi-token prediction modules may be kept for decoding).  The q_len
 * new tokens of sequence b are the last q_len of its seq_lens[b] cached tokens:
 * new token t sits at position seq_lens[b] - q_len + t and attends to cache
 * tokens [0, seq_lens[b] - q_len + t + 1) (none if that is empty: o_lat = 0,
 * lse = -inf).
 *   q_lat: [batch, q_len, n_h, d_c], q_pe: [batch, q_len, n_h, d_rope] (q_dt);
 *   o_lat: [batch, q_len, n_h, d_c] (o_dt), lse: [batch, q_len, n_h] or NULL.
 * One call runs the whole attention, merge included: each (sequence, new
 * token) pair is a virtual sequence of mla_decode's batch * q_len, with the
 * partition `part` applied to the virtual batch; the kernels derive virtual
 * sequence b*q_len + t's length from seq_lens[b] and read sequence b's
 * block-table row in place (no extra launch).  Same cache and dtype rules as
 * mla_decode.
 *   workspace: mla_decode_multi_workspace_size(...) bytes (those of mla_decode
 *       over the virtual batch), 16-B aligned; may be NULL when that is 0.
 */
mla_status_t mla_decode_multi_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                             int32_t max_pages_per_seq, int32_t page_size,
                                             const mla_partition_t* part, size_t* bytes,
                                             int32_t* num_slots);
mla_status_t mla_decode_multi(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                              const void* q_lat, const void* q_pe, mla_dtype_t q_dt,
                              const mla_paged_cache_t* cache, float softmax_scale,
                              const mla_partition_t* part, void* workspace, size_t workspace_bytes,
                              void* o_lat, mla_dtype_t o_dt, float* lse, void* stream);

/*
 * mla_decode_multi followed by mla_out_proj over the batch * q_len rows, with
 * the split merge and the W^UV projection in one launch (mla_merge_out_proj).
 * o_lat / lse are written as by mla_decode_multi; o_heads: [batch, q_len,
 * n_h * d_h] (out_dt), equal to mla_out_proj's result up to the order of fp32
 * additions.  All arguments (those of the projection included) are validated
 * before anything is enqueued.
 */
mla_status_t mla_decode_multi_out_proj(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                       const void* q_lat, const void* q_pe, mla_dtype_t q_dt,
                                       const mla_paged_cache_t* cache, float softmax_scale,
                                       const mla_partition_t* part, void* workspace,
                                       size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse,
                                       const void* w_uv, mla_dtype_t w_dt, void* o_heads,
                                       mla_dtype_t out_dt, void* stream);

/*
 * o_heads[b, i*d_h + k] = sum_c W^UV[i*d_h + k, c] o_lat[b, i, c]  (W^UV applied
 * after attention, [DeepSeek-V2 explainer §2.2.2]).
 *   o_lat: [batch, n_h, d_c] (o_dt);  w_uv: [n_h * d_h, d_c] (w_dt);
 *   o_heads: [batch, n_h * d_h] (out_dt).  fp32 accumulation.
 */
mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t batch,
                          const void* o_lat, mla_dtype_t o_dt,
                          const void* w_uv, mla_dtype_t w_dt,
                          void* o_heads, mla_dtype_t out_dt, void* stream);

/*
 * mla_merge_splits followed by mla_out_proj, in one launch where it can:
 * the split partials of each sequence are merged (o_lat and lse written
 * exactly as mla_merge_splits writes them) and o_heads = W^UV_i o_lat_i is
 * computed from the merged rows without reading o_lat back.  Arguments are
 * those of the two calls; o_dt is both the partials' and o_lat's dtype.
 *   Single launch for d_h = 128, d_c = 512, o_dt = w_dt = out_dt = MLA_BF16
 *   (any n_h, any partition); otherwise the two calls run in sequence.
 *   o_heads then equals mla_out_proj's result up to the order of fp32
 *   additions (the contraction is split into four quarters).
 */
mla_status_t mla_merge_out_proj(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens,
                                int32_t page_size, int32_t max_pages_per_seq,
                                const mla_partition_t* part, const void* workspace,
                                size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse,
                                const void* w_uv, mla_dtype_t w_dt, void* o_heads,
                                mla_dtype_t out_dt, void* stream);

/*
 * Store one new token row per sequence into the paged cache, the step that
 * precedes decoding it: the cache keeps per token [c^KV | k^R] with k^R after
 * its rotation [DeepSeek-V2 explainer §2.2.2].
 *   rows: [batch, d_c + d_rope] (rows_dt MLA_F32 or MLA_BF16): the new rows.
 *   positions: [batch] int32 DEVICE array: token index t of each row; it is
 *       written to page block_table[b * max_pages_per_seq + t / page_size], slot
 *       t % page_size.  Sequences with t < 0, t >= max_pages_per_seq * page_size
 *       or a page id outside [0, num_pages) are skipped.
 *   rope_base: > 0 rotates the last d_rope columns first: pair (2k, 2k+1) by the
 *       angle t * rope_base^(-2k/d_rope) (evaluated in fp64); 0 stores the rows
 *       as given (k^R already rotated).
 *   cache: kv (and, for fp8, scales) are WRITTEN at those slots only (the const
 *       in mla_paged_cache_t is cast away); seq_lens is neither read nor updated.
 *       Rounding: bf16 to nearest even; fp8 per token and 128-column group:
 *       scale = amax / 448 in fp32 (1 for an all-zero group), code = E4M3 nearest
 *       even of x / scale (the 1x128 format of the V3 interview notes, section
 *       F8量化策略).
 * d_c and d_rope must be even, d_c + d_rope <= 1280.
 */
mla_status_t mla_cache_store(const mla_dims_t* dims, int32_t batch, const void* rows, mla_dtype_t rows_dt,
                             const int32_t* positions, float rope_base, const mla_paged_cache_t* cache,
                             void* stream);

/*
 * Project and store: rows = [W^DKV h ; W^KR h] per sequence (the cache-side
 * projections of [DeepSeek-V2 explainer §2.2.1 and §2.2.2]), fp32 accumulation,
 * written to `rows`; then mla_cache_store(rows, positions, rope_base, cache).
 *   h: [batch, d_model] (h_dt f32 or bf16) hidden state of the new token.
 *   w_dkv: [d_c, d_model], w_kr: [d_rope, d_model] (w_dt f32 or bf16).
 *   rows: fp32 device scratch of 8 * batch * (d_c + d_rope) floats; on return
 *       its first batch * (d_c + d_rope) floats hold the rows before rotation
 *       and rounding (the rest holds partial sums of the projection).
 */
mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t d_model, int32_t batch, const void* h,
                              mla_dtype_t h_dt, const void* w_dkv, const void* w_kr, mla_dtype_t w_dt, float* rows,
                              const int32_t* positions, float rope_base, const mla_paged_cache_t* cache,
                              void* stream);

/*
 * Query side of a decode step, before absorption [DeepSeek-V2 explainer §2.2.1
 * (query compression) and §2.2.2 (decoupled RoPE); deepseek(2) 關鍵技術 §1]:
 *   c^Q = W^DQ h,   q^C = W^UQ c^Q,   q^R = RoPE(W^QR c^Q) per head,
 * with fp32 accumulation; c^Q is rounded to w_dt between the two products.
 *   h: [batch, d_model] (h_dt f32 or bf16); w_dq: [d_qlatent, d_model];
 *   w_uq: [n_h * d_h, d_qlatent]; w_qr: [n_h * d_rope, d_qlatent] (w_dt).
 *   positions: [batch] int32 DEVICE array: the query token's position; head
 *       i's q^R pair (2k, 2k+1) is rotated by position * rope_base^(-2k/d_rope)
 *       (angle in fp64); rope_base = 0 leaves q^R unrotated.
 *   q_nope: [batch, n_h, d_h], q_pe: [batch, n_h, d_rope] (out_dt f32 or bf16),
 *       the inputs of mla_absorb_q and mla_decode.
 *   scratch: device memory of mla_query_prep_scratch_size(...) bytes, 16-B
 *       aligned (k-slice partial sums and c^Q).
 * d_qlatent = 0: the query is not compressed (DeepSeek-V2-Lite, [DeepSeek-V2
 *   explainer] V2-Lite paragraph): q^C = W^UQ h, q^R = RoPE(W^QR h) in one
 *   product; w_dq is unused (may be NULL), w_uq is [n_h * d_h, d_model] and
 *   w_qr [n_h * d_rope, d_model].
 * d_h and d_rope must be even.
 */
size_t mla_query_prep_scratch_size(const mla_dims_t* dims, int32_t d_qlatent, int32_t batch);
mla_status_t mla_query_prep(const mla_dims_t* dims, int32_t d_model, int32_t d_qlatent, int32_t batch,
                            const void* h, mla_dtype_t h_dt, const void* w_dq, const void* w_uq, const void* w_qr,
                            mla_dtype_t w_dt, const int32_t* positions, float rope_base, void* q_nope, void* q_pe,
                            mla_dtype_t out_dt, void* scratch, size_t scratch_bytes, void* stream);

/*
 * RoPE frequencies for the cache and query writers, with YaRN context
 * extension [DeepSeek-V2 explainer §3.1.3: YaRN on the decoupled key k^R, scale
 * s = 40, alpha = 1, beta = 32, from a 4K to a 160K context].  Pair k of the
 * d_rope-wide RoPE slice turns at theta_k = base^(-2k/d_rope) radians per
 * position; with yarn_scale s > 1, with r_k = yarn_orig_ctx * theta_k / (2 pi)
 * its turns over the original context and gamma_k = clip((r_k - yarn_alpha) /
 * (yarn_beta - yarn_alpha), 0, 1), it turns at (1 - gamma_k) theta_k / s +
 * gamma_k theta_k instead (the YaRN ramp: slow pairs interpolated, fast pairs
 * kept).  Both the cached k^R (mla_cache_*_rope) and the query's q^R
 * (mla_query_prep_rope) must use the same parameters.  The matching softmax
 * scale is mla_yarn_attention_factor(s) / sqrt(d_h + d_rope).
 *   base >= 0 (0: no rotation); yarn_scale >= 1 (1: plain RoPE, the other
 *   fields ignored); when yarn_scale > 1: 0 <= yarn_alpha < yarn_beta,
 *   yarn_orig_ctx >= 1.  Anything else: MLA_ERR_INVALID_ARG.
 * mla_cache_store / mla_cache_append / mla_query_prep are these calls with
 * {rope_base, 1, 0, 0, 0}.
 */
typedef struct {
  float base;
  float yarn_scale;
  float yarn_alpha;
  float yarn_beta;
  int32_t yarn_orig_ctx;
} mla_rope_t;

mla_status_t mla_cache_store_rope(const mla_dims_t* dims, int32_t batch, const void* rows, mla_dtype_t rows_dt,
                                  const int32_t* positions, const mla_rope_t* rope, const mla_paged_cache_t* cache,
                                  void* stream);
mla_status_t mla_cache_append_rope(const mla_dims_t* dims, int32_t d_model, int32_t batch, const void* h,
                                   mla_dtype_t h_dt, const void* w_dkv, const void* w_kr, mla_dtype_t w_dt,
                                   float* rows, const int32_t* positions, const mla_rope_t* rope,
                                   const mla_paged_cache_t* cache, void* stream);
mla_status_t mla_query_prep_rope(const mla_dims_t* dims, int32_t d_model, int32_t d_qlatent, int32_t batch,
                                 const void* h, mla_dtype_t h_dt, const void* w_dq, const void* w_uq,
                                 const void* w_qr, mla_dtype_t w_dt, const int32_t* positions,
                                 const mla_rope_t* rope, void* q_nope, void* q_pe, mla_dtype_t out_dt, void* scratch,
                                 size_t scratch_bytes, void* stream);

/* YaRN's attention factor in MLA [DeepSeek-V2 explainer §3.1.3: the length
 * factor sqrt(t) = 0.0707 ln s + 1 on each side of the dot product]: returns
 * t = (0.0707 ln s + 1)^2, the multiplier of the softmax scale (1 for s <= 1). */
float mla_yarn_attention_factor(float yarn_scale);

/*
 * mla_decode followed by mla_merge_splits without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The split partials
 * live in a library-owned device array of MLA_NOALLOC_SCRATCH_BYTES per GPU
 * (held until the process ends), packed at the output dtype's size; a
 * partition whose partials need more returns MLA_ERR_WORKSPACE before
 * anything is enqueued (see mla_decode_workspace_size for the fp32-sized
 * public layout; here bf16 output needs half of its o_part area).  The call
 * allocates nothing.  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (other streams or host threads) race and must be
 * serialised by the caller.  Arguments and results are those of mla_decode +
 * mla_merge_splits: o_lat / lse hold every sequence's final output.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (48u << 20)
mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch,
                                const void* q_lat, const void* q_pe, mla_dtype_t q_dt,
                                const mla_paged_cache_t* cache, float softmax_scale,
                                const mla_partition_t* part,
                                void* o_lat, mla_dtype_t o_dt, float* lse, void* stream);

/*
 * Prefill: attention of a batch of new prompt tokens over their sequences'
 * paged caches, in the non-absorbed form [DeepSeek-V2 explainer §2.2.1: per
 * head, k^C_{j,i} = W^UK_i c^KV_j and v_{j,i} = W^UV_i c^KV_j; deepseek(2) 關鍵技術
 * §1: s = [q^C_i; q^R_i] . [k^C_{j,i}; k^R_j] * softmax_scale, softmax over the
 * positions up to the query's own, o_i = sum_j p_j v_{j,i}].  Keys and values
 * are up-projected once per cached token (into the workspace), so the
 * attention runs at d_h + d_h^R = 192 score dims and d_h = 128 output dims
 * instead of the absorbed 576 / 512: the cheaper form once a sequence has more
 * than a few hundred new tokens.  The new tokens of sequence b are rows
 * [q_offsets[b], q_offsets[b+1]) of q_nope / q_pe / o_heads, and they are the
 * last q_len_b = q_offsets[b+1] - q_offsets[b] of its seq_lens[b] cached tokens
 * (already written to the cache, e.g. by mla_cache_append): new token t sits
 * at position seq_lens[b] - q_len_b + t and attends to cache positions
 * 0 .. seq_lens[b] - q_len_b + t (none when that is negative: zeros, lse -inf).
 * Earlier cached tokens (a prefix from an earlier chunk) are attended too.
 *   q_offsets: [batch + 1] int32, device; non-decreasing, q_offsets[batch] <= total_q.
 *   total_q: rows of q_nope / q_pe / o_heads / lse (host value).
 *   max_q_len: host bound on every q_len_b (tokens past it are not computed).
 *   q_nope: [total_q, n_h, d_h], q_pe: [total_q, n_h, d_rope] (RoPE applied), q_dt.
 *   total_kv: host bound on the sum of the (clamped) seq_lens; the gathered and
 *       up-projected rows are sized by it (if the sum exceeds it, the later
 *       sequences' trailing positions are not attended).
 *   w_uk, w_uv: [n_h * d_h, d_c] (w_dt), W^UK and W^UV as on the pages.
 *   o_heads: [total_q, n_h, d_h] (out_dt) = [o_1; ...; o_nh] per token, the
 *       input of W^O; lse: [total_q, n_h] fp32 (natural log) or NULL.
 *   workspace: mla_prefill_workspace_size(...) bytes, 256-B aligned: the
 *       gathered rows (bf16, an fp8 cache dequantised), then the up-projected
 *       keys and values ([2 n_h, rows, d_h] bf16, about 64 KB per cached token
 *       at 128 heads).
 * Supported: d_h = 128, d_c = 512, d_rope = 64, page_size = 64, any n_h;
 * q_dt = w_dt = out_dt = MLA_BF16; bf16 or fp8 cache (others:
 * MLA_ERR_UNSUPPORTED).  total_kv < 2^24.  fp32 accumulation; keys, values
 * and probabilities are rounded to bf16 before their products.
 */
mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t total_kv,
                                        size_t* bytes);
mla_status_t mla_prefill(const mla_dims_t* dims, int32_t batch, const int32_t* q_offsets,
                         int32_t total_q, int32_t max_q_len,
                         const void* q_nope, const void* q_pe, mla_dtype_t q_dt,
                         const mla_paged_cache_t* cache, int64_t total_kv,
                         const void* w_uk, const void* w_uv, mla_dtype_t w_dt,
                         float softmax_scale, void* workspace, size_t workspace_bytes,
                         void* o_heads, mla_dtype_t out_dt, float* lse, void* stream);

/*
 * Host check (no device access) of a paged cache's metadata, on host copies of
 * its block table and lengths [DeepSeek-V2 explainer §2.1.1 names the paged KV
 * memory; the layout is that of mla_paged_cache_t above]:
 *   - 0 <= seq_lens_host[b] <= max_pages_per_seq * page_size, and
 *   - every block-table entry the kernels read for sequence b (the first
 *     ceil(seq_lens_host[b] / page_size) of its row) is in [0, num_pages).
 *   block_table_host: [batch, max_pages_per_seq] int32; seq_lens_host: [batch].
 * Returns MLA_OK, or MLA_ERR_INVALID_ARG with *bad_seq (if not NULL) set to the
 * first sequence that breaks a rule (-1 when the arguments themselves are
 * invalid: null pointers, batch < 0, non-positive sizes).
 * The device kernels never fault on such input (a length is clamped to its
 * row, a page id outside the cache reads as a page of zero rows) but their
 * results for it are meaningless; call this where lengths or tables come from
 * untrusted code.
 */
mla_status_t mla_validate_cache_host(const int32_t* block_table_host, const int32_t* seq_lens_host,
                                     int32_t batch, int32_t max_pages_per_seq, int32_t page_size,
                                     int32_t num_pages, int32_t* bad_seq);

/*
 * Host helper (no device access): for host copies of seq_lens, the workspace
 * slots that hold sequence b's partials: slots part_first[b] .. part_first[b] +
 * part_count[b] - 1.  part_count[b] == 1 means mla_decode writes the final
 * output directly; 0 means the sequence is empty.  num_parts must be >= 0.
 */
mla_status_t mla_partition_host(const int32_t* seq_lens_host, int32_t batch,
                                int32_t page_size, int32_t max_pages_per_seq,
                                const mla_partition_t* part,
                                int32_t* part_first, int32_t* part_count);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
