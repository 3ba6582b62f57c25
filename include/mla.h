/*
 * mla.h -- C ABI of libmla: absorbed Multi-head Latent Attention decode on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (what every entry point below is a step of):
 *   Each query head's 128-wide no-rope part is moved into latent space through
 *   W_UK once per query token ("absorbed" into the query), then all heads score
 *   the same cached rows -- one 512-wide latent plus a 64-wide decoupled rope
 *   key per token, shared by every head -- softmax the scores, average the
 *   rows' 512 latent columns, and project that latent output back per head
 *   through W_UV.  Sources: "MLA, dim by dim" (section "MLA Decode": decode
 *   score order (q W_UK^T) C^T and value order (p C) W_UV, and the fused
 *   decode kernel it sketches); "Why MLA and MTP Fight Each Other" (sections
 *   3.1, 3.2, 4 and Appendix A); "The MLA decode speedup hiding in your model
 *   card" ("The identity", "The absorbed form": same inputs and outputs as the
 *   naive form, different order of multiplication).
 *
 * Fixed widths: d_nope = 128, d_rope = 64, d_c = 512, d_v = 128; a cached row
 * is 576 elements [latent 0..511 | rope key 512..575]; a query row is 192
 * elements [nope 0..127 | rope 128..191]; a latent query row is 576 elements
 * [q_abs 0..511 | q_rope 512..575].  The rope rotation is applied by the
 * caller before these calls (queries and cached rope keys arrive rotated).
 *
 * Conventions for every call:
 *   - Every pointer is a DEVICE pointer unless marked "host".  The caller owns
 *     all memory: the library never allocates or frees memory and keeps no
 *     host state between calls.
 *   - Tensors are dense and row-major with the last dimension contiguous.
 *     bf16 is the 16-bit brain float; fp8 is OCP FP8 E4M3 ("e4m3fn").
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it and returns without synchronising.
 *   - Argument errors that the host can see are reported BEFORE any HIP call,
 *     and then nothing has been enqueued: MLA_ERR_ARG (null pointer, size <= 0,
 *     bad dtype, s_q > max_seqlen, ...), MLA_ERR_UNSUPPORTED (a width other than
 *     the fixed ones above, paged block size other than 64), MLA_ERR_WORKSPACE
 *     (workspace smaller than the *_workspace_bytes() figure).  A failed kernel
 *     launch returns MLA_ERR_HIP.
 *   - Device-resident values (sequence lengths, block-table entries) are not
 *     read by the host.  Preconditions on them: s_q <= seqlens[b] <= max_seqlen,
 *     seqlens[b] <= T_stride (contiguous) or <= max_blocks * 64 (paged), and
 *     every block id in the first ceil(seqlens[b] / 64) entries of a row of the
 *     block table is a valid pool block.  Entries past that are never read.
 *     mla_validate_kv checks them (a debugging aid that synchronises).
 *   - Calls are reentrant; results for a fixed argument set are bitwise
 *     reproducible run to run (no floating-point atomics).
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
  MLA_ERR_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_WORKSPACE = 3,
  MLA_ERR_HIP = 4
} mla_status;

typedef enum {
  MLA_BF16 = 0,
  MLA_FP8_E4M3 = 1,
  MLA_FP32 = 2
} mla_dtype;

/* Description of the latent cache (a HOST struct holding device pointers).
 *
 * contiguous (block_table == NULL): rows is [B, T_stride, 576]; sequence b's
 *   cached row t is rows[b, t, :].
 * paged (block_table != NULL): rows is a pool [n_blocks, block_size, 576];
 *   sequence b's row t is rows[block_table[b * max_blocks + t / 64], t % 64, :].
 *   block_size must be 64.  The block layout is this library's own reading: the
 *   pages describe only a contiguous cache.
 * dtype MLA_BF16: rows hold bf16.  dtype MLA_FP8_E4M3: rows hold e4m3 codes and
 *   row_scale holds one fp32 scale per row, indexed like the rows
 *   ([B, T_stride] or [n_blocks, 64]); the cached value is code * scale (the
 *   pages' FP8 latent cache of "Decode attention intensity...", read and
 *   dequantised in registers).  row_scale must be NULL for bf16.
 * seqlens: int32 [B], the number of valid rows of each sequence, including the
 *   s_q rows of the current query tokens.
 * max_seqlen: a host-side upper bound on every seqlens[b]; it sizes the split
 *   plan and the workspace.
 */
typedef struct {
  const void* rows;
  const float* row_scale;
  const int32_t* block_table;
  const int32_t* seqlens;
  int32_t dtype;        /* mla_dtype: MLA_BF16 or MLA_FP8_E4M3 */
  int32_t T_stride;     /* contiguous: rows per sequence in `rows`; paged: ignored */
  int32_t block_size;   /* paged: must be 64; contiguous: ignored */
  int32_t max_blocks;   /* paged: columns of block_table; contiguous: ignored */
  int32_t max_seqlen;   /* host bound on seqlens[b] */
} mla_kv_desc;

/* Step 1 -- absorb W_UK into the query ("MLA, dim by dim", "MLA Decode",
 * decode score order; "Why MLA and MTP Fight Each Other", section 3.1).
 *   q_lat[n, h, c]       = sum_{k<128} q[n, h, k] * w_uk[h, k, c]    (c < 512)
 *   q_lat[n, h, 512 + r] = q[n, h, 128 + r]                          (r < 64)
 * q      bf16 [N, H, 192]   (N = B * s_q query tokens)
 * w_uk   bf16 [H, 128, 512] (head, d_nope, d_c)
 * q_lat  bf16 [N, H, 576]   output; fp32 accumulation, rounded to nearest even.
 * d_nope, d_rope, d_c must be 128, 64, 512 (else MLA_ERR_UNSUPPORTED). */
mla_status mla_absorb_q(const void* q, const void* w_uk, void* q_lat,
                        int32_t N, int32_t H, int32_t d_nope, int32_t d_rope,
                        int32_t d_c, void* stream);

/* Bytes of device workspace mla_decode_attn needs for these sizes, with the
 * library's own split count.  Returns 0 for invalid sizes. */
size_t mla_decode_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen);

/* The same for mla_decode_attn_ex and the split-level calls below.
 * num_splits: the number of parts a sequence of max_seqlen rows is scanned
 * in; 0 lets the library choose (then equal to mla_decode_workspace_bytes), a
 * positive value forces it (any count gives the same result up to rounding;
 * it is capped at ceil(max_seqlen / 64)).  Returns 0 for invalid sizes. */
size_t mla_decode_workspace_bytes_ex(int32_t B, int32_t s_q, int32_t H,
                                     int32_t max_seqlen, int32_t num_splits);

/* The split count S the scan will use for these sizes (host integers only). */
int32_t mla_decode_num_splits(int32_t B, int32_t s_q, int32_t H,
                              int32_t max_seqlen, int32_t num_splits);

/* Steps 2 and 3 -- attention of the latent queries against the shared latent
 * cache ("MLA, dim by dim", "MLA Decode": stream the cache blocks, online
 * softmax, accumulate p C; "Why MLA and MTP Fight Each Other", section 4.2:
 * each latent tile read once serves both the scores and the weighted sum).
 * For query token j of sequence b and head h, with T = seqlens[b]:
 *   visible rows  V = { t : t <= T - s_q + j } if causal, else { t < T }
 *   s_t           = softmax_scale * <q_lat[b, j, h, :], row_t[0:576]>
 *   o_lat[b,j,h,:] = sum_{t in V} softmax(s)_t * row_t[0:512]
 *   lse[b,j,h]     = ln sum_{t in V} exp(s_t)
 * The causal rule (the s_q newest rows are the query tokens themselves, each
 * seeing itself and earlier rows) is this library's reading of speculative
 * verification of s_q tokens ("Why MLA and MTP Fight Each Other", section 8).
 * The cache is scanned in parallel parts (split-T flash decode): the 64-row
 * tiles of all sequences, in sequence order, are cut into B * S equal ranges
 * (S = mla_decode_num_splits(...)), so work is balanced over ragged lengths
 * and a sequence of max_seqlen rows gets S parts.  Each part (the piece of
 * one sequence inside one range) produces a normalised partial output and its
 * log-sum-exp in the workspace; a second kernel merges each sequence's parts
 * with log-sum-exp weights.
 * q_lat        bf16 [B, s_q, H, 576]
 * kv           host pointer to the cache description (read during the call only)
 * o_lat        [B, s_q, H, 512], dtype o_lat_dtype (MLA_FP32 or MLA_BF16)
 * lse          fp32 [B, s_q, H], or NULL when not wanted
 * workspace    device scratch of ws_bytes >= mla_decode_workspace_bytes(...);
 *              contents on entry are ignored; it may be reused after the
 *              stream has finished the call. */
mla_status mla_decode_attn(const void* q_lat, const mla_kv_desc* kv,
                           int32_t B, int32_t s_q, int32_t H,
                           float softmax_scale, int32_t causal,
                           void* o_lat, int32_t o_lat_dtype, float* lse,
                           void* workspace, size_t ws_bytes, void* stream);

/* mla_decode_attn with the split count forced (num_splits as for
 * mla_decode_workspace_bytes_ex; ws_bytes >= that figure).  num_splits = 0
 * is mla_decode_attn. */
mla_status mla_decode_attn_ex(const void* q_lat, const mla_kv_desc* kv,
                              int32_t B, int32_t s_q, int32_t H,
                              float softmax_scale, int32_t causal,
                              void* o_lat, int32_t o_lat_dtype, float* lse,
                              void* workspace, size_t ws_bytes, int32_t num_splits,
                              void* stream);

/* Steps 2 and 3 without any allocation: mla_decode_attn with its workspace
 * in a fixed device array inside the library instead of a caller buffer.
 * For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *   Arguments and results as mla_decode_attn (library split count).
 *   The array holds mla_decode_noalloc_max_bytes() = 64 MiB; argument sets
 *   whose mla_decode_workspace_bytes(...) exceeds it get MLA_ERR_WORKSPACE
 *   before anything is enqueued (for example B = 64, H = 128, 4096 rows with
 *   an fp32 o_lat needs 84 MB; with a bf16 o_lat, 42 MB).
 *   Each GPU the library runs on holds its own copy of the array until the
 *   process ends; its address is looked up once per device on the first call
 *   there (no allocation: hipGetSymbolAddress).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, other threads) race and must be serialised by the
 *   caller.  The kernels write every scratch byte before they read it, so
 *   what an earlier call left there does not matter. */
size_t mla_decode_noalloc_max_bytes(void);
mla_status mla_decode_attn_noalloc(const void* q_lat, const mla_kv_desc* kv,
                                   int32_t B, int32_t s_q, int32_t H,
                                   float softmax_scale, int32_t causal,
                                   void* o_lat, int32_t o_lat_dtype, float* lse,
                                   void* stream);

/* Steps 2 and 3 as two separate calls, for callers that keep or move the
 * split partials themselves (for example to merge ranges of one sequence that
 * were scanned on different devices).  mla_decode_attn is exactly
 * mla_decode_partial followed by mla_decode_combine on the same workspace.
 *
 * mla_decode_partial: same arguments as mla_decode_attn_ex minus the outputs,
 *   plus part_dtype, the element type of the partial outputs: MLA_FP32, or
 *   MLA_BF16 (each value rounded to nearest even: half the partial traffic,
 *   about 2^-9 relative error on each partial; mla_decode_attn uses the
 *   precision of its o_lat_dtype).  Any other value gives MLA_ERR_ARG.
 *   ws_bytes >= mla_decode_workspace_bytes_ex(B, s_q, H, kv->max_seqlen,
 *   num_splits).
 *   Scans every part and writes into the workspace, with
 *   S = mla_decode_num_splits(B, s_q, H, kv->max_seqlen, num_splits),
 *   R = s_q * H and M = B * (S + 1) partial slots (aligned = rounded up to a
 *   multiple of 256 bytes):
 *     part_o    part_dtype [M, R, 512] at offset 0: slot m holds the normalised
 *               partial latent output of one part for each of the R rows;
 *     part_lse  fp32 [M, R] at aligned(M * R * 512 * 4): the base-2
 *               log-sum-exp of the part's scaled scores (-inf when it holds
 *               no visible row);
 *     seg_first int32 [B], then seg_count int32 [B], at aligned(...) after
 *               part_lse: sequence b's parts are the slots seg_first[b] ..
 *               seg_first[b] + seg_count[b] - 1, in row order;
 *     part_mrun fp32 [M, R] at aligned(...) after the seg tables: each
 *               part's maximum scaled score per row (log2 domain), written
 *               by mla_decode_partial_fp8 for its accuracy check (unused by
 *               the other calls).
 *   The offsets do not depend on part_dtype (bf16 partials use the first half
 *   of the part_o region).  Slots outside every sequence's run are left
 *   unwritten.
 * mla_decode_combine: merges the parts of every query row with weights
 *   2^(lse_s - max_s lse_s) and writes o_lat and (if not NULL) the natural-log
 *   lse, exactly as mla_decode_attn does.  B, s_q, H, max_seqlen, num_splits
 *   and part_dtype must be those given to mla_decode_partial. */
mla_status mla_decode_partial(const void* q_lat, const mla_kv_desc* kv,
                              int32_t B, int32_t s_q, int32_t H,
                              float softmax_scale, int32_t causal,
                              void* workspace, size_t ws_bytes, int32_t num_splits,
                              int32_t part_dtype, void* stream);
mla_status mla_decode_combine(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                              int32_t num_splits, int32_t part_dtype,
                              const void* workspace, size_t ws_bytes,
                              void* o_lat, int32_t o_lat_dtype, float* lse, void* stream);

/* Step 4 -- project the latent output back per head ("MLA, dim by dim",
 * "MLA Decode", decode value order; "Why MLA and MTP Fight Each Other",
 * section 3.2).
 *   out[n, h, v] = sum_{c<512} o_lat[n, h, c] * w_uv[h, c, v]      (v < 128)
 * o_lat  [N, H, 512] of dtype o_lat_dtype (MLA_FP32 or MLA_BF16).  An fp32
 *        o_lat is split into two bf16 terms (high + low part) so that it keeps
 *        about 16 mantissa bits through the bf16 matrix cores.
 * w_uv   bf16 [H, 512, 128] (head, d_c, d_v)
 * out    bf16 [N, H, 128]; fp32 accumulation, rounded to nearest even.
 * d_c, d_v must be 512, 128 (else MLA_ERR_UNSUPPORTED). */
mla_status mla_absorb_out(const void* o_lat, int32_t o_lat_dtype, const void* w_uv,
                          void* out, int32_t N, int32_t H, int32_t d_c,
                          int32_t d_v, void* stream);

/* Steps 3 + 4 fused -- merge the split partials and project back per head in
 * one pass, so the latent output is not written to and re-read from memory
 * (the value order of "MLA, dim by dim", "MLA Decode": the latent output of
 * each head goes straight through W_UV[h]).  The result is bitwise equal to
 * mla_decode_combine followed by mla_absorb_out with the same o_lat_dtype.
 *   B, s_q, H, max_seqlen, num_splits, part_dtype, workspace, ws_bytes: as
 *          given to mla_decode_partial (the workspace holds its partials).
 *   w_uv   bf16 [H, 512, 128]
 *   out    bf16 [B * s_q, H, 128]
 *   o_lat  NULL, or [B, s_q, H, 512] of o_lat_dtype: also written when given.
 *   o_lat_dtype  MLA_FP32 (the latent output enters the projection as high +
 *          low bf16 terms) or MLA_BF16 (rounded to bf16 first), whether or not
 *          o_lat is written.
 *   lse    NULL or fp32 [B, s_q, H], natural log. */
mla_status mla_decode_combine_out(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                                  int32_t num_splits, int32_t part_dtype,
                                  const void* workspace, size_t ws_bytes,
                                  const void* w_uv, void* out, void* o_lat, int32_t o_lat_dtype,
                                  float* lse, void* stream);

/* Step 2 with FP8 arithmetic ("Decode attention intensity is fixed at the
 * query-to-KV head ratio...": FP8 halves the cache bytes; with FP8 matrix
 * arithmetic the path is priced against the FP8 ridge).  Same arguments,
 * workspace and partials as mla_decode_partial (merge them with
 * mla_decode_combine or mla_decode_combine_out); kv->dtype must be
 * MLA_FP8_E4M3 (else MLA_ERR_UNSUPPORTED).  The cached codes enter the matrix
 * products as they are; each latent query row is quantised to E4M3 with its
 * own scale amax/448, and the softmax weights times the row scales to E4M3
 * (against a power-of-two normaliser).  That is accurate to the FP8 bar
 * (6e-2 absolute on unit-scale outputs) only where many comparable weights
 * average out the E4M3 rounding.  The scan records each part's maximum
 * score per row; the call then runs the bf16-arithmetic scan as a fix-up
 * that recomputes (and overwrites the partials of) every (sequence, row
 * group) holding a query row whose largest probability exceeds 1/32 of the
 * row's total (few visible rows, or a peaked softmax).  Where no row does,
 * that second scan exits after its work plan. */
mla_status mla_decode_partial_fp8(const void* q_lat, const mla_kv_desc* kv, int32_t B,
                                  int32_t s_q, int32_t H, float softmax_scale, int32_t causal,
                                  void* workspace, size_t ws_bytes, int32_t num_splits,
                                  int32_t part_dtype, void* stream);

/* Sparse top-k decode ("Why MLA and MTP Fight Each Other", section 6: a
 * selector keeps the top-k cached latents and attention runs over those only,
 * gathered by index; the cost follows k instead of the context length).
 * The selection of sequence b is sel_idx[b, 0 .. sel_count[b] - 1]:
 * positions in its cache (0 <= pos < seqlens[b]), in any order; a repeated
 * position counts once per entry; a position outside that range gathers a
 * zero row (nothing is read for it).  The selection is the visible set of all
 * s_q query tokens of the sequence (no causal mask); a sequence with no
 * selected row gets zeros.  For query token j, head h:
 *   o_lat[b,j,h,:] = sum_{i < sel_count[b]} softmax_i(scale * <q_lat[b,j,h,:],
 *                    row_{sel_idx[b,i]}>) * row_{sel_idx[b,i]}[0:512]
 * Steps: for a contiguous bf16 cache (T_stride * 1152 <= 2^30) the split-T
 * scan loads the selected rows itself; otherwise (paged or e4m3 caches) they
 * are first gathered into a compact cache inside the workspace, which the
 * scan then reads.
 *   kv         the full cache (contiguous or paged, bf16 or e4m3)
 *   sel_idx    int32 [B, k_max]; sel_count int32 [B], each <= k_max
 *   k_max      row stride of sel_idx and the largest selection (>= s_q)
 *   workspace  ws_bytes >= mla_sparse_workspace_bytes(B, s_q, H, k_max,
 *              num_splits, kv->dtype).  Its first part has the layout of
 *              mla_decode_partial's workspace with max_seqlen = k_max, so
 *              mla_decode_combine and mla_decode_combine_out (given k_max as
 *              max_seqlen and the same part_dtype) merge the partials of
 *              mla_sparse_decode_partial.
 *   part_dtype MLA_FP32 or MLA_BF16 partials, as for mla_decode_partial.
 * mla_sparse_decode_attn = mla_sparse_decode_partial + mla_decode_combine,
 * with partials in the precision of o_lat_dtype. */
size_t mla_sparse_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t k_max,
                                  int32_t num_splits, int32_t cache_dtype);
mla_status mla_sparse_decode_partial(const void* q_lat, const mla_kv_desc* kv,
                                     const int32_t* sel_idx, const int32_t* sel_count,
                                     int32_t k_max, int32_t B, int32_t s_q, int32_t H,
                                     float softmax_scale, void* workspace, size_t ws_bytes,
                                     int32_t num_splits, int32_t part_dtype, void* stream);
mla_status mla_sparse_decode_attn(const void* q_lat, const mla_kv_desc* kv,
                                  const int32_t* sel_idx, const int32_t* sel_count,
                                  int32_t k_max, int32_t B, int32_t s_q, int32_t H,
                                  float softmax_scale, void* o_lat, int32_t o_lat_dtype,
                                  float* lse, void* workspace, size_t ws_bytes,
                                  int32_t num_splits, void* stream);

/* Ablation only -- the naive up-project-then-attend form ("The MLA decode
 * speedup hiding in your model card", "The naive form, written out"; "Why MLA
 * and MTP Fight Each Other", section 5.1, expand bracketing).  Every visible
 * cached row is expanded per head into a 192-wide key [W_UK[h] row[0:512] |
 * row[512:576]] and a 128-wide value row[0:512]^T W_UV[h], then ordinary
 * softmax attention with the 192-wide query q [B, s_q, H, 192] gives
 * out [B, s_q, H, 128] bf16.  Same inputs, outputs and causal rule as the
 * absorbed steps 1-4 chained; about 120x their arithmetic.
 * Expanded keys and values are rounded to bf16 (as a materialised bf16 K/V
 * would be); scores, softmax and the value sum accumulate in fp32.
 * s_q must be <= 4 (else MLA_ERR_UNSUPPORTED).  softmax_scale finite and > 0.
 * workspace: ws_bytes >= mla_naive_workspace_bytes(...): a per-head transposed
 * copy of W_UV (H * 128 * 512 bf16), the scores of every (query row, cached
 * row) pair (B * s_q * H * T_cap fp32, T_cap = max_seqlen rounded up to 64)
 * and their row sums (B * s_q * H fp32), each rounded up to 256 bytes, all
 * written by the call; 0 from mla_naive_workspace_bytes means an invalid or
 * unreasonably large size argument (s_q > 4 included). */
size_t mla_naive_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen);
mla_status mla_naive_decode(const void* q, const mla_kv_desc* kv,
                            const void* w_uk, const void* w_uv,
                            int32_t B, int32_t s_q, int32_t H,
                            float softmax_scale, int32_t causal, void* out,
                            void* workspace, size_t ws_bytes, void* stream);

/* Latent append -- the step that produces the cached row of each new token
 * ("Why MLA and MTP Fight Each Other", section 3: the hidden state x is
 * compressed to the 512-wide latent c = x W_DKV that the cache stores;
 * Appendix A there and "MLA, dim by dim", "Why RoPE Gets in the Way": a
 * 64-wide rope key, rotated by the token's position and shared by all heads,
 * is stored beside the latent).  For token n with hidden state x[n]:
 *   row[c]       = sum_k x[n, k] * w_dkr[c, k]                      (c < 512)
 *   key[r]       = sum_k x[n, k] * w_dkr[512 + r, k]                (r < 64)
 *   row[512 + r] = key turned pairwise: for i < 32 and
 *                  a = pos[n] * rope_base^(-2 i / 64),
 *                  row[512 + 2i]     = key[2i] cos a - key[2i+1] sin a,
 *                  row[512 + 2i + 1] = key[2i] sin a + key[2i+1] cos a
 * (the pages leave the rotation's pairing and frequencies unwritten; this is
 * the rotary embedding on consecutive pairs).  The row is stored at position
 * pos[n] of sequence seq_id[n] of the cache `kv` describes (contiguous
 * [B, T_stride, 576] or paged through kv->block_table):
 *   MLA_BF16      each value rounded to nearest even;
 *   MLA_FP8_E4M3  scale = amax|row| / 448 (fp32, 1 for a zero row) written to
 *                 kv->row_scale, codes = E4M3(row / scale) rounded to nearest
 *                 even from the fp32 quotient, clamped to +-448, sign kept.
 * The call WRITES kv->rows and kv->row_scale (the descriptor's const
 * qualifiers describe the decode calls); kv->seqlens and kv->max_seqlen are
 * not used (the caller advances its lengths).
 *   x        bf16 [N, d_model]; w_dkr bf16 [576, d_model] (W_DKV^T in rows
 *            0..511, the rope-key projection W_KR^T in rows 512..575, the
 *            (out, in) order of a linear layer); d_model % 64 == 0.
 *   seq_id, pos  int32 [N].  A token whose seq_id is outside [0, B), whose
 *            pos is outside [0, T_stride) (contiguous) or [0, max_blocks * 64)
 *            (paged), or whose block-table entry is negative writes nothing.
 *            Two tokens with the same slot race.
 *   rope_base  finite and > 0 (10000 in the original rotary embedding).
 *   workspace  ws_bytes >= mla_append_workspace_bytes(N, d_model): fp32
 *            split-K partial rows, overwritten by the call.
 * Products accumulate in fp32 on the matrix cores; the rotation angles and
 * their sines and cosines are computed in fp64.  0 from
 * mla_append_workspace_bytes means an invalid size. */
size_t mla_append_workspace_bytes(int32_t N, int32_t d_model);
mla_status mla_latent_append(const void* x, const void* w_dkr, int32_t N, int32_t d_model,
                             const int32_t* seq_id, const int32_t* pos, float rope_base,
                             const mla_kv_desc* kv, int32_t B, void* workspace,
                             size_t ws_bytes, void* stream);

/* Prefill by expansion -- the other bracketing ("Why MLA and MTP Fight Each
 * Other", sections 5.5-5.6: with many query tokens per cached row, expanding
 * every row once into per-head keys and values and attending over them costs
 * fewer FLOPs than absorbing; "MLA, dim by dim", "MLA Prefill": materialise
 * K = C W_UK and V = C W_UV, then run standard attention).  Same inputs,
 * outputs and masking as mla_naive_decode (and as steps 1-4 chained):
 *   K_nope[t, h, :] = W_UK[h] row_t[0:512],  V[t, h, :] = row_t[0:512]^T W_UV[h]
 *   key_t = [K_nope[t, h, :] | row_t[512:576]]
 *   out[b, j, h, :] = sum_{t visible} softmax_t(scale * <q[b,j,h,:], key_t>) V[t, h, :]
 * with the causal rule of mla_decode_attn.  Keys and values are rounded to
 * bf16 in the workspace (FP8 rows are dequantised first); scores, softmax and
 * the value sum accumulate in fp32 on the matrix cores.
 *   q        bf16 [B, s_q, H, 192];  out  bf16 [B, s_q, H, 128]
 *   workspace  ws_bytes >= mla_prefill_workspace_bytes(B, s_q, H, max_seqlen):
 *            W_UV^T, K_nope and V [B, T_pad, H * 128 + 64] (token-major) and the rope keys
 *            [B, T_pad, 64], T_pad = max_seqlen rounded up to 128.
 * s_q <= max_seqlen; 0 from mla_prefill_workspace_bytes means an invalid size.
 * The expansion is a hand-written kernel for every cache kind. */
size_t mla_prefill_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen);
mla_status mla_prefill_expand(const void* q, const mla_kv_desc* kv, const void* w_uk,
                              const void* w_uv, int32_t B, int32_t s_q, int32_t H,
                              float softmax_scale, int32_t causal, void* out,
                              void* workspace, size_t ws_bytes, void* stream);

/* Dispatch between the two bracketings by their FLOP counts ("Why MLA and MTP
 * Fight Each Other", section 5.6): the expand path is used when
 *   s_q >= S*(L) = L d_c (d_k + d_v) / (d_c (d_k + d_v) + L (2 d_c - d_k - d_v)),
 * L = max_seqlen (S* is 128 at L = 512 and tends to 170.7), else the absorbed
 * path (mla_absorb_q, mla_decode_partial with bf16 partials,
 * mla_decode_combine_out).
 * mla_attend_uses_expand returns 1 (expand), 0 (absorbed) or -1 (bad sizes).
 * mla_attend takes the inputs and output of mla_prefill_expand and a
 * workspace of mla_attend_workspace_bytes(...) for the path it picks. */
int32_t mla_attend_uses_expand(int32_t s_q, int32_t max_seqlen);
size_t mla_attend_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen);
mla_status mla_attend(const void* q, const mla_kv_desc* kv, const void* w_uk, const void* w_uv,
                      int32_t B, int32_t s_q, int32_t H, float softmax_scale, int32_t causal,
                      void* out, void* workspace, size_t ws_bytes, void* stream);

/* Check of the device-resident preconditions of a cache description (a
 * debugging aid: the lengths and the block table are copied to the host and
 * the call waits for the copies on `stream`).  For every b < B:
 *   s_q <= seqlens[b] <= kv->max_seqlen;
 *   contiguous: seqlens[b] <= kv->T_stride;
 *   paged: seqlens[b] <= kv->max_blocks * 64, and every block id in the first
 *   ceil(seqlens[b] / 64) entries of row b of the block table lies in
 *   [0, n_pool_blocks).
 * n_pool_blocks: blocks in the pool (paged caches; ignored otherwise).
 * Returns MLA_OK, MLA_ERR_ARG (a precondition or an argument fails),
 * MLA_ERR_UNSUPPORTED (block size other than 64) or MLA_ERR_HIP (a copy
 * failed).  mla_validate_kv_host does the same on host copies of the arrays
 * (seqlens_host [B]; block_table_host [B, max_blocks], NULL for a
 * contiguous cache) and makes no HIP call. */
mla_status mla_validate_kv(const mla_kv_desc* kv, int32_t B, int32_t s_q,
                           int64_t n_pool_blocks, void* stream);
mla_status mla_validate_kv_host(const mla_kv_desc* kv, const int32_t* seqlens_host,
                                const int32_t* block_table_host, int32_t B, int32_t s_q,
                                int64_t n_pool_blocks);

/* Static, human-readable name of a status code (host). */
const char* mla_status_string(mla_status s);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
