// C ABI of libmla (declared in include/mla.h): argument validation, split
// planning and kernel launches on the caller's stream.  Every check that the
// host can make happens before the first HIP call, so a rejected call enqueues
// nothing.
#include "mla.h"

#include <cmath>
#include <cstdint>
#include <vector>

#include "mla_internal.h"

namespace {

constexpr int kRowsPerGroup = 128;   // query rows per work-group of the split-T scans
constexpr int kTileRows = 64;        // cached rows per plan tile
constexpr int kTargetWorkGroups = 256;  // one work-group per compute unit of an MI355X
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int32_t R, n_groups, n_split, n_ranges, n_work, work_per_xcd;
  int64_t n_slots;
  size_t part_o_bytes, part_lse_bytes, seg_bytes, mrun_bytes, ws_bytes;
};

// The plan depends on host integers only, so the workspace size and the
// reduction order are fixed for a given argument set.  n_split is the number
// of parts a sequence of max_seqlen rows is scanned in; the device cuts the
// tiles of all sequences into n_ranges = B * n_split equal ranges, so shorter
// sequences get proportionally fewer parts.  A range covers at most one part
// per sequence it touches: at most n_ranges + B partial slots.
bool make_plan(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen, int32_t forced, Plan* pl) {
  if (B <= 0 || s_q <= 0 || H <= 0 || max_seqlen <= 0 || forced < 0) return false;
  const int64_t R = (int64_t)s_q * H;
  if (R > (1 << 24) || B > (1 << 20) || max_seqlen > (1 << 28)) return false;
  pl->R = (int32_t)R;
  const int64_t tiles = (max_seqlen + kTileRows - 1) / kTileRows;
  pl->n_groups = (int32_t)((R + kRowsPerGroup - 1) / kRowsPerGroup);
  const int64_t base = (int64_t)B * pl->n_groups;
  int64_t ns = forced > 0 ? forced : (kTargetWorkGroups + base - 1) / base;
  if (ns < 1) ns = 1;
  if (ns > tiles) ns = tiles;
  pl->n_split = (int32_t)ns;
  const int64_t n_ranges = (int64_t)B * ns;
  pl->n_slots = n_ranges + B;
  const int64_t n_work = pl->n_slots * pl->n_groups;   // one work-group per (slot, row group)
  if (n_work > (int64_t)1 << 30) return false;
  pl->n_ranges = (int32_t)n_ranges;
  pl->n_work = (int32_t)n_work;
  pl->work_per_xcd = (int32_t)((n_work + 7) / 8);
  pl->part_o_bytes = align_up((size_t)pl->n_slots * R * mla::D_C * sizeof(float));
  pl->part_lse_bytes = align_up((size_t)pl->n_slots * R * sizeof(float));
  pl->seg_bytes = align_up((size_t)2 * B * sizeof(int32_t));
  // per-part maximum scores of the FP8-arithmetic scan (its accuracy check)
  pl->mrun_bytes = pl->part_lse_bytes;
  pl->ws_bytes = pl->part_o_bytes + pl->part_lse_bytes + pl->seg_bytes + pl->mrun_bytes;
  return true;
}

mla_status check_kv(const mla_kv_desc* kv, int32_t s_q) {
  if (kv == nullptr || kv->rows == nullptr || kv->seqlens == nullptr) return MLA_ERR_ARG;
  if (kv->dtype != MLA_BF16 && kv->dtype != MLA_FP8_E4M3) return MLA_ERR_ARG;
  if ((kv->dtype == MLA_FP8_E4M3) != (kv->row_scale != nullptr)) return MLA_ERR_ARG;
  if (kv->max_seqlen <= 0 || s_q > kv->max_seqlen) return MLA_ERR_ARG;
  if (kv->block_table != nullptr) {
    if (kv->block_size != kTileRows) return MLA_ERR_UNSUPPORTED;
    if (kv->max_blocks <= 0) return MLA_ERR_ARG;
    if ((int64_t)kv->max_seqlen > (int64_t)kv->max_blocks * kTileRows) return MLA_ERR_ARG;
  } else {
    if (kv->T_stride <= 0) return MLA_ERR_ARG;
    if (kv->max_seqlen > kv->T_stride) return MLA_ERR_ARG;
  }
  return MLA_OK;
}

mla_status hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Split-K layout of the append projection: about kTargetWorkGroups
// work-groups over the 18 column blocks and the 64-token blocks.
constexpr int kAppendColBlocks = mla::ROWW / 32;
bool append_split(int32_t N, int32_t d_model, int32_t* ks_count, int32_t* chunks_per_split) {
  if (N <= 0 || N > (1 << 20) || d_model < 64 || d_model % 64 != 0 || d_model > (1 << 20)) return false;
  const int64_t chunks = d_model / 64;
  const int64_t nz = (N + 63) / 64;
  int64_t ks = (kTargetWorkGroups + kAppendColBlocks * nz - 1) / (kAppendColBlocks * nz);
  if (ks > chunks) ks = chunks;
  if (ks < (chunks + 7) / 8) ks = (chunks + 7) / 8;     // at most 8 chunks (two per wave)
  if (ks < 1) ks = 1;
  const int64_t cps = (chunks + ks - 1) / ks;
  *chunks_per_split = (int32_t)cps;
  *ks_count = (int32_t)((chunks + cps - 1) / cps);
  return true;
}

struct PrefillLayout {
  int32_t T_pad;
  size_t wuvt_off, kn_off, v_off, rope_off, bytes;
};

// Workspace of the expand path: W_UV^T per head, then K_nope and V
// [B, T_pad, H * 128 + 64] (token-major; T_pad: max_seqlen rounded up to 128) and the rope keys [B, T_pad, 64] (bf16), 256-aligned.
bool prefill_layout(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen, PrefillLayout* l) {
  if (B <= 0 || s_q <= 0 || H <= 0 || max_seqlen <= 0 || s_q > max_seqlen) return false;
  if (B > (1 << 16) || H > (1 << 12) || max_seqlen > (1 << 24)) return false;
  if ((int64_t)B * s_q * H > (1 << 30)) return false;
  l->T_pad = (int32_t)((max_seqlen + 127) / 128 * 128);
  const size_t kv = (size_t)B * l->T_pad * mla::prefill_kv_ld(H) * sizeof(uint16_t);
  l->wuvt_off = 0;
  l->kn_off = align_up((size_t)H * mla::D_V * mla::D_C * sizeof(uint16_t));
  l->v_off = l->kn_off + align_up(kv);
  l->rope_off = l->v_off + align_up(kv);
  l->bytes = l->rope_off + align_up((size_t)B * l->T_pad * mla::D_ROPE * sizeof(uint16_t));
  return true;
}

// The query-token count from which expanding the cache is cheaper in FLOPs
// than absorbing: S*(L) = L d_c (d_k + d_v) / (d_c (d_k + d_v) + L (2 d_c - d_k - d_v))
// with d_k = d_v = 128 ("Why MLA and MTP Fight Each Other", section 5.6; the
// rope segment adds the same 64 to both per-pair costs and cancels).
double crossover_tokens(int32_t L) {
  const double expand = (double)mla::D_C * (mla::D_NOPE + mla::D_V);
  return (double)L * expand / (expand + (double)L * (2.0 * mla::D_C - mla::D_NOPE - mla::D_V));
}

bool use_expand(int32_t s_q, int32_t max_seqlen) { return (double)s_q >= crossover_tokens(max_seqlen); }

mla_status prefill_impl(const void* q, const mla_kv_desc* kv, const void* w_uk, const void* w_uv, int32_t B,
                        int32_t s_q, int32_t H, float softmax_scale, int32_t causal, void* out, void* workspace,
                        size_t ws_bytes, hipStream_t st) {
  if (q == nullptr || w_uk == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  PrefillLayout l;
  if (!prefill_layout(B, s_q, H, kv->max_seqlen, &l)) return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < l.bytes) return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  mla::PrefillParams p{};
  p.q = (const uint16_t*)q;
  p.rows = kv->rows;
  p.row_scale = kv->row_scale;
  p.block_table = kv->block_table;
  p.seqlens = kv->seqlens;
  p.w_uk = (const uint16_t*)w_uk;
  p.w_uv = (const uint16_t*)w_uv;
  p.w_uvt = (uint16_t*)(ws + l.wuvt_off);
  p.k_nope = (uint16_t*)(ws + l.kn_off);
  p.v = (uint16_t*)(ws + l.v_off);
  p.rope = (uint16_t*)(ws + l.rope_off);
  p.out = (uint16_t*)out;
  p.T_stride = kv->T_stride;
  p.max_blocks = kv->max_blocks;
  p.B = B;
  p.s_q = s_q;
  p.H = H;
  p.T_pad = l.T_pad;
  p.kv_ld = (int32_t)mla::prefill_kv_ld(H);
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.causal = causal;
  p.fp8 = kv->dtype == MLA_FP8_E4M3;
  return hip_status(mla::launch_prefill(p, st));
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_ARG: return "MLA_ERR_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported width, block size or dtype";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch failed";
  }
  return "unknown mla_status";
}

mla_status mla_absorb_q(const void* q, const void* w_uk, void* q_lat, int32_t N, int32_t H,
                        int32_t d_nope, int32_t d_rope, int32_t d_c, void* stream) {
  if (q == nullptr || w_uk == nullptr || q_lat == nullptr) return MLA_ERR_ARG;
  if (N <= 0 || H <= 0 || (int64_t)N * H > (1 << 26)) return MLA_ERR_ARG;
  if (d_nope != mla::D_NOPE || d_rope != mla::D_ROPE || d_c != mla::D_C) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_absorb_q((const uint16_t*)q, (const uint16_t*)w_uk, (uint16_t*)q_lat,
                                         N, H, (hipStream_t)stream));
}

size_t mla_decode_workspace_bytes_ex(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                                     int32_t num_splits) {
  Plan pl;
  if (!make_plan(B, s_q, H, max_seqlen, num_splits, &pl)) return 0;
  return pl.ws_bytes;
}

size_t mla_decode_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen) {
  return mla_decode_workspace_bytes_ex(B, s_q, H, max_seqlen, 0);
}

int32_t mla_decode_num_splits(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                              int32_t num_splits) {
  Plan pl;
  if (!make_plan(B, s_q, H, max_seqlen, num_splits, &pl)) return 0;
  return pl.n_split;
}

namespace {

// sel_idx != null: sparse top-k with the gather fused into the scan's loader
// (contiguous bf16 caches only); sel_count / k_max replace the lengths
mla_status decode_partial_impl(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q,
                               int32_t H, float softmax_scale, int32_t causal, void* workspace,
                               size_t ws_bytes, int32_t num_splits, int32_t part_dtype, hipStream_t st,
                               bool fp8_math = false,
                               const int32_t* sel_idx = nullptr, const int32_t* sel_count = nullptr,
                               int32_t k_max = 0) {
  if (q_lat == nullptr) return MLA_ERR_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || num_splits < 0) return MLA_ERR_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_ARG;
  if (part_dtype != MLA_FP32 && part_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  Plan pl;
  const int32_t plan_len = sel_idx != nullptr ? k_max : kv->max_seqlen;
  if (!make_plan(B, s_q, H, plan_len, num_splits, &pl)) return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < pl.ws_bytes) return MLA_ERR_WORKSPACE;

  mla::DecodeParams p{};
  p.q_lat = (const uint16_t*)q_lat;
  p.rows = kv->rows;
  p.row_scale = kv->row_scale;
  p.block_table = kv->block_table;
  p.seqlens = kv->seqlens;
  p.part_o = workspace;
  p.part_bf16 = part_dtype == MLA_BF16;
  p.part_lse = (float*)((char*)workspace + pl.part_o_bytes);
  p.seg_first = (int32_t*)((char*)workspace + pl.part_o_bytes + pl.part_lse_bytes);
  p.seg_count = p.seg_first + B;
  p.T_stride = kv->T_stride;
  p.max_blocks = kv->max_blocks;
  p.B = B;
  p.s_q = s_q;
  p.H = H;
  p.R = pl.R;
  p.n_groups = pl.n_groups;
  p.n_ranges = pl.n_ranges;
  p.n_work = pl.n_work;
  p.work_per_xcd = pl.work_per_xcd;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.causal = causal;
  p.paged = kv->block_table != nullptr;
  p.fp8 = kv->dtype == MLA_FP8_E4M3;
  if (sel_idx != nullptr) {
    p.seqlens = sel_count;
    p.src_len = kv->seqlens;
    p.sel_idx = sel_idx;
    p.k_max = k_max;
  }
  if (fp8_math) {
    if (!p.fp8) return MLA_ERR_UNSUPPORTED;
    // E4M3 arithmetic, then the bf16-arithmetic scan over the (sequence, row
    // group) pairs holding a row it cannot resolve to the FP8 bar (a peaked
    // softmax or few rows)
    p.part_mrun = (float*)((char*)workspace + pl.part_o_bytes + pl.part_lse_bytes + pl.seg_bytes);
    const hipError_t e = mla::launch_decode_split_f8(p, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    p.fixup = 1;
    return hip_status(mla::launch_decode_split(p, st));
  }
  return hip_status(mla::launch_decode_split(p, st));
}

mla_status decode_combine_impl(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                               int32_t num_splits, int32_t part_dtype, const void* workspace, size_t ws_bytes,
                               void* o_lat, int32_t o_lat_dtype, float* lse, hipStream_t st) {
  if (o_lat == nullptr) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (part_dtype != MLA_FP32 && part_dtype != MLA_BF16) return MLA_ERR_ARG;
  Plan pl;
  if (!make_plan(B, s_q, H, max_seqlen, num_splits, &pl)) return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < pl.ws_bytes) return MLA_ERR_WORKSPACE;
  const float* part_lse = (const float*)((const char*)workspace + pl.part_o_bytes);
  const int32_t* seg_first = (const int32_t*)((const char*)workspace + pl.part_o_bytes + pl.part_lse_bytes);
  return hip_status(mla::launch_combine(workspace, part_dtype == MLA_BF16, part_lse, seg_first, seg_first + B, B,
                                        pl.R, o_lat, o_lat_dtype == MLA_BF16, lse, st));
}

}  // namespace

mla_status mla_decode_partial(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q,
                              int32_t H, float softmax_scale, int32_t causal, void* workspace,
                              size_t ws_bytes, int32_t num_splits, int32_t part_dtype, void* stream) {
  return decode_partial_impl(q_lat, kv, B, s_q, H, softmax_scale, causal, workspace, ws_bytes,
                             num_splits, part_dtype, (hipStream_t)stream);
}

mla_status mla_decode_combine(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                              int32_t num_splits, int32_t part_dtype, const void* workspace, size_t ws_bytes,
                              void* o_lat, int32_t o_lat_dtype, float* lse, void* stream) {
  return decode_combine_impl(B, s_q, H, max_seqlen, num_splits, part_dtype, workspace, ws_bytes, o_lat,
                             o_lat_dtype, lse, (hipStream_t)stream);
}

mla_status mla_decode_combine_out(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen,
                                  int32_t num_splits, int32_t part_dtype, const void* workspace, size_t ws_bytes,
                                  const void* w_uv, void* out, void* o_lat, int32_t o_lat_dtype,
                                  float* lse, void* stream) {
  if (w_uv == nullptr || out == nullptr) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (part_dtype != MLA_FP32 && part_dtype != MLA_BF16) return MLA_ERR_ARG;
  Plan pl;
  if (!make_plan(B, s_q, H, max_seqlen, num_splits, &pl)) return MLA_ERR_ARG;
  if ((int64_t)B * s_q * H > (1 << 26)) return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < pl.ws_bytes) return MLA_ERR_WORKSPACE;
  const float* part_lse = (const float*)((const char*)workspace + pl.part_o_bytes);
  const int32_t* seg_first = (const int32_t*)((const char*)workspace + pl.part_o_bytes + pl.part_lse_bytes);
  return hip_status(mla::launch_combine_out(workspace, part_dtype == MLA_BF16, part_lse, seg_first, seg_first + B,
                                            B, s_q, H,
                                            (const uint16_t*)w_uv, (uint16_t*)out, o_lat,
                                            o_lat_dtype == MLA_BF16, lse, (hipStream_t)stream));
}

mla_status mla_decode_attn(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q,
                           int32_t H, float softmax_scale, int32_t causal, void* o_lat,
                           int32_t o_lat_dtype, float* lse, void* workspace, size_t ws_bytes,
                           void* stream) {
  return mla_decode_attn_ex(q_lat, kv, B, s_q, H, softmax_scale, causal, o_lat, o_lat_dtype, lse, workspace,
                            ws_bytes, 0, stream);
}

mla_status mla_decode_attn_ex(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q,
                              int32_t H, float softmax_scale, int32_t causal, void* o_lat,
                              int32_t o_lat_dtype, float* lse, void* workspace, size_t ws_bytes,
                              int32_t num_splits, void* stream) {
  // validate the outputs too before anything is enqueued
  if (o_lat == nullptr) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  // the partials are kept in the precision asked for the latent output
  const mla_status s = decode_partial_impl(q_lat, kv, B, s_q, H, softmax_scale, causal, workspace,
                                           ws_bytes, num_splits, o_lat_dtype, (hipStream_t)stream);
  if (s != MLA_OK) return s;
  return decode_combine_impl(B, s_q, H, kv->max_seqlen, num_splits, o_lat_dtype, workspace, ws_bytes, o_lat,
                             o_lat_dtype, lse, (hipStream_t)stream);
}

size_t mla_decode_noalloc_max_bytes(void) { return mla::NOALLOC_SCRATCH_BYTES; }

mla_status mla_decode_attn_noalloc(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q,
                                   int32_t H, float softmax_scale, int32_t causal, void* o_lat,
                                   int32_t o_lat_dtype, float* lse, void* stream) {
  // every argument check of mla_decode_attn, before any HIP call
  if (q_lat == nullptr || o_lat == nullptr) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0) return MLA_ERR_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  Plan pl;
  if (!make_plan(B, s_q, H, kv->max_seqlen, 0, &pl)) return MLA_ERR_ARG;
  if (pl.ws_bytes > mla::NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (mla::noalloc_scratch(&scratch) != hipSuccess) return MLA_ERR_HIP;
  return mla_decode_attn(q_lat, kv, B, s_q, H, softmax_scale, causal, o_lat, o_lat_dtype, lse, scratch,
                         mla::NOALLOC_SCRATCH_BYTES, stream);
}

mla_status mla_absorb_out(const void* o_lat, int32_t o_lat_dtype, const void* w_uv, void* out,
                          int32_t N, int32_t H, int32_t d_c, int32_t d_v, void* stream) {
  if (o_lat == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_ARG;
  if (N <= 0 || H <= 0 || (int64_t)N * H > (1 << 26)) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (d_c != mla::D_C || d_v != mla::D_V) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_absorb_out(o_lat, o_lat_dtype == MLA_BF16, (const uint16_t*)w_uv,
                                           (uint16_t*)out, N, H, (hipStream_t)stream));
}

namespace {

// Sparse workspace: [scan workspace for max_seqlen = k_max][compact rows]
// [clamped counts][compact scales (e4m3 only)]
bool sparse_layout(int32_t B, int32_t s_q, int32_t H, int32_t k_max, int32_t num_splits, int32_t dtype,
                   Plan* pl, size_t* rows_off, size_t* count_off, size_t* scale_off, size_t* total) {
  if (k_max <= 0 || (dtype != MLA_BF16 && dtype != MLA_FP8_E4M3)) return false;
  if (!make_plan(B, s_q, H, k_max, num_splits, pl)) return false;
  const size_t eb = dtype == MLA_FP8_E4M3 ? 1 : 2;
  *rows_off = pl->ws_bytes;
  *count_off = *rows_off + align_up((size_t)B * k_max * mla::ROWW * eb);
  *scale_off = *count_off + align_up((size_t)B * sizeof(int32_t));
  *total = *scale_off + (dtype == MLA_FP8_E4M3 ? align_up((size_t)B * k_max * sizeof(float)) : 0);
  return true;
}

}  // namespace

size_t mla_sparse_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t k_max, int32_t num_splits,
                                  int32_t cache_dtype) {
  Plan pl;
  size_t ro, co, so, total;
  if (!sparse_layout(B, s_q, H, k_max, num_splits, cache_dtype, &pl, &ro, &co, &so, &total)) return 0;
  return total;
}

mla_status mla_sparse_decode_partial(const void* q_lat, const mla_kv_desc* kv, const int32_t* sel_idx,
                                     const int32_t* sel_count, int32_t k_max, int32_t B, int32_t s_q,
                                     int32_t H, float softmax_scale, void* workspace, size_t ws_bytes,
                                     int32_t num_splits, int32_t part_dtype, void* stream) {
  if (q_lat == nullptr || sel_idx == nullptr || sel_count == nullptr) return MLA_ERR_ARG;
  if (part_dtype != MLA_FP32 && part_dtype != MLA_BF16) return MLA_ERR_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || k_max <= 0 || num_splits < 0) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, 1);
  if (ks != MLA_OK) return ks;
  Plan pl;
  size_t rows_off, count_off, scale_off, total;
  if (!sparse_layout(B, s_q, H, k_max, num_splits, kv->dtype, &pl, &rows_off, &count_off, &scale_off, &total))
    return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < total) return MLA_ERR_WORKSPACE;
  const bool fp8 = kv->dtype == MLA_FP8_E4M3;
  // contiguous bf16 caches whose sequences fit the loader's 32-bit window:
  // the scan gathers the selected rows itself
  if (kv->block_table == nullptr && !fp8 && (int64_t)kv->T_stride * mla::ROWW * 2 <= ((int64_t)1 << 30))
    return decode_partial_impl(q_lat, kv, B, s_q, H, softmax_scale, 0, workspace, pl.ws_bytes, num_splits,
                               part_dtype, (hipStream_t)stream, false, sel_idx, sel_count, k_max);
  mla::GatherParams g{};
  g.rows = kv->rows;
  g.row_scale = kv->row_scale;
  g.block_table = kv->block_table;
  g.seqlens = kv->seqlens;
  g.sel_idx = sel_idx;
  g.sel_count = sel_count;
  g.out_rows = (char*)workspace + rows_off;
  g.out_scale = fp8 ? (float*)((char*)workspace + scale_off) : nullptr;
  g.out_count = (int32_t*)((char*)workspace + count_off);
  g.T_stride = kv->T_stride;
  g.max_blocks = kv->max_blocks;
  g.B = B;
  g.k_max = k_max;
  g.fp8 = fp8;
  const hipError_t e = mla::launch_gather(g, (hipStream_t)stream);
  if (e != hipSuccess) return MLA_ERR_HIP;
  // scan the compact cache: sequence b holds sel_count[b] rows, no causal mask
  mla_kv_desc compact{};
  compact.rows = g.out_rows;
  compact.row_scale = g.out_scale;
  compact.block_table = nullptr;
  compact.seqlens = g.out_count;
  compact.dtype = kv->dtype;
  compact.T_stride = k_max;
  compact.block_size = 0;
  compact.max_blocks = 0;
  compact.max_seqlen = k_max;
  return decode_partial_impl(q_lat, &compact, B, s_q, H, softmax_scale, 0, workspace, pl.ws_bytes, num_splits,
                             part_dtype, (hipStream_t)stream);
}

mla_status mla_sparse_decode_attn(const void* q_lat, const mla_kv_desc* kv, const int32_t* sel_idx,
                                  const int32_t* sel_count, int32_t k_max, int32_t B, int32_t s_q, int32_t H,
                                  float softmax_scale, void* o_lat, int32_t o_lat_dtype, float* lse,
                                  void* workspace, size_t ws_bytes, int32_t num_splits, void* stream) {
  if (o_lat == nullptr) return MLA_ERR_ARG;
  if (o_lat_dtype != MLA_FP32 && o_lat_dtype != MLA_BF16) return MLA_ERR_ARG;
  const mla_status s = mla_sparse_decode_partial(q_lat, kv, sel_idx, sel_count, k_max, B, s_q, H, softmax_scale,
                                                 workspace, ws_bytes, num_splits, o_lat_dtype, stream);
  if (s != MLA_OK) return s;
  return decode_combine_impl(B, s_q, H, k_max, num_splits, o_lat_dtype, workspace, ws_bytes, o_lat, o_lat_dtype,
                             lse, (hipStream_t)stream);
}

size_t mla_naive_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen) {
  if (B <= 0 || s_q <= 0 || H <= 0 || max_seqlen <= 0 || H > (1 << 16) || B > (1 << 16)) return 0;
  if (s_q > mla::NAIVE_MAX_SQ || max_seqlen > (1 << 28)) return 0;
  if ((double)B * s_q * H * max_seqlen * 4.0 > (double)(1ull << 46)) return 0;   // 64 TiB: not a real size
  // W_UV re-laid out per head with the latent dimension contiguous, the
  // scores / probabilities [B, s_q, H, T_cap] and their sums [B, s_q, H]
  const size_t t_cap = ((size_t)max_seqlen + 63) / 64 * 64;
  return align_up((size_t)H * mla::D_V * mla::D_C * sizeof(uint16_t)) +
         align_up((size_t)B * s_q * H * t_cap * sizeof(float)) + align_up((size_t)B * s_q * H * sizeof(float));
}

mla_status mla_naive_decode(const void* q, const mla_kv_desc* kv, const void* w_uk, const void* w_uv,
                            int32_t B, int32_t s_q, int32_t H, float softmax_scale, int32_t causal,
                            void* out, void* workspace, size_t ws_bytes, void* stream) {
  if (q == nullptr || w_uk == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || H > (1 << 16) || B > (1 << 16)) return MLA_ERR_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  if (s_q > mla::NAIVE_MAX_SQ) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla_naive_workspace_bytes(B, s_q, H, kv->max_seqlen);
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  mla::NaiveParams p{};
  p.q = (const uint16_t*)q;
  p.rows = kv->rows;
  p.row_scale = kv->row_scale;
  p.block_table = kv->block_table;
  p.seqlens = kv->seqlens;
  p.w_uk = (const uint16_t*)w_uk;
  p.w_uv = (const uint16_t*)w_uv;
  const size_t t_cap = ((size_t)kv->max_seqlen + 63) / 64 * 64;
  const size_t wuvt_bytes = align_up((size_t)H * mla::D_V * mla::D_C * sizeof(uint16_t));
  const size_t score_bytes = align_up((size_t)B * s_q * H * t_cap * sizeof(float));
  p.w_uvt = (uint16_t*)workspace;
  p.scores = (float*)((char*)workspace + wuvt_bytes);
  p.lsum = (float*)((char*)workspace + wuvt_bytes + score_bytes);
  p.out = (uint16_t*)out;
  p.T_stride = kv->T_stride;
  p.max_blocks = kv->max_blocks;
  p.B = B;
  p.s_q = s_q;
  p.H = H;
  p.T_cap = (int32_t)t_cap;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.causal = causal;
  p.fp8 = kv->dtype == MLA_FP8_E4M3;
  return hip_status(mla::launch_naive(p, (hipStream_t)stream));
}

size_t mla_append_workspace_bytes(int32_t N, int32_t d_model) {
  int32_t ks, spp;
  if (!append_split(N, d_model, &ks, &spp)) return 0;
  return align_up((size_t)ks * N * mla::ROWW * sizeof(float));
}

mla_status mla_latent_append(const void* x, const void* w_dkr, int32_t N, int32_t d_model,
                             const int32_t* seq_id, const int32_t* pos, float rope_base,
                             const mla_kv_desc* kv, int32_t B, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (x == nullptr || w_dkr == nullptr || seq_id == nullptr || pos == nullptr || kv == nullptr) return MLA_ERR_ARG;
  int32_t ks, spp;
  if (!append_split(N, d_model, &ks, &spp)) return MLA_ERR_ARG;
  if (B <= 0 || !std::isfinite(rope_base) || !(rope_base > 0.f)) return MLA_ERR_ARG;
  if (kv->rows == nullptr) return MLA_ERR_ARG;
  if (kv->dtype != MLA_BF16 && kv->dtype != MLA_FP8_E4M3) return MLA_ERR_ARG;
  if ((kv->dtype == MLA_FP8_E4M3) != (kv->row_scale != nullptr)) return MLA_ERR_ARG;
  if (kv->block_table != nullptr) {
    if (kv->block_size != kTileRows) return MLA_ERR_UNSUPPORTED;
    if (kv->max_blocks <= 0) return MLA_ERR_ARG;
  } else if (kv->T_stride <= 0) {
    return MLA_ERR_ARG;
  }
  if (workspace == nullptr || ws_bytes < mla_append_workspace_bytes(N, d_model)) return MLA_ERR_WORKSPACE;
  mla::AppendParams p{};
  p.x = (const uint16_t*)x;
  p.w = (const uint16_t*)w_dkr;
  p.part = (float*)workspace;
  p.seq_id = seq_id;
  p.pos = pos;
  p.rows = const_cast<void*>(kv->rows);
  p.row_scale = const_cast<float*>(kv->row_scale);
  p.block_table = kv->block_table;
  p.T_stride = kv->T_stride;
  p.max_blocks = kv->max_blocks;
  p.B = B;
  p.N = N;
  p.d = d_model;
  p.ks_count = ks;
  p.chunks_per_split = spp;
  p.log2_base = std::log2((double)rope_base);
  p.fp8 = kv->dtype == MLA_FP8_E4M3;
  return hip_status(mla::launch_append(p, (hipStream_t)stream));
}

size_t mla_prefill_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen) {
  PrefillLayout l;
  return prefill_layout(B, s_q, H, max_seqlen, &l) ? l.bytes : 0;
}

mla_status mla_prefill_expand(const void* q, const mla_kv_desc* kv, const void* w_uk, const void* w_uv,
                              int32_t B, int32_t s_q, int32_t H, float softmax_scale, int32_t causal,
                              void* out, void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(q, kv, w_uk, w_uv, B, s_q, H, softmax_scale, causal, out, workspace, ws_bytes,
                      (hipStream_t)stream);
}

int32_t mla_attend_uses_expand(int32_t s_q, int32_t max_seqlen) {
  if (s_q <= 0 || max_seqlen <= 0) return -1;
  return use_expand(s_q, max_seqlen) ? 1 : 0;
}

size_t mla_attend_workspace_bytes(int32_t B, int32_t s_q, int32_t H, int32_t max_seqlen) {
  if (B <= 0 || s_q <= 0 || H <= 0 || max_seqlen <= 0) return 0;
  if (use_expand(s_q, max_seqlen)) return mla_prefill_workspace_bytes(B, s_q, H, max_seqlen);
  if ((int64_t)B * s_q * H > (1 << 26)) return 0;
  Plan pl;
  if (!make_plan(B, s_q, H, max_seqlen, 0, &pl)) return 0;
  return align_up((size_t)B * s_q * H * mla::ROWW * sizeof(uint16_t)) + pl.ws_bytes;
}

mla_status mla_attend(const void* q, const mla_kv_desc* kv, const void* w_uk, const void* w_uv, int32_t B,
                      int32_t s_q, int32_t H, float softmax_scale, int32_t causal, void* out, void* workspace,
                      size_t ws_bytes, void* stream) {
  if (kv == nullptr || q == nullptr || w_uk == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_ARG;
  if (B <= 0 || s_q <= 0 || H <= 0 || kv->max_seqlen <= 0) return MLA_ERR_ARG;
  const hipStream_t st = (hipStream_t)stream;
  if (use_expand(s_q, kv->max_seqlen))
    return prefill_impl(q, kv, w_uk, w_uv, B, s_q, H, softmax_scale, causal, out, workspace, ws_bytes, st);
  // absorbed: q_lat in the workspace, then the split-T scan and the fused
  // merge + W_UV projection on the rest of it
  if ((int64_t)B * s_q * H > (1 << 26)) return MLA_ERR_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  const size_t need = mla_attend_workspace_bytes(B, s_q, H, kv->max_seqlen);
  if (need == 0) return MLA_ERR_ARG;
  if (workspace == nullptr || ws_bytes < need) return MLA_ERR_WORKSPACE;
  const size_t ql_bytes = align_up((size_t)B * s_q * H * mla::ROWW * sizeof(uint16_t));
  void* q_lat = workspace;
  void* dws = (char*)workspace + ql_bytes;
  const size_t dws_bytes = ws_bytes - ql_bytes;
  mla_status s = mla_absorb_q(q, w_uk, q_lat, B * s_q, H, mla::D_NOPE, mla::D_ROPE, mla::D_C, stream);
  if (s != MLA_OK) return s;
  // bf16 partials: the output is bf16
  s = decode_partial_impl(q_lat, kv, B, s_q, H, softmax_scale, causal, dws, dws_bytes, 0, MLA_BF16, st);
  if (s != MLA_OK) return s;
  return mla_decode_combine_out(B, s_q, H, kv->max_seqlen, 0, MLA_BF16, dws, dws_bytes, w_uv, out, nullptr,
                                MLA_FP32, nullptr, stream);
}

mla_status mla_decode_partial_fp8(const void* q_lat, const mla_kv_desc* kv, int32_t B, int32_t s_q, int32_t H,
                                  float softmax_scale, int32_t causal, void* workspace, size_t ws_bytes,
                                  int32_t num_splits, int32_t part_dtype, void* stream) {
  return decode_partial_impl(q_lat, kv, B, s_q, H, softmax_scale, causal, workspace, ws_bytes, num_splits,
                             part_dtype, (hipStream_t)stream, true);
}

mla_status mla_validate_kv_host(const mla_kv_desc* kv, const int32_t* seqlens_host,
                                const int32_t* block_table_host, int32_t B, int32_t s_q,
                                int64_t n_pool_blocks) {
  if (kv == nullptr || seqlens_host == nullptr || B <= 0 || s_q <= 0) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  const bool paged = kv->block_table != nullptr;
  if (paged && (block_table_host == nullptr || n_pool_blocks <= 0)) return MLA_ERR_ARG;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t T = seqlens_host[b];
    if (T < s_q || T > kv->max_seqlen) return MLA_ERR_ARG;
    if (!paged) {
      if (T > kv->T_stride) return MLA_ERR_ARG;
      continue;
    }
    if (T > (int64_t)kv->max_blocks * kTileRows) return MLA_ERR_ARG;
    const int32_t* row = block_table_host + (int64_t)b * kv->max_blocks;
    for (int64_t i = 0; i < (T + kTileRows - 1) / kTileRows; ++i)
      if (row[i] < 0 || row[i] >= n_pool_blocks) return MLA_ERR_ARG;
  }
  return MLA_OK;
}

mla_status mla_validate_kv(const mla_kv_desc* kv, int32_t B, int32_t s_q, int64_t n_pool_blocks,
                           void* stream) {
  if (kv == nullptr || B <= 0 || B > (1 << 24) || s_q <= 0) return MLA_ERR_ARG;
  const mla_status ks = check_kv(kv, s_q);
  if (ks != MLA_OK) return ks;
  const bool paged = kv->block_table != nullptr;
  if (paged && n_pool_blocks <= 0) return MLA_ERR_ARG;
  const hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> lens((size_t)B);
  std::vector<int32_t> table(paged ? (size_t)B * kv->max_blocks : 0);
  if (hipMemcpyAsync(lens.data(), kv->seqlens, lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
      hipSuccess)
    return MLA_ERR_HIP;
  if (paged && hipMemcpyAsync(table.data(), kv->block_table, table.size() * sizeof(int32_t),
                              hipMemcpyDeviceToHost, st) != hipSuccess)
    return MLA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return MLA_ERR_HIP;
  return mla_validate_kv_host(kv, lens.data(), paged ? table.data() : nullptr, B, s_q, n_pool_blocks);
}

}  // extern "C"



