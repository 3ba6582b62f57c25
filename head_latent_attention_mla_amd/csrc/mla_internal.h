// Host-side launch interface between the C ABI layer (mla_api.cpp) and the
// HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Fixed widths of the DeepSeek-V3-style latent attention.
constexpr int D_NOPE = 128;          // per-head no-rope query/key width
constexpr int D_ROPE = 64;           // decoupled rope key width (shared by heads)
constexpr int D_QK = D_NOPE + D_ROPE;  // 192: query row
constexpr int D_C = 512;             // latent width
constexpr int D_V = 128;             // per-head value width
constexpr int ROWW = D_C + D_ROPE;   // 576: cached row / latent query row


// One launch of the split-T latent-attention kernel.
struct DecodeParams {
  const uint16_t* q_lat;        // bf16 [B, R, 576], R = s_q * H
  const void* rows;             // cache rows (contiguous or pool), bf16 or e4m3
  const float* row_scale;       // e4m3 only
  const int32_t* block_table;   // paged only
  const int32_t* seqlens;       // [B]
  void* part_o;                 // [n_ranges + B, R, 512] normalised partial outputs, fp32 or bf16
  float* part_lse;              // fp32 [n_ranges + B, R], log2-domain log-sum-exp
  int32_t* seg_first;           // [B] first partial slot of each sequence
  int32_t* seg_count;           // [B] number of partial slots of each sequence
  int64_t T_stride;
  int32_t max_blocks;
  int32_t B, s_q, H, R;
  int32_t n_groups;             // ceil(R / 128) row groups per sequence
  int32_t n_ranges;             // equal ranges of the tiles of all sequences
  int32_t n_work, work_per_xcd; // n_ranges * n_groups work items over 8 XCDs
  float scale_log2;             // softmax scale * log2(e)
  int32_t causal;
  int32_t paged;
  int32_t fp8;
  // sparse top-k with the gather fused into the loader (contiguous bf16
  // caches): seqlens then holds the selection counts
  const int32_t* sel_idx;       // [B, k_max] selected positions, or null
  const int32_t* src_len;       // [B] cache lengths
  int32_t k_max;
  int32_t part_bf16;            // partial outputs stored as bf16 (else fp32)
  // FP8-arithmetic scan: fp32 [n_slots, R], each part's running maximum of
  // every query row's scaled scores (log2 domain, like part_lse); null: not
  // written
  float* part_mrun;
  // bf16-arithmetic scan run as a fix-up after the FP8-arithmetic one: a
  // (sequence, row group) is recomputed only if one of its query rows has a
  // largest probability above 1/32 of the row's total (max over parts of
  // part_mrun against the merged log-sum-exp); the rest exit after the plan
  int32_t fixup;
};

// One call of the naive (expand-then-attend) ablation.
struct NaiveParams {
  const uint16_t* q;            // bf16 [B, s_q, H, 192]
  const void* rows;             // cache rows (contiguous or pool), bf16 or e4m3
  const float* row_scale;       // e4m3 only
  const int32_t* block_table;   // paged only (else null)
  const int32_t* seqlens;       // [B]
  const uint16_t* w_uk;         // bf16 [H, 128, 512]
  const uint16_t* w_uv;         // bf16 [H, 512, 128]
  uint16_t* w_uvt;              // workspace: bf16 [H, 128, 512]
  float* scores;                // workspace: fp32 [B, s_q, H, T_cap], scores then probabilities
  float* lsum;                  // workspace: fp32 [B, s_q, H], sums of the probabilities
  uint16_t* out;                // bf16 [B, s_q, H, 128]
  int64_t T_stride;
  int32_t max_blocks;
  int32_t B, s_q, H;
  int32_t T_cap;                // max_seqlen rounded up to 64 (row pitch of scores)
  float scale_log2;
  int32_t causal;
  int32_t fp8;
};
constexpr int NAIVE_MAX_SQ = 4;

// One gather of selected cache rows into a compact contiguous cache.
struct GatherParams {
  const void* rows;             // source cache rows (contiguous or pool), bf16 or e4m3
  const float* row_scale;       // e4m3 only
  const int32_t* block_table;   // paged source only (else null)
  const int32_t* seqlens;       // [B] source lengths
  const int32_t* sel_idx;       // [B, k_max] selected positions
  const int32_t* sel_count;     // [B] entries used per sequence
  void* out_rows;               // [B, k_max, 576] compact rows
  float* out_scale;             // [B, k_max] (e4m3 only)
  int32_t* out_count;           // [B] counts clamped to [0, k_max]
  int64_t T_stride;
  int32_t max_blocks;
  int32_t B, k_max;
  int32_t fp8;
};

// One latent append: project, rotate and store the rows of N new tokens.
struct AppendParams {
  const uint16_t* x;            // bf16 [N, d] hidden states
  const uint16_t* w;            // bf16 [576, d]: W_DKV^T rows 0..511, W_KR^T rows 512..575
  float* part;                  // workspace: fp32 [ks_count, N, 576] split-K partial rows
  const int32_t* seq_id;        // [N] sequence of each token
  const int32_t* pos;           // [N] position of each token in its sequence
  void* rows;                   // cache rows (contiguous [B, T_stride] or pool), bf16 or e4m3
  float* row_scale;             // e4m3 only
  const int32_t* block_table;   // paged only (else null)
  int64_t T_stride;
  int32_t max_blocks;
  int32_t B, N, d;
  int32_t ks_count;             // K splits
  int32_t chunks_per_split;     // 64-wide k-chunks per split
  double log2_base;             // log2 of the rope base
  int32_t fp8;
};

// One call of the expand (prefill) path: expand every cached row per head
// into K_nope and V, then causal flash attention with the 192-wide queries.
// Token rows of the expanded keys and values hold the H heads' 128 values
// and 64 elements of padding, so that the rows of one head are not a power
// of two apart (those map a tile's rows onto few cache sets and channels).
inline int64_t prefill_kv_ld(int64_t H) { return H * D_NOPE + 64; }

struct PrefillParams {
  const uint16_t* q;            // bf16 [B, s_q, H, 192]
  const void* rows;             // cache rows (contiguous or pool), bf16 or e4m3
  const float* row_scale;       // e4m3 only
  const int32_t* block_table;   // paged only (else null)
  const int32_t* seqlens;       // [B]
  const uint16_t* w_uk;         // bf16 [H, 128, 512]
  const uint16_t* w_uv;         // bf16 [H, 512, 128]
  uint16_t* w_uvt;              // workspace: bf16 [H, 128, 512], W_UV per head transposed
  uint16_t* k_nope;             // workspace: bf16 [B, T_pad, kv_ld] (token-major, head h at h * 128)
  uint16_t* v;                  // workspace: bf16 [B, T_pad, kv_ld] (token-major, head h at h * 128)
  uint16_t* rope;               // workspace: bf16 [B, T_pad, 64]
  uint16_t* out;                // bf16 [B, s_q, H, 128]
  int64_t T_stride;
  int32_t max_blocks;
  int32_t B, s_q, H;
  int32_t T_pad;                // rows per sequence in the expanded buffers (multiple of 128)
  int32_t kv_ld;                // elements per token row of K_nope and V: H * 128 + 64
  float scale_log2;
  int32_t causal;
  int32_t fp8;
};

// Allocation-free decode: the split workspace is a file-scope device array of
// this many bytes (mla_noalloc.hip); noalloc_scratch() gives the current
// device's address of it (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_decode_split(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_split_f8(const DecodeParams& p, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
// part_o: fp32 partials, or bf16 when part_bf16 is set
hipError_t launch_combine(const void* part_o, int part_bf16, const float* part_lse, const int32_t* seg_first,
                          const int32_t* seg_count, int B, int R, void* o_lat, int o_bf16, float* lse,
                          hipStream_t stream);
hipError_t launch_absorb_q(const uint16_t* q, const uint16_t* w_uk, uint16_t* q_lat, int N, int H,
                           hipStream_t stream);
hipError_t launch_absorb_out(const void* o_lat, int o_bf16, const uint16_t* w_uv, uint16_t* out,
                             int N, int H, hipStream_t stream);
hipError_t launch_combine_out(const void* part_o, int part_bf16, const float* part_lse, const int32_t* seg_first,
                              const int32_t* seg_count, int B, int s_q, int H, const uint16_t* w_uv,
                              uint16_t* out, void* o_lat, int o_bf16, float* lse, hipStream_t stream);
hipError_t launch_naive(const NaiveParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_transpose_wuv(const uint16_t* w_uv, uint16_t* w_uvt, int H, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace mla
