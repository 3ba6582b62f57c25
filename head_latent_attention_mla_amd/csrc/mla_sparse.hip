// Sparse top-k decode, gather step: copy the selected cached rows of every
// sequence into a compact contiguous cache, which the split-T scan then reads
// like any contiguous cache ("Why MLA and MTP Fight Each Other", section 6:
// the selected latents are gathered by index and only they are scored and
// averaged).
//
// One wave per selected row: 64 lanes x 16 bytes stream the row (1152 bytes
// bf16 or 576 bytes of e4m3 codes; lane 0 also copies the row scale).  An
// index outside [0, seqlens[b]) gathers a zero row (scale 0) and reads
// nothing; counts are clamped to [0, k_max].
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

__global__ __launch_bounds__(256) void gather_rows_kernel(GatherParams p) {
  const int b = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;                 // selected entry of sequence b
  const int cnt = min(max(p.sel_count[b], 0), p.k_max);
  // the scan reads this clamped count, so it never walks past the compact rows
  if (blockIdx.x == 0 && threadIdx.x == 0) p.out_count[b] = cnt;
  if (i >= cnt) return;                                  // wave-uniform; no barriers follow
  const int row_bytes = ROWW * (p.fp8 ? 1 : 2);
  const int pos = p.sel_idx[(int64_t)b * p.k_max + i];
  const bool valid = pos >= 0 && pos < p.seqlens[b];
  int64_t src_row = 0;
  if (valid) {
    src_row = p.block_table != nullptr
                  ? (int64_t)p.block_table[(int64_t)b * p.max_blocks + (pos >> 6)] * 64 + (pos & 63)
                  : (int64_t)b * p.T_stride + pos;
  }
  const char* src = (const char*)p.rows + src_row * row_bytes;
  char* dst = (char*)p.out_rows + ((int64_t)b * p.k_max + i) * row_bytes;
  for (int c = lane; c < row_bytes / 16; c += 64) {
    const u32x4 v = valid ? *(const u32x4*)(src + c * 16) : u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(dst + c * 16) = v;
  }
  if (p.fp8 && lane == 0) p.out_scale[(int64_t)b * p.k_max + i] = valid ? p.row_scale[src_row] : 0.f;
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3((p.k_max + 3) / 4, p.B), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
