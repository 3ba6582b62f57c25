// Naive (expand) MLA decode, kept as an ablation of the absorbed path.
//
// Every visible cached row is re-expanded per head on every call: the key
// K[t] = [W_UK[h] c_t[0:512] | c_t[512:576]] and the value V[t] =
// c_t[0:512]^T W_UV[h], then ordinary softmax attention with the 192-wide
// query ("The MLA decode speedup hiding in your model card", "The naive form,
// written out"; "Why MLA and MTP Fight Each Other", section 5.1: expanding
// bills the up-projection to every cached token, about 120x the absorbed
// arithmetic at these widths).  Expanded keys and values are rounded to bf16,
// as materialised ones would be; scores, softmax and sums are fp32.
//
// Three passes, each walking every cached row of its sequences once per head:
//   1. naive_pass_kernel<*, false>: K_nope^T = W_UK[h] C^T on MFMA, then the
//      scores of the s_q query tokens (log2 units) into the workspace;
//   2. naive_softmax_kernel: per query row, the maximum, the exponentials
//      (in place) and their sum;
//   3. naive_pass_kernel<*, true>: V^T = W_UV[h]^T C^T on MFMA, then
//      out = sum_t p_t V[t] / sum_t p_t.
// One work-group per (head, part of the batch), one per compute unit.  The
// head's weight (W_UK[h], or W_UV[h] transposed) stays in registers as MFMA A
// fragments for the whole pass (wave w: outputs 32 w .. 32 w + 31, 128 VGPRs
// a lane) and the cached rows stream through LDS in 64-row tiles,
// double-buffered, in the latent scan's tile layout (direct-to-LDS loads,
// 16-byte chunks XOR-swizzled per row), so every cached byte is read from
// LDS once per pass.  The work-groups of one XCD take consecutive heads of
// one part of the batch, so they walk the same rows through that XCD's L2.
#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int MAX_SQ = NAIVE_MAX_SQ;       // query tokens handled per work-group

// W_UV [H][512][128] -> W_UV^T [H][128][512] (contracted dimension contiguous)
__global__ __launch_bounds__(256) void transpose_wuv_kernel(const uint16_t* __restrict__ w_uv,
                                                            uint16_t* __restrict__ w_uvt) {
  __shared__ uint16_t t[64][65];
  const int h = blockIdx.z, c0 = blockIdx.x * 64, v0 = blockIdx.y * 64;
  const uint16_t* src = w_uv + (int64_t)h * D_C * D_V;
  uint16_t* dst = w_uvt + (int64_t)h * D_V * D_C;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    t[r][c] = src[(int64_t)(c0 + r) * D_V + v0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    dst[(int64_t)(v0 + r) * D_C + c0 + c] = t[c][r];
  }
}

constexpr int XT = 64;                          // cached rows per tile
constexpr int XCH = ROWW * 2 / 16;              // 72 16-byte chunks per bf16 row
constexpr int XTILE = XT * ROWW * 2;            // 73,728: bf16 tile
constexpr int XSTAGE = XT * ROWW;               // 36,864: e4m3 codes of a tile
constexpr int X_RING = 4;                       // k-steps of cached-row fragments in flight
static_assert(XTILE + 2 * XSTAGE == 2 * XTILE, "E4M3 layout fits the bf16 one");

// LDS byte offset of element e of tile row t (the latent scan's tile layout)
__device__ __forceinline__ int xoff(int t, int e) { return (t * XCH + ((e >> 3) ^ tile_swz(t))) * 16 + (e & 7) * 2; }

__device__ __forceinline__ float round_bf16(float x) { return bf16_bits_to_float(bf16_bits(to_bf16(x))); }

template <bool FP8, bool VALUES>
__global__ __launch_bounds__(256, 1) void naive_pass_kernel(NaiveParams p, int n_parts, int per_xcd) {
  // bf16 rows: tile buffers 0 and 1; E4M3 rows: the bf16 tile, then two code buffers
  __shared__ __attribute__((aligned(1024))) char smem[2 * XTILE];
  __shared__ __attribute__((aligned(16))) float qsh[MAX_SQ][D_QK];   // the sequence's queries (scores)
  __shared__ float red[4][MAX_SQ][XT];                              // per-wave partial scores
  const uint32_t smem_a = lds_addr(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = p.H, s_q = p.s_q;
  // XCD-aware order: launch slot L runs on XCD L % 8, which takes the
  // consecutive items (part-major, then head) L % 8 * per_xcd ..
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= H * n_parts) return;
  const int part = item / H, h = item % H;
  const int b_lo = (int)((int64_t)part * p.B / n_parts), b_hi = (int)((int64_t)(part + 1) * p.B / n_parts);

  // the tile loader of the latent scan: wave w copies rows 16 w .. + 15, 18
  // loads of 1 KB (9 for E4M3 codes, plain order into a staging buffer)
  uint32_t loff[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 18; ++k) {
    const int sl = 64 * (k % 9) + lane;
    const int tl = sl / XCH;
    const int c = (sl - tl * XCH) ^ tile_swz(tl + (k >= 9 ? 8 : 0));
    loff[k >> 1] |= (uint32_t)(tl * ROWW * 2 + c * 16) << (16 * (k & 1));
  }
  constexpr int ELEM = FP8 ? 1 : 2;
  const int soff = wave * (16 * ROWW * ELEM);
  float sc_next = 0.f;                            // E4M3: scale of row tid / 4 of the next tile
  // tile `tile` of sequence b (T rows) into buffer tile & 1; live = false
  // gives an empty window (the loads fetch nothing and write zeros), so the
  // loop issues loads on every tile with no branch around them
  auto issue_tile = [&](int b, int T, int tile, bool live) {
    const int t0 = tile * XT;
    const int valid = __builtin_amdgcn_readfirstlane(live ? min(XT, T - t0) : 0);
    int64_t r0 = 0;
    if (valid == 0)
      r0 = 0;
    else if (p.block_table != nullptr)
      r0 = (int64_t)__builtin_amdgcn_readfirstlane(p.block_table[(int64_t)b * p.max_blocks + (t0 >> 6)]) * XT;
    else
      r0 = (int64_t)b * p.T_stride + t0;
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.rows + r0 * ROWW * ELEM), (short)0,
                                                        valid * ROWW * ELEM, 0x00020000);
    const int buf = tile & 1;
    if constexpr (FP8) {
      char* dst = smem + XTILE + buf * XSTAGE + wave * (16 * ROWW);
      static_for<0, 9>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + k * 1024), 16, lane * 16, soff + k * 1024, 0, 0);
      });
      const int t = tid >> 2;
      sc_next = t < valid ? p.row_scale[r0 + t] : 0.f;
    } else {
      char* dst = smem + buf * XTILE + wave * (16 * ROWW * 2);
      static_for<0, 18>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const uint32_t vo = (loff[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + k * 1024), 16, vo,
                                                 soff + (k >= 9 ? 8 * ROWW * 2 : 0), 0, 0);
      });
    }
  };
  // E4M3: thread tid converts row tid / 4, quarter tid % 4 (144 codes); the
  // nine 16-code chunks are read first, then converted two values per
  // conversion instruction
  auto convert_tile = [&](int buf, float scale) {
    const int t = tid >> 2, cq = tid & 3;
    const char* src = smem + XTILE + buf * XSTAGE + t * ROWW + cq * 9 * 16;
    u32x4 w[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = *(const u32x4*)(src + i * 16);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int m = cq * 9 + i;
      uint64_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i][d], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i][d], true);
        o[d] = pack_bf16x4(f32x4{lo[0] * scale, lo[1] * scale, hi[0] * scale, hi[1] * scale});
      }
      *(u32x4*)(smem + xoff(t, 16 * m)) = u32x4{(uint32_t)o[0], (uint32_t)(o[0] >> 32), (uint32_t)o[1], (uint32_t)(o[1] >> 32)};
      *(u32x4*)(smem + xoff(t, 16 * m + 8)) = u32x4{(uint32_t)o[2], (uint32_t)(o[2] >> 32), (uint32_t)o[3], (uint32_t)(o[3] >> 32)};
    }
  };

  // B-fragment reads: tile row l32 (+ 32), logical chunk 2 ks + half; for
  // ks = 4 m + i the XOR touches only the low 3 bits, so 4 lane offsets and
  // an immediate 128 m cover every read (rows 32 apart share the pattern)
  uint32_t boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) boff[i] = l32 * (XCH * 16) + 16 * ((2 * i + half) ^ tile_swz(l32));

  // A fragments: weight row 32 wave + l32, columns 16 ks + 8 half .. + 7
  i16x8 aw[D_C / 16];
  {
    const uint16_t* W = (VALUES ? p.w_uvt : p.w_uk) + ((int64_t)h * D_NOPE + 32 * wave + l32) * D_C + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D_C / 16; ++ks) aw[ks] = *(const i16x8*)(W + 16 * ks);
  }

  for (int b = b_lo; b < b_hi; ++b) {
    const int T = __builtin_amdgcn_readfirstlane(min(p.seqlens[b], p.T_cap));
    const int n_tiles = (T + XT - 1) / XT;
    const int64_t srow0 = ((int64_t)b * s_q * H + h) * p.T_cap;   // scores row of query 0; query j at + j H T_cap
    __syncthreads();                     // the previous sequence's LDS is consumed
    if constexpr (!VALUES) {
      for (int i = tid; i < s_q * D_QK; i += 256) {
        const int j = i / D_QK, k = i - j * D_QK;
        qsh[j][k] = bf16_bits_to_float(p.q[(((int64_t)b * s_q + j) * H + h) * D_QK + k]);
      }
    }
    // value sums of this lane's 16 outputs (n = 32 wave + 8 g + 4 half + e)
    float oacc[MAX_SQ][16];
#pragma unroll
    for (int j = 0; j < MAX_SQ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[j][r] = 0.f;
    if (n_tiles > 0) issue_tile(b, T, 0, true);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int tile = 0; tile < n_tiles; ++tile) {
      barrier_tile_ready();            // tile landed; every wave is past the previous tile
      const int t0 = tile * XT;
      uint32_t tb_a;
      if constexpr (FP8) {
        convert_tile(tile & 1, sc_next);
        barrier_lds();
        tb_a = smem_a;
      } else {
        tb_a = smem_a + (tile & 1) * XTILE;
      }
      // values: the probabilities of this lane's two rows, fetched before the
      // next tile's loads are issued (so waiting for them does not wait for those)
      float pj[MAX_SQ][2];
      if constexpr (VALUES) {
#pragma unroll
        for (int j = 0; j < MAX_SQ; ++j)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const int t = t0 + 32 * tb + l32;
            pj[j][tb] = (j < s_q && t < T) ? p.scores[srow0 + (int64_t)j * H * p.T_cap + t] : 0.f;
          }
      }
      issue_tile(b, T, tile + 1, tile + 1 < n_tiles);
      uint32_t ba[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ba[i] = tb_a + boff[i];
      i16x8 rb[X_RING][2];
      auto issue_b = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        lds_read_b128<128 * (ks >> 2)>(rb[ks % X_RING][0], ba[ks & 3]);
        lds_read_b128<128 * (ks >> 2) + 32 * XCH * 16>(rb[ks % X_RING][1], ba[ks & 3]);
      };
      static_for<0, X_RING - 1>(issue_b);
      static_for<0, D_C / 16>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int last = D_C / 16 - 1;
        constexpr int ahead = (last - ks) < (X_RING - 1) ? (last - ks) : (X_RING - 1);
        if constexpr (ks + X_RING - 1 <= last) issue_b(std::integral_constant<int, ks + X_RING - 1>{});
        constexpr int slot = ks % X_RING;
        wait_lgkm<2 * ahead>(rb[slot][0], rb[slot][1]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, aw[ks]);
        acc[0] = mfma32(a, __builtin_bit_cast(bf16x8, rb[slot][0]), acc[0]);
        acc[1] = mfma32(a, __builtin_bit_cast(bf16x8, rb[slot][1]), acc[1]);
      });
      // lane holds X[n = 32 wave + 8 g + 4 half + e][t = t0 + 32 tb + l32], r = 4 g + e,
      // rounded to bf16 as a materialised key or value
      if constexpr (VALUES) {
#pragma unroll
        for (int j = 0; j < MAX_SQ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[j][r] += pj[j][0] * round_bf16(acc[0][r]) + pj[j][1] * round_bf16(acc[1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < MAX_SQ; ++j) {
          if (j >= s_q) break;
          float ps[2] = {0.f, 0.f};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 qv = *(const f32x4*)&qsh[j][32 * wave + 8 * g + 4 * half];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int e = 0; e < 4; ++e) ps[tb] += qv[e] * round_bf16(acc[tb][4 * g + e]);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            float x0, x1;
            halves(ps[tb], x0, x1);            // the other 4 outputs of each group of 8
            if (half == 0) red[wave][j][32 * tb + l32] = x0 + x1;
          }
        }
        barrier_lds();
        // thread (j, t): the four waves' sums plus the rope part, masked, in log2 units
        if (tid < s_q * XT) {
          const int j = tid >> 6, t = tid & 63;
          float sv = (red[0][j][t] + red[1][j][t]) + (red[2][j][t] + red[3][j][t]);
          // the rope key of row t (inline-asm reads: a plain read of the tile
          // buffer would make the compiler wait for the next tile's loads)
          i16x8 kr[D_ROPE / 8];
          static_for<0, D_ROPE / 8>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            lds_read_b128<0>(kr[c], tb_a + xoff(t, D_C + 8 * c));
          });
          wait_lgkm<0>(kr[0], kr[1], kr[2], kr[3], kr[4], kr[5], kr[6], kr[7]);
#pragma unroll
          for (int c = 0; c < D_ROPE / 8; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) sv += qsh[j][D_NOPE + 8 * c + e] * bf16_bits_to_float((uint16_t)kr[c][e]);
          const int visible = p.causal ? (T - s_q + j + 1) : T;
          if (t0 + t < T)
            p.scores[srow0 + (int64_t)j * H * p.T_cap + t0 + t] = (t0 + t < visible) ? sv * p.scale_log2 : -INFINITY;
        }
      }
      acc[0] = f32x16{};
      acc[1] = f32x16{};
    }
    if constexpr (VALUES) {
      // sum over the 32 rows a lane group holds (lanes of one half), then
      // lanes 0 and 32 of each wave write their 16 outputs
#pragma unroll
      for (int j = 0; j < MAX_SQ; ++j) {
        if (j >= s_q) break;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = oacc[j][r];
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off, 64);
          oacc[j][r] = v;
        }
        if (l32 == 0) {
          const float l = p.lsum[((int64_t)b * s_q + j) * H + h];
          const float inv = l > 0.f ? 1.0f / l : 0.f;
          uint16_t* o = p.out + (((int64_t)b * s_q + j) * H + h) * D_V + 32 * wave + 4 * half;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v4 = {oacc[j][4 * g] * inv, oacc[j][4 * g + 1] * inv, oacc[j][4 * g + 2] * inv,
                              oacc[j][4 * g + 3] * inv};
            *(uint64_t*)(o + 8 * g) = pack_bf16x4(v4);
          }
        }
      }
    }
  }
}

// Pass 2: per query row (b, j, h), over its T visible-or-masked scores:
// the maximum, exp2(s - max) in place (0 for masked entries), and the sum.
__global__ __launch_bounds__(256) void naive_softmax_kernel(NaiveParams p) {
  __shared__ float wred[4];
  const int row = blockIdx.x;                      // (b * s_q + j) * H + h
  const int b = row / (p.s_q * p.H);
  const int T = min(p.seqlens[b], p.T_cap);
  float* s = p.scores + (int64_t)row * p.T_cap;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_reduce = [&](float v, bool is_max) -> float {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float u = __shfl_xor(v, off, 64);
      v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if (lane == 0) wred[wave] = v;
    __syncthreads();
    return is_max ? fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3])) : (wred[0] + wred[1]) + (wred[2] + wred[3]);
  };
  float mx = -INFINITY;
  for (int t = tid; t < T; t += 256) mx = fmaxf(mx, s[t]);
  mx = block_reduce(mx, true);
  float sum = 0.f;
  for (int t = tid; t < T; t += 256) {
    const float v = s[t];
    const float e = (v == -INFINITY || mx == -INFINITY) ? 0.f : exp2f(v - mx);
    s[t] = e;
    sum += e;
  }
  sum = block_reduce(sum, false);
  if (tid == 0) p.lsum[row] = sum;
}

}  // namespace

hipError_t launch_transpose_wuv(const uint16_t* w_uv, uint16_t* w_uvt, int H, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_wuv_kernel, dim3(D_C / 64, D_V / 64, H), dim3(256), 0, stream, w_uv, w_uvt);
  return hipGetLastError();
}

hipError_t launch_naive(const NaiveParams& p, hipStream_t stream) {
  hipError_t e = launch_transpose_wuv(p.w_uv, p.w_uvt, p.H, stream);
  if (e != hipSuccess) return e;
  // enough (head, part) work-groups to cover the compute units once
  const int n_parts = std::max(1, std::min(p.B, (256 + p.H - 1) / p.H));
  const int items = p.H * n_parts;
  const int per_xcd = (items + 7) / 8;
  const dim3 grid(8 * per_xcd);
  if (p.fp8)
    hipLaunchKernelGGL((naive_pass_kernel<true, false>), grid, dim3(256), 0, stream, p, n_parts, per_xcd);
  else
    hipLaunchKernelGGL((naive_pass_kernel<false, false>), grid, dim3(256), 0, stream, p, n_parts, per_xcd);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(naive_softmax_kernel, dim3(p.B * p.s_q * p.H), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.fp8)
    hipLaunchKernelGGL((naive_pass_kernel<true, true>), grid, dim3(256), 0, stream, p, n_parts, per_xcd);
  else
    hipLaunchKernelGGL((naive_pass_kernel<false, true>), grid, dim3(256), 0, stream, p, n_parts, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
