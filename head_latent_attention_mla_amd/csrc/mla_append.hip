// Latent append: the step that makes the cached row of each new token
// ("Why MLA and MTP Fight Each Other", section 3: the hidden state is
// compressed through W_DKV into the latent that the cache holds; Appendix A
// and "MLA, dim by dim", "Why RoPE Gets in the Way": a 64-wide rope key,
// rotated by the token's position and shared by all heads, is stored beside
// it).
//
// Two kernels:
//   append_project_kernel  split-K MFMA product rows^T = W_DKR x^T: one
//       work-group per (32 output columns, K range, 64 tokens); its four waves
//       take interleaved 64-wide k-chunks and are summed through LDS into an
//       fp32 partial [split][token][576].  The weight is [576, d_model] with
//       d_model contiguous, so both MFMA operands come straight from memory
//       (no transpose).  Within a chunk the k order is permuted the same way
//       for both operands: lane half h of row i holds k = 32 h .. 32 h + 31,
//       and MFMA j of the chunk takes its 8 values 8 j .. 8 j + 7, so each
//       lane reads 64 contiguous bytes and the two halves a full 128-byte
//       line per row.
//   append_finalize_kernel one wave per token: sums the partials, turns the
//       rope pairs by the position's angles (computed in fp64), then stores
//       the row as bf16 (nearest even) or as E4M3 codes with one fp32 scale
//       (amax / 448) at the token's slot of the contiguous or paged cache.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int COLS = 32;        // output columns per work-group
constexpr int TOKS = 64;        // tokens per work-group (two 32-token MFMA blocks)
constexpr int WAVE_CHUNKS = 2;  // most 64-wide k-chunks one wave takes (a split has <= 8)

__device__ __forceinline__ i16x8 load16(const uint16_t* p) { return *(const i16x8*)p; }

__global__ __launch_bounds__(256) void append_project_kernel(AppendParams p) {
  const int cb = blockIdx.x;
  const int ks = blockIdx.y;
  const int tok0 = blockIdx.z * TOKS;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, half = lane >> 5;
  const int n_chunks = p.d / 64;
  const int c0 = ks * p.chunks_per_split;
  const int c1 = min(n_chunks, c0 + p.chunks_per_split);

  const int col = cb * COLS + l32;                       // < 576: the grid has 576 / 32 column blocks
  const uint16_t* wrow = p.w + (int64_t)col * p.d + half * 32;
  // rows past the last token read the last token again (their results are
  // never stored), so every load is unconditional and in bounds
  const int t0 = min(tok0 + l32, p.N - 1), t1 = min(tok0 + 32 + l32, p.N - 1);
  const uint16_t* x0 = p.x + (int64_t)t0 * p.d + half * 32;
  const uint16_t* x1 = p.x + (int64_t)t1 * p.d + half * 32;

  // every load of the wave is issued before the first product: the whole
  // weight is only a few MB, so the step is bound by memory latency unless
  // all of it is in flight at once.  Chunks past the split's end reload its
  // last chunk and are skipped (a wave-uniform test).
  const int n_mine = c1 - c0 > wave ? (c1 - c0 - wave + 3) / 4 : 0;
  i16x8 a[WAVE_CHUNKS][4], b0[WAVE_CHUNKS][4], b1[WAVE_CHUNKS][4];
#pragma unroll
  for (int u = 0; u < WAVE_CHUNKS; ++u) {
    const int ch = min(c0 + wave + 4 * u, c1 - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[u][j] = load16(wrow + ch * 64 + 8 * j);
      b0[u][j] = load16(x0 + ch * 64 + 8 * j);
      b1[u][j] = load16(x1 + ch * 64 + 8 * j);
    }
  }
  // pin the loads here (otherwise the compiler sinks the first chunk's loads
  // into the test below and serialises them with the products)
#pragma unroll
  for (int u = 0; u < WAVE_CHUNKS; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      touch_reg(a[u][j]);
      touch_reg(b0[u][j]);
      touch_reg(b1[u][j]);
    }
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int u = 0; u < WAVE_CHUNKS; ++u) {
    if (u < n_mine) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a[u][j]);
        acc0 = mfma32(av, __builtin_bit_cast(bf16x8, b0[u][j]), acc0);
        acc1 = mfma32(av, __builtin_bit_cast(bf16x8, b1[u][j]), acc1);
      }
    }
  }

  // sum the four waves' accumulators; each wave then writes a quarter
  __shared__ f32x16 red[4][2][64];
  red[wave][0][lane] = acc0;
  red[wave][1][lane] = acc1;
  __syncthreads();
  // wave w writes token block (w >> 1), register quarter group (w & 1): the
  // accumulator element r of lane l is D[8 (r / 4) + 4 half + r % 4][l32] with
  // D[i][j] = partial row (token j) at column cb * 32 + i
  const int blk = wave >> 1;
  const int tok = tok0 + 32 * blk + l32;
  if (tok < p.N) {
    float* dst = p.part + ((int64_t)ks * p.N + tok) * ROWW + cb * COLS + 4 * half;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int q = 2 * (wave & 1) + q2;        // register group: elements 4q .. 4q + 3
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v += *(const f32x4*)((const float*)&red[w][blk][lane] + 4 * q);
      }
      *(f32x4*)(dst + 8 * q) = v;
    }
  }
}

// E4M3 code of a non-negative value (round to nearest even; callers clamp to 448)
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__global__ __launch_bounds__(256) void append_finalize_kernel(AppendParams p) {
  const int n = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = p.seq_id[n];
  const int ps = p.pos[n];
  if (b < 0 || b >= p.B || ps < 0) return;                   // uniform: one token per work-group
  int64_t row;
  if (p.block_table != nullptr) {
    if (ps >= p.max_blocks * 64) return;
    const int blk = p.block_table[(int64_t)b * p.max_blocks + (ps >> 6)];
    if (blk < 0) return;
    row = (int64_t)blk * 64 + (ps & 63);
  } else {
    if (ps >= p.T_stride) return;
    row = (int64_t)b * p.T_stride + ps;
  }

  // the row: latent columns 8 lane .. 8 lane + 7 and rope column lane.  Wave
  // w sums splits w, w + 4, ... (in order, four loads of each kind in
  // flight); the four wave sums are added in wave order through LDS.
  f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
  float vr = 0.f;
  const float* base = p.part + (int64_t)n * ROWW;
  const int64_t split_stride = (int64_t)p.N * ROWW;
  for (int k0 = wave; k0 < p.ks_count; k0 += 16) {
    f32x4 l0[4], l1[4];
    float lr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* src = base + min(k0 + 4 * u, p.ks_count - 1) * split_stride;   // in bounds; extra loads unused
      l0[u] = *(const f32x4*)(src + 8 * lane);
      l1[u] = *(const f32x4*)(src + 8 * lane + 4);
      lr[u] = src[D_C + lane];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (k0 + 4 * u < p.ks_count) {      // uniform
        v0 += l0[u];
        v1 += l1[u];
        vr += lr[u];
      }
    }
  }
  __shared__ float red[4][64][9];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    red[wave][lane][e] = v0[e];
    red[wave][lane][4 + e] = v1[e];
  }
  red[wave][lane][8] = vr;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v0[e] = ((red[0][lane][e] + red[1][lane][e]) + red[2][lane][e]) + red[3][lane][e];
    v1[e] = ((red[0][lane][4 + e] + red[1][lane][4 + e]) + red[2][lane][4 + e]) + red[3][lane][4 + e];
  }
  vr = ((red[0][lane][8] + red[1][lane][8]) + red[2][lane][8]) + red[3][lane][8];
  // rope pair (2i, 2i + 1), i = lane / 2: angle = pos * base^(-2i / 64)
  {
    const int i = lane >> 1;
    const double theta = exp2(-(double)(2 * i) / 64.0 * p.log2_base);
    double sn, cs;
    sincos((double)ps * theta, &sn, &cs);
    const double mine = vr;
    const double other = __shfl_xor(vr, 1, 64);
    vr = (lane & 1) == 0 ? (float)(mine * cs - other * sn) : (float)(other * sn + mine * cs);
  }
  const float vals[9] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3], vr};

  if (!p.fp8) {
    uint16_t* out = (uint16_t*)p.rows + row * ROWW;
    i16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (short)bf16_bits(to_bf16(vals[e]));
    *(i16x8*)(out + 8 * lane) = o;
    out[D_C + lane] = bf16_bits(to_bf16(vr));
    return;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 9; ++e) amax = fmaxf(amax, fabsf(vals[e]));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  // magnitudes are converted, the sign bit is set from the value (a negative
  // value that rounds to zero keeps its sign)
  uint32_t code[9];
#pragma unroll
  for (int e = 0; e < 9; e += 2) {
    const float qa = fminf(fabsf(__fdiv_rn(vals[e], scale)), 448.0f);
    const float qb = e + 1 < 9 ? fminf(fabsf(__fdiv_rn(vals[e + 1], scale)), 448.0f) : 0.f;
    const uint32_t pr = e4m3_pair(qa, qb);
    code[e] = (pr & 0xFFu) | (__builtin_signbitf(vals[e]) ? 0x80u : 0u);
    if (e + 1 < 9) code[e + 1] = (pr >> 8) | (__builtin_signbitf(vals[e + 1]) ? 0x80u : 0u);
  }
  uint8_t* out = (uint8_t*)p.rows + row * ROWW;
  const uint32_t lo = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
  const uint32_t hi = code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24);
  *(uint2*)(out + 8 * lane) = make_uint2(lo, hi);
  out[D_C + lane] = (uint8_t)code[8];
  if (lane == 0) p.row_scale[row] = scale;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  const dim3 grid(ROWW / COLS, p.ks_count, (p.N + TOKS - 1) / TOKS);
  hipLaunchKernelGGL(append_project_kernel, grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_finalize_kernel, dim3(p.N), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
