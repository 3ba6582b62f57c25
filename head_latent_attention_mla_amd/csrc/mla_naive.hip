// Naive (expand) MLA decode, kept as an ablation of the absorbed path.
//
// Every visible cached row is re-expanded per head on every call: the key
// K[t] = [W_UK[h] c_t[0:512] | c_t[512:576]] and the value V[t] =
// c_t[0:512]^T W_UV[h], then ordinary softmax attention with the 192-wide
// query ("The MLA decode speedup hiding in your model card", "The naive form,
// written out"; "Why MLA and MTP Fight Each Other", section 5.1: expanding
// bills the up-projection to every cached token, about 120x the absorbed
// arithmetic at these widths).
//
// One work-group per (head, sequence), 4 waves.  Per 128-row tile each wave
// expands 32 rows on MFMA (A = cached rows straight from global memory,
// B = W_UK[h] rows and W_UV[h] transposed, both contiguous in the contracted
// dimension), parks K and V in LDS, and the work-group then scores, runs an
// online softmax and accumulates the value sum on the VALU.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int NT = 128;                    // cached rows per tile
constexpr int KV_STRIDE = D_NOPE + 8;      // padded LDS row (bf16) of K and V tiles
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

__global__ __launch_bounds__(256) void naive_decode_kernel(NaiveParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[NT][KV_STRIDE];   // expanded K_nope tile
  __shared__ __attribute__((aligned(16))) uint16_t vs[NT][KV_STRIDE];   // expanded V tile
  __shared__ float qs[MAX_SQ][D_QK];                                     // query rows
  __shared__ float sc[MAX_SQ][NT];                                       // scores -> probabilities
  __shared__ float alpha_s[MAX_SQ];

  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int H = p.H, s_q = p.s_q;
  const int T = p.seqlens[b];
  const uint16_t* w_uk = p.w_uk + (int64_t)h * D_NOPE * D_C;
  const uint16_t* w_uvt = p.w_uvt + (int64_t)h * D_V * D_C;

  for (int i = tid; i < s_q * D_QK; i += 256) {
    const int j = i / D_QK, k = i % D_QK;
    qs[j][k] = bf16_bits_to_float(p.q[(((int64_t)b * s_q + j) * H + h) * D_QK + k]);
  }

  // cached row t of sequence b as an element pointer (contiguous or paged)
  auto row_ptr = [&](int t) -> int64_t {
    if (p.block_table != nullptr)
      return ((int64_t)p.block_table[(int64_t)b * p.max_blocks + (t >> 6)] * 64 + (t & 63)) * ROWW;
    return ((int64_t)b * p.T_stride + t) * ROWW;
  };
  // cached element as fp32 (bf16, or e4m3 code times the row scale)
  auto elem = [&](int64_t base, int t, int c) -> float {
    if (p.fp8) {
      const uint8_t code = ((const uint8_t*)p.rows)[base + c];
      const float sc_t = p.row_scale[base / ROWW];
      return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0] * sc_t;
    }
    return bf16_bits_to_float(((const uint16_t*)p.rows)[base + c]);
  };

  // online softmax state of query j lives with thread j (j < s_q)
  float m_run = -INFINITY, l_run = 0.f;
  // value accumulator: thread -> (query j = tid / 64, value columns 2 (tid % 64) ..)
  const int oj = tid >> 6, ov = (tid & 63) * 2;
  float o0 = 0.f, o1 = 0.f;

  for (int t0 = 0; t0 < T; t0 += NT) {
    __syncthreads();   // the previous tile's K, V and probabilities are consumed
    // ---- expand 32 rows per wave: K_nope = C W_UK^T, V = C W_UV
    {
      const int t = t0 + wave * 32 + l32;
      const bool t_ok = t < T;
      const int64_t base = row_ptr(t_ok ? t : T - 1);
      f32x16 kacc[4], vacc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { kacc[i] = f32x16{}; vacc[i] = f32x16{}; }
      for (int kk = 0; kk < D_C / 16; ++kk) {
        const int c = kk * 16 + half * 8;
        bf16x8 a;
        if (p.fp8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = to_bf16(t_ok ? elem(base, t, c + e) : 0.f);
        } else {
          i16x8 v = *(const i16x8*)((const uint16_t*)p.rows + base + c);
          if (!t_ok) v = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
          a = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = nb * 32 + l32;
          const bf16x8 bk = __builtin_bit_cast(bf16x8, *(const i16x8*)(w_uk + (int64_t)n * D_C + c));
          const bf16x8 bv = __builtin_bit_cast(bf16x8, *(const i16x8*)(w_uvt + (int64_t)n * D_C + c));
          kacc[nb] = mfma32(a, bk, kacc[nb]);
          vacc[nb] = mfma32(a, bv, vacc[nb]);
        }
      }
      // accumulator layout: column n = 32 nb + l32, rows 8 (r/4) + 4 half + r%4
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = wave * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          ks[tr][nb * 32 + l32] = bf16_bits(to_bf16(kacc[nb][r]));
          vs[tr][nb * 32 + l32] = bf16_bits(to_bf16(vacc[nb][r]));
        }
    }
    __syncthreads();
    // ---- scores: thread -> row tr = tid / 2, part = tid % 2 (nope | rope)
    {
      const int tr = tid >> 1, part = tid & 1;
      const int t = t0 + tr;
      float acc_j[MAX_SQ] = {0.f, 0.f, 0.f, 0.f};
      if (t < T) {
        if (part == 0) {
          for (int k = 0; k < D_NOPE; ++k) {
            const float kv = bf16_bits_to_float(ks[tr][k]);
#pragma unroll
            for (int j = 0; j < MAX_SQ; ++j)
              if (j < s_q) acc_j[j] += qs[j][k] * kv;
          }
        } else {
          const int64_t base = row_ptr(t);
          for (int r = 0; r < D_ROPE; ++r) {
            const float kr = elem(base, t, D_C + r);
#pragma unroll
            for (int j = 0; j < MAX_SQ; ++j)
              if (j < s_q) acc_j[j] += qs[j][D_NOPE + r] * kr;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < MAX_SQ; ++j) acc_j[j] += __shfl_xor(acc_j[j], 1);
      if (part == 0) {
#pragma unroll
        for (int j = 0; j < MAX_SQ; ++j) {
          if (j >= s_q) break;
          const int visible = p.causal ? (T - s_q + j + 1) : T;
          sc[j][tr] = (t < visible) ? acc_j[j] * p.scale_log2 : -INFINITY;
        }
      }
    }
    __syncthreads();
    // ---- online softmax: thread j < s_q owns query j
    if (tid < s_q) {
      const int j = tid;
      float mx = -INFINITY;
      for (int i = 0; i < NT; ++i) mx = fmaxf(mx, sc[j][i]);
      const float m_new = fmaxf(m_run, mx);
      const float a = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      float ls = 0.f;
      for (int i = 0; i < NT; ++i) {
        const float pr = exp2f(sc[j][i] - base);
        sc[j][i] = pr;
        ls += pr;
      }
      l_run = l_run * a + ls;
      m_run = m_new;
      alpha_s[j] = a;
    }
    __syncthreads();
    // ---- value sum
    if (oj < s_q) {
      const float a = alpha_s[oj];
      o0 *= a;
      o1 *= a;
      for (int i = 0; i < NT; ++i) {
        const float pr = sc[oj][i];
        o0 += pr * bf16_bits_to_float(vs[i][ov]);
        o1 += pr * bf16_bits_to_float(vs[i][ov + 1]);
      }
    }
  }
  __syncthreads();
  if (tid < s_q) alpha_s[tid] = l_run > 0.f ? 1.0f / l_run : 0.f;
  __syncthreads();
  if (oj < s_q) {
    const float inv = alpha_s[oj];
    uint16_t* o = p.out + (((int64_t)b * s_q + oj) * H + h) * D_V + ov;
    o[0] = bf16_bits(to_bf16(o0 * inv));
    o[1] = bf16_bits(to_bf16(o1 * inv));
  }
}

}  // namespace

hipError_t launch_transpose_wuv(const uint16_t* w_uv, uint16_t* w_uvt, int H, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_wuv_kernel, dim3(D_C / 64, D_V / 64, H), dim3(256), 0, stream, w_uv, w_uvt);
  return hipGetLastError();
}

hipError_t launch_naive(const NaiveParams& p, hipStream_t stream) {
  hipError_t e = launch_transpose_wuv(p.w_uv, p.w_uvt, p.H, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(naive_decode_kernel, dim3(p.H, p.B), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
