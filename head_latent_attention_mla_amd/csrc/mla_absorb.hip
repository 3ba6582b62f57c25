// The two per-head absorption GEMMs of MLA decode on gfx950.
//
//   absorb_q:  q_lat[n,h,0:512] = q[n,h,0:128] W_UK[h]   (+ q_rope copied to 512:576)
//   absorb_out: out[n,h,:]      = o_lat[n,h,:] W_UV[h]
//
// ("MLA, dim by dim", "MLA Decode": W_UK^T is absorbed into the current query
// and W_UV is applied once to the latent output; "Why MLA and MTP Fight Each
// Other", sections 3.1-3.2.)  Both are small per-head products whose cost is
// reading the weights (16.8 MB each at H = 128), so each work-group stages one
// weight tile in LDS once and runs all query tokens through it on MFMA.  The
// weights are stored with the contracted dimension outermost, so the MFMA B
// fragments are taken with gfx950 transpose reads from LDS.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

// ---------------------------------------------------------------------------
// absorb_q: grid (H, 4 column blocks of 128), 4 waves, wave w -> 32 columns.
// ---------------------------------------------------------------------------
constexpr int AQ_COLS = 128;
constexpr int AQ_CHUNKS = AQ_COLS * 2 / 16;   // 16 chunks per LDS row

__device__ __forceinline__ int aq_off(int k, int c) {
  return (k * AQ_CHUNKS + ((c >> 3) ^ chunk_swz(k))) * 16 + (c & 7) * 2;
}

__global__ __launch_bounds__(256) void absorb_q_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ w_uk,
                                                       uint16_t* __restrict__ q_lat, int N, int H) {
  __shared__ __attribute__((aligned(1024))) char wt[D_NOPE * AQ_COLS * 2];   // 32 KB
  const int h = blockIdx.x, cblk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  // stage W_UK[h][0:128][cblk*128 : +128]
  {
    const uint16_t* src0 = w_uk + (int64_t)h * D_NOPE * D_C + cblk * AQ_COLS;
    char* dst = wt + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < D_NOPE * AQ_CHUNKS / 256; ++i) {
      const int slot = i * 256 + wave * 64 + lane;
      const int k = slot / AQ_CHUNKS;
      const int cc = (slot % AQ_CHUNKS) ^ chunk_swz(k);
      __builtin_amdgcn_global_load_lds((const void*)(src0 + (int64_t)k * D_C + cc * 8),
                                       (lds_void_t*)(dst + i * 256 * 16), 16, 0, 0);
    }
  }
  // rope part of the query rows is carried over unchanged
  if (cblk == 0) {
    for (int i = tid; i < N * (D_ROPE / 8); i += 256) {
      const int n = i / (D_ROPE / 8), c8 = i % (D_ROPE / 8);
      const int64_t qr = (int64_t)n * H + h;
      *(i16x8*)(q_lat + qr * ROWW + D_C + c8 * 8) = *(const i16x8*)(q + qr * D_QK + D_NOPE + c8 * 8);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int c0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = c0 + grp * 16 + 4 * (jj & 3);
  for (int nb = 0; nb * 32 < N; ++nb) {
    const int n = nb * 32 + l32;
    const bool n_ok = n < N;
    const uint16_t* qrow = q + ((int64_t)(n_ok ? n : 0) * H + h) * D_QK + half * 8;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 16; ++ks) {
      i16x8 a = *(const i16x8*)(qrow + ks * 16);
      if (!n_ok) a = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const int krow = ks * 16 + 8 * half + (jj >> 2);
      const i16x4 lo = ds_read_tr16(wt + aq_off(krow, bcol));
      const i16x4 hi = ds_read_tr16(wt + aq_off(krow + 4, bcol));
      acc = mfma32(__builtin_bit_cast(bf16x8, a), join_tr(lo, hi), acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int nn = nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (nn < N)
        q_lat[((int64_t)nn * H + h) * ROWW + cblk * AQ_COLS + c0 + l32] = bf16_bits(to_bf16(acc[r]));
    }
  }
}

// ---------------------------------------------------------------------------
// absorb_out: grid (H, 2 column blocks of 64), 2 waves, wave w -> 32 columns.
// An fp32 latent output is fed as hi + lo bf16 terms.
// ---------------------------------------------------------------------------
constexpr int AO_COLS = 64;
constexpr int AO_CHUNKS = AO_COLS * 2 / 16;   // 8 chunks per LDS row

__device__ __forceinline__ int ao_off(int k, int c) {
  return (k * AO_CHUNKS + ((c >> 3) ^ chunk_swz(k))) * 16 + (c & 7) * 2;
}

template <bool IN_BF16>
__global__ __launch_bounds__(128) void absorb_out_kernel(const void* __restrict__ o_lat,
                                                         const uint16_t* __restrict__ w_uv,
                                                         uint16_t* __restrict__ out, int N, int H) {
  __shared__ __attribute__((aligned(1024))) char wt[D_C * AO_COLS * 2];   // 64 KB
  const int h = blockIdx.x, vblk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  {
    const uint16_t* src0 = w_uv + (int64_t)h * D_C * D_V + vblk * AO_COLS;
    char* dst = wt + wave * 64 * 16;
#pragma unroll 8
    for (int i = 0; i < D_C * AO_CHUNKS / 128; ++i) {
      const int slot = i * 128 + wave * 64 + lane;
      const int k = slot / AO_CHUNKS;
      const int cc = (slot % AO_CHUNKS) ^ chunk_swz(k);
      __builtin_amdgcn_global_load_lds((const void*)(src0 + (int64_t)k * D_V + cc * 8),
                                       (lds_void_t*)(dst + i * 128 * 16), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int v0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = v0 + grp * 16 + 4 * (jj & 3);
  for (int nb = 0; nb * 32 < N; ++nb) {
    const int n = nb * 32 + l32;
    const bool n_ok = n < N;
    const int64_t orow = ((int64_t)(n_ok ? n : 0) * H + h) * D_C + half * 8;
    f32x16 acc = f32x16{};
    for (int ks = 0; ks < D_C / 16; ++ks) {
      const int krow = ks * 16 + 8 * half + (jj >> 2);
      const i16x4 blo = ds_read_tr16(wt + ao_off(krow, bcol));
      const i16x4 bhi = ds_read_tr16(wt + ao_off(krow + 4, bcol));
      const bf16x8 bw = join_tr(blo, bhi);
      if (IN_BF16) {
        i16x8 a = *(const i16x8*)((const uint16_t*)o_lat + orow + ks * 16);
        if (!n_ok) a = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
        acc = mfma32(__builtin_bit_cast(bf16x8, a), bw, acc);
      } else {
        const float* src = (const float*)o_lat + orow + ks * 16;
        f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
        if (!n_ok) { x0 = f32x4{0.f, 0.f, 0.f, 0.f}; x1 = x0; }
        bf16x8 ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ahi[e] = to_bf16(x0[e]);
          ahi[e + 4] = to_bf16(x1[e]);
          alo[e] = to_bf16(x0[e] - (float)ahi[e]);
          alo[e + 4] = to_bf16(x1[e] - (float)ahi[e + 4]);
        }
        acc = mfma32(ahi, bw, acc);
        acc = mfma32(alo, bw, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int nn = nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (nn < N)
        out[((int64_t)nn * H + h) * D_V + vblk * AO_COLS + v0 + l32] = bf16_bits(to_bf16(acc[r]));
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t* q, const uint16_t* w_uk, uint16_t* q_lat, int N, int H,
                           hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H, D_C / AQ_COLS), dim3(256), 0, stream, q, w_uk, q_lat, N, H);
  return hipGetLastError();
}

hipError_t launch_absorb_out(const void* o_lat, int o_bf16, const uint16_t* w_uv, uint16_t* out,
                             int N, int H, hipStream_t stream) {
  if (o_bf16)
    hipLaunchKernelGGL(absorb_out_kernel<true>, dim3(H, D_V / AO_COLS), dim3(128), 0, stream, o_lat, w_uv, out, N, H);
  else
    hipLaunchKernelGGL(absorb_out_kernel<false>, dim3(H, D_V / AO_COLS), dim3(128), 0, stream, o_lat, w_uv, out, N, H);
  return hipGetLastError();
}

}  // namespace mla
