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
  __shared__ __attribute__((aligned(16))) uint16_t ot[32][AQ_COLS + 8];        // output block, padded
  const int h = blockIdx.x, cblk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int nblocks = (N + 31) / 32;

  // query fragments of a 32-row block (8 k-steps of 16), loaded ahead of use
  auto load_a = [&](int nb, i16x8 (&a)[D_NOPE / 16]) {
    const int n = nb * 32 + l32;
    const bool ok = n < N;
    const uint16_t* qrow = q + ((int64_t)(ok ? n : 0) * H + h) * D_QK + half * 8;
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 16; ++ks) {
      a[ks] = *(const i16x8*)(qrow + ks * 16);
      if (!ok) a[ks] = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  i16x8 abuf[2][D_NOPE / 16];
  load_a(0, abuf[0]);

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
  bf16x8 bw[D_NOPE / 16];
#pragma unroll
  for (int ks = 0; ks < D_NOPE / 16; ++ks) {
    const int krow = ks * 16 + 8 * half + (jj >> 2);
    bw[ks] = join_tr(ds_read_tr16(wt + aq_off(krow, bcol)), ds_read_tr16(wt + aq_off(krow + 4, bcol)));
  }
  for (int nb = 0; nb < nblocks; ++nb) {
    i16x8(&a)[D_NOPE / 16] = abuf[nb & 1];
    if (nb + 1 < nblocks) load_a(nb + 1, abuf[(nb + 1) & 1]);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 16; ++ks) acc = mfma32(__builtin_bit_cast(bf16x8, a[ks]), bw[ks], acc);
    // stage the 32 x 128 output block in LDS, then write whole 256-byte rows
    __syncthreads();   // previous block's rows have been written out
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[8 * (r >> 2) + 4 * half + (r & 3)][c0 + l32] = bf16_bits(to_bf16(acc[r]));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chunk = i * 256 + tid;          // 32 rows x 16 chunks of 16 B
      const int rr = chunk >> 4, cc = chunk & 15;
      const int nn = nb * 32 + rr;
      if (nn < N)
        *(i16x8*)(q_lat + ((int64_t)nn * H + h) * ROWW + cblk * AQ_COLS + cc * 8) = *(const i16x8*)&ot[rr][cc * 8];
    }
  }
}

// ---------------------------------------------------------------------------
// absorb_out: an fp32 latent output is fed as hi + lo bf16 terms.
// ---------------------------------------------------------------------------
constexpr int AO_COLS = 64;
constexpr int AO_CHUNKS = AO_COLS * 2 / 16;   // 8 chunks per LDS row

__device__ __forceinline__ int ao_off(int k, int c) {
  return (k * AO_CHUNKS + ((c >> 3) ^ chunk_swz(k))) * 16 + (c & 7) * 2;
}

// grid (H, 2 column blocks of 64), 4 waves: wave w computes columns
// 32 (w & 1) of the block for row blocks nb = w >> 1, w >> 1 + 2, ...
template <bool IN_BF16>
__global__ __launch_bounds__(256) void absorb_out_kernel(const void* __restrict__ o_lat,
                                                         const uint16_t* __restrict__ w_uv,
                                                         uint16_t* __restrict__ out, int N, int H) {
  __shared__ __attribute__((aligned(1024))) char wt[D_C * AO_COLS * 2];   // 64 KB
  __shared__ __attribute__((aligned(16))) uint16_t ot[2][32][AO_COLS + 8];   // output blocks, padded
  const int h = blockIdx.x, vblk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int nblocks = (N + 31) / 32;
  constexpr int KS = D_C / 16;     // 32 k-steps
  constexpr int AHEAD = 8;         // latent-output fragments in flight

  {
    const uint16_t* src0 = w_uv + (int64_t)h * D_C * D_V + vblk * AO_COLS;
    char* dst = wt + wave * 64 * 16;
#pragma unroll 8
    for (int i = 0; i < D_C * AO_CHUNKS / 256; ++i) {
      const int slot = i * 256 + wave * 64 + lane;
      const int k = slot / AO_CHUNKS;
      const int cc = (slot % AO_CHUNKS) ^ chunk_swz(k);
      __builtin_amdgcn_global_load_lds((const void*)(src0 + (int64_t)k * D_V + cc * 8),
                                       (lds_void_t*)(dst + i * 256 * 16), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int v0 = (wave & 1) * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = v0 + grp * 16 + 4 * (jj & 3);
  // both row-block streams run the same number of iterations so that every
  // wave reaches the staging barriers; past the last block a stream computes
  // zeros (its rows are >= N) and stores nothing
  for (int it = 0; it < (nblocks + 1) / 2; ++it) {
    const int nb = 2 * it + (wave >> 1);
    const int n = nb * 32 + l32;
    const bool n_ok = n < N;
    const int64_t orow = ((int64_t)(n_ok ? n : 0) * H + h) * D_C + half * 8;
    // a ring of AHEAD fragments of this lane's latent-output row
    f32x4 ring[AHEAD][2];
    i16x8 ringb[AHEAD];
    auto load = [&](int ks, int slot) {
      if (IN_BF16) {
        ringb[slot] = *(const i16x8*)((const uint16_t*)o_lat + orow + ks * 16);
      } else {
        const float* src = (const float*)o_lat + orow + ks * 16;
        ring[slot][0] = *(const f32x4*)src;
        ring[slot][1] = *(const f32x4*)(src + 4);
      }
    };
#pragma unroll
    for (int ks = 0; ks < AHEAD; ++ks) load(ks, ks);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = ks % AHEAD;
      bf16x8 ahi, alo;
      if (IN_BF16) {
        i16x8 v = ringb[slot];
        if (!n_ok) v = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
        ahi = __builtin_bit_cast(bf16x8, v);
      } else {
        f32x4 x0 = ring[slot][0], x1 = ring[slot][1];
        if (!n_ok) { x0 = f32x4{0.f, 0.f, 0.f, 0.f}; x1 = x0; }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ahi[e] = to_bf16(x0[e]);
          ahi[e + 4] = to_bf16(x1[e]);
          alo[e] = to_bf16(x0[e] - (float)ahi[e]);
          alo[e + 4] = to_bf16(x1[e] - (float)ahi[e + 4]);
        }
      }
      if (ks + AHEAD < KS) load(ks + AHEAD, slot);
      const int krow = ks * 16 + 8 * half + (jj >> 2);
      const bf16x8 bw = join_tr(ds_read_tr16(wt + ao_off(krow, bcol)), ds_read_tr16(wt + ao_off(krow + 4, bcol)));
      acc = mfma32(ahi, bw, acc);
      if (!IN_BF16) acc = mfma32(alo, bw, acc);
    }
    // stage the 32 x 64 output block in LDS (the two waves sharing this row
    // block fill one half each), then write whole 128-byte rows
    uint16_t(&o2)[32][AO_COLS + 8] = ot[wave >> 1];
#pragma unroll
    for (int r = 0; r < 16; ++r) o2[8 * (r >> 2) + 4 * half + (r & 3)][v0 + l32] = bf16_bits(to_bf16(acc[r]));
    __syncthreads();
    {
      const int t128 = (wave & 1) * 64 + lane;   // 128 threads of this row-block stream
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int chunk = i * 128 + t128;       // 32 rows x 8 chunks of 16 B
        const int rr = chunk >> 3, cc = chunk & 7;
        const int nn = nb * 32 + rr;
        if (nn < N)
          *(i16x8*)(out + ((int64_t)nn * H + h) * D_V + vblk * AO_COLS + cc * 8) = *(const i16x8*)&o2[rr][cc * 8];
      }
    }
    __syncthreads();
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
    hipLaunchKernelGGL(absorb_out_kernel<true>, dim3(H, D_V / AO_COLS), dim3(256), 0, stream, o_lat, w_uv, out, N, H);
  else
    hipLaunchKernelGGL(absorb_out_kernel<false>, dim3(H, D_V / AO_COLS), dim3(256), 0, stream, o_lat, w_uv, out, N, H);
  return hipGetLastError();
}

}  // namespace mla
