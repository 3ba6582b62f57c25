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
// absorb_q: grid (H x row groups of 64 query tokens, 4 column blocks of 128),
// 4 waves, wave w -> 32 columns of both 32-row blocks.  Every global load of
// a work-group (its weight slice, its query rows and, in column block 0, the
// rope parts it carries over) is issued before the first wait, so a
// work-group costs one memory round trip; the 64 rows of a group are spread
// over the grid instead of looped over.
// ---------------------------------------------------------------------------
constexpr int AQ_COLS = 128;
constexpr int AQ_CHUNKS = AQ_COLS * 2 / 16;   // 16 chunks per LDS row
constexpr int AQ_ROWS = 64;                   // query tokens per work-group

__device__ __forceinline__ int aq_off(int k, int c) {
  return (k * AQ_CHUNKS + ((c >> 3) ^ chunk_swz(k))) * 16 + (c & 7) * 2;
}

__global__ __launch_bounds__(256) void absorb_q_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ w_uk,
                                                       uint16_t* __restrict__ q_lat, int N, int H) {
  __shared__ __attribute__((aligned(1024))) char wt[D_NOPE * AQ_COLS * 2];      // 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t ot[AQ_ROWS][AQ_COLS + 8];     // output block, padded
  const int h = blockIdx.x % H, n0 = (blockIdx.x / H) * AQ_ROWS, cblk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // stage W_UK[h][0:128][cblk*128 : +128] (direct to LDS)
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
  // query fragments of both 32-row blocks (8 k-steps of 16 each); rows past
  // N re-read row n0 (always valid) and are zeroed after the wait
  i16x8 a0[D_NOPE / 16], a1[D_NOPE / 16];
  const bool ok0 = n0 + l32 < N, ok1 = n0 + 32 + l32 < N;
  {
    const uint16_t* r0 = q + ((int64_t)(ok0 ? n0 + l32 : n0) * H + h) * D_QK + half * 8;
    const uint16_t* r1 = q + ((int64_t)(ok1 ? n0 + 32 + l32 : n0) * H + h) * D_QK + half * 8;
#pragma unroll
    for (int ks = 0; ks < D_NOPE / 16; ++ks) {
      a0[ks] = *(const i16x8*)(r0 + ks * 16);
      a1[ks] = *(const i16x8*)(r1 + ks * 16);
    }
  }
  // rope parts of the group's rows (column block 0 only): 64 rows x 8 chunks
  // of 16 B, two per thread, stored after the projection
  i16x8 rope[2];
  const int rr0 = tid >> 3, rc = tid & 7;             // rows rr0 and rr0 + 32, chunk rc
  const bool rope_on = cblk == 0;
  if (rope_on) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + rr0 + 32 * i;
      rope[i] = *(const i16x8*)(q + ((int64_t)(n < N ? n : n0) * H + h) * D_QK + D_NOPE + rc * 8);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int c0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = c0 + grp * 16 + 4 * (jj & 3);
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D_NOPE / 16; ++ks) {
    const int krow = ks * 16 + 8 * half + (jj >> 2);
    const bf16x8 bw = join_tr(ds_read_tr16(wt + aq_off(krow, bcol)), ds_read_tr16(wt + aq_off(krow + 4, bcol)));
    const i16x8 z = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    acc0 = mfma32(__builtin_bit_cast(bf16x8, ok0 ? a0[ks] : z), bw, acc0);
    acc1 = mfma32(__builtin_bit_cast(bf16x8, ok1 ? a1[ks] : z), bw, acc1);
  }
  // stage the 64 x 128 output block in LDS, then write whole 256-byte rows
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * half + (r & 3);
    ot[row][c0 + l32] = bf16_bits(to_bf16(acc0[r]));
    ot[row + 32][c0 + l32] = bf16_bits(to_bf16(acc1[r]));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = i * 256 + tid;          // 64 rows x 16 chunks of 16 B
    const int rr = chunk >> 4, cc = chunk & 15;
    const int nn = n0 + rr;
    if (nn < N)
      *(i16x8*)(q_lat + ((int64_t)nn * H + h) * ROWW + cblk * AQ_COLS + cc * 8) = *(const i16x8*)&ot[rr][cc * 8];
  }
  // the rope part of the query rows is carried over unchanged
  if (rope_on) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + rr0 + 32 * i;
      if (n < N) *(i16x8*)(q_lat + ((int64_t)n * H + h) * ROWW + D_C + rc * 8) = rope[i];
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

// ---------------------------------------------------------------------------
// combine_out: the log-sum-exp merge of the split partials fused with the
// projection through W_UV, so the latent output never round-trips through
// HBM.  grid (H, ceil(N / 32)), 4 waves.  Per work-group: merge the partials
// of 32 query rows of one head (the merge arithmetic is the one of the
// stand-alone merge kernel, term for term), stage them as bf16 high + low
// MFMA operands in LDS, then stream W_UV[h] through LDS in four 128-row
// chunks; wave w computes output columns 32 w .. 32 w + 31.
// ---------------------------------------------------------------------------
constexpr int CO_ROWS = 32;
constexpr int CO_KC = 128;                        // W_UV rows per staged chunk
constexpr int CO_WBYTES = CO_KC * D_V * 2;        // 32 KB
constexpr int CO_ABYTES = CO_ROWS * D_C * 2;      // one bf16 operand plane, 32 KB

// row-major [32][512] bf16 operand plane; the 16-byte chunk index is XORed
// with the row so that the 32 rows of an MFMA fragment read hit all banks
__device__ __forceinline__ int co_aoff(int r, int k) {
  return r * (D_C * 2) + (((k >> 3) ^ (r & 15)) << 4) + (k & 7) * 2;
}

template <bool PB16>
__global__ __launch_bounds__(256) void combine_out_kernel(const void* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ seg_first,
                                                          const int32_t* __restrict__ seg_count,
                                                          int s_q, int H, int N,
                                                          const uint16_t* __restrict__ w_uv,
                                                          uint16_t* __restrict__ out, void* o_lat,
                                                          int o_bf16, float* lse_out) {
  __shared__ __attribute__((aligned(1024))) char wt[3][CO_WBYTES];   // W_UV chunks 0-2, then 3 in slot 0
  __shared__ __attribute__((aligned(1024))) char at[2][CO_ABYTES];   // [hi, lo]
  const int h = blockIdx.x, n0 = blockIdx.y * CO_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int R = s_q * H;
  const uint16_t* wsrc = w_uv + (int64_t)h * D_C * D_V;

  auto issue_w = [&](int kc) {
    char* dst = wt[kc % 3] + wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < CO_KC * AQ_CHUNKS / 256; ++i) {
      const int slot = i * 256 + wave * 64 + lane;
      const int k = slot / AQ_CHUNKS;
      const int cc = (slot % AQ_CHUNKS) ^ chunk_swz(k);
      __builtin_amdgcn_global_load_lds((const void*)(wsrc + (int64_t)(kc * CO_KC + k) * D_V + cc * 8),
                                       (lds_void_t*)(dst + i * 256 * 16), 16, 0, 0);
    }
  };

  // ---- merge: thread -> row r = tid / TPR, columns VW (tid % TPR) + VW TPR i
  // (VW = 8 bf16 or 4 fp32 partial values: 16-byte loads, so the TPR threads
  // of a row read whole 128-byte lines); fewer rows in the block get more
  // threads each (TPR = 8, 16 or 32)
  auto merge = [&](auto tprc) {
    constexpr int TPR = decltype(tprc)::value;
    constexpr int VW = PB16 ? 8 : 4;
    constexpr int NCH = D_C / VW / TPR;      // 16-byte column chunks per thread
    using Raw = typename std::conditional<PB16, u32x4, f32x4>::type;
    const int r = tid / TPR, cq = (tid % TPR) * VW;
    const int n = n0 + r;
    const bool ok = r < CO_ROWS && n < N;
    const int b = ok ? n / s_q : 0;
    const int row = ok ? (n - b * s_q) * H + h : 0;
    const int64_t sb = seg_first[b];
    const int n_split = seg_count[b];
    // splits are taken four at a time with every load of the group in flight
    // together (indices past the last split reload it and get weight 0), and
    // added in split order.  The first group's partials are loaded with the
    // log-sum-exps, before the maximum is known (it only sets their weights).
    constexpr int SG = 4;
    auto load_group = [&](int s0, float (&l)[SG], Raw (&d)[SG][NCH]) {
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const int s = max(min(s0 + u, n_split - 1), 0);
        l[u] = part_lse[(sb + s) * R + row];
        const int64_t src = ((sb + s) * R + row) * D_C + cq;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          if constexpr (PB16) d[u][i] = *(const u32x4*)((const uint16_t*)part_o + src + VW * TPR * i);
          else d[u][i] = *(const f32x4*)((const float*)part_o + src + VW * TPR * i);
        }
      }
    };
    // values 4 j .. 4 j + 3 of a loaded chunk
    auto vals = [&](const Raw& x, int j) -> f32x4 {
      if constexpr (PB16) {
        const uint32_t lo = x[2 * j], hi = x[2 * j + 1];
        return f32x4{__builtin_bit_cast(float, lo << 16), __builtin_bit_cast(float, lo & 0xFFFF0000u),
                     __builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xFFFF0000u)};
      } else {
        return x;
      }
    };
    float l[SG];
    Raw d[SG][NCH];
    load_group(0, l, d);
    // the first three W_UV chunks load behind the first group of partials
    // (so the merge waits only for its own loads) and during the merge
    issue_w(0);
    issue_w(1);
    issue_w(2);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < SG; ++u) mx = fmaxf(mx, l[u]);
    for (int s0 = SG; s0 < n_split; s0 += SG) {
#pragma unroll
      for (int u = 0; u < SG; ++u) mx = fmaxf(mx, part_lse[(sb + min(s0 + u, n_split - 1)) * R + row]);
    }
    float wsum = 0.f;
    f32x4 acc[NCH][VW / 4];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_split; s0 += SG) {
      if (s0 > 0) load_group(s0, l, d);
      float w[SG];
#pragma unroll
      for (int u = 0; u < SG; ++u) w[u] = (s0 + u < n_split && l[u] != -INFINITY) ? exp2f(l[u] - mx) : 0.f;
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        if (w[u] == 0.f) continue;      // absent or empty split: its partial may hold anything
        wsum += w[u];
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
          for (int j = 0; j < VW / 4; ++j) acc[i][j] += w[u] * vals(d[u][i], j);
      }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    if (r >= CO_ROWS) return;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) {
        f32x4 v = acc[i][j] * inv;
        if (!ok) v = f32x4{0.f, 0.f, 0.f, 0.f};
        const int k = cq + VW * TPR * i + 4 * j;
        if (ok && o_lat != nullptr) {
          const int64_t o = ((int64_t)n * H + h) * D_C + k;
          part_store(o_lat, o, v, o_bf16 != 0);
        }
        // the projection sees the latent output at the precision the caller
        // asked for: bf16 as is, fp32 as high + low bf16 terms
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 bh = to_bf16(v[e]);
          hi[e] = bf16_bits(bh);
          lo[e] = o_bf16 ? (uint16_t)0 : bf16_bits(to_bf16(v[e] - (float)bh));
        }
        const uint64_t ph = (uint64_t)hi[0] | ((uint64_t)hi[1] << 16) | ((uint64_t)hi[2] << 32) | ((uint64_t)hi[3] << 48);
        const uint64_t pl = (uint64_t)lo[0] | ((uint64_t)lo[1] << 16) | ((uint64_t)lo[2] << 32) | ((uint64_t)lo[3] << 48);
        *(uint64_t*)(at[0] + co_aoff(r, k)) = ph;
        *(uint64_t*)(at[1] + co_aoff(r, k)) = pl;
      }
    if (ok && lse_out != nullptr && (tid % TPR) == 0)
      lse_out[(int64_t)n * H + h] = wsum > 0.f ? (mx + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
  };
  {
    const int rows_here = min(CO_ROWS, N - n0);
    if (rows_here > 16) merge(std::integral_constant<int, 8>{});
    else if (rows_here > 8) merge(std::integral_constant<int, 16>{});
    else merge(std::integral_constant<int, 32>{});
  }

  // ---- projection: out[32 rows][32 w ..] over 4 chunks of 128 latent rows
  const int v0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = v0 + grp * 16 + 4 * (jj & 3);
  f32x16 acc = f32x16{};
  constexpr int NKC = D_C / CO_KC;
  constexpr int W_LOADS = CO_KC * AQ_CHUNKS / 256;     // direct loads per thread per chunk
  for (int kc = 0; kc < NKC; ++kc) {
    // chunk kc of this thread's loads is done once at most the younger
    // chunks' loads are outstanding: chunks 1 and 2 at kc = 0, then one
    // chunk (2, then 3, issued at kc = 1 into the slot chunk 0 used)
    if (kc == 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * W_LOADS) : "memory");
    else if (kc + 1 < NKC)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(W_LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // chunk kc (and the merged operands) visible; chunk kc-1 consumed
    if (kc == 1) issue_w(3);
    const char* w = wt[kc % 3];
#pragma unroll
    for (int ks = 0; ks < CO_KC / 16; ++ks) {
      const int kg = kc * CO_KC + ks * 16 + half * 8;        // A columns of this lane
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *(const i16x8*)(at[0] + co_aoff(l32, kg)));
      const bf16x8 alo = __builtin_bit_cast(bf16x8, *(const i16x8*)(at[1] + co_aoff(l32, kg)));
      const int krow = ks * 16 + 8 * half + (jj >> 2);
      const bf16x8 bw = join_tr(ds_read_tr16(w + aq_off(krow, bcol)), ds_read_tr16(w + aq_off(krow + 4, bcol)));
      acc = mfma32(ahi, bw, acc);
      if (!o_bf16) acc = mfma32(alo, bw, acc);
    }
  }
  // ---- stage the 32 x 128 output block, then write whole 256-byte rows
  __syncthreads();
  uint16_t(*ot)[D_V + 8] = (uint16_t(*)[D_V + 8])at[0];
#pragma unroll
  for (int r = 0; r < 16; ++r) ot[8 * (r >> 2) + 4 * half + (r & 3)][v0 + l32] = bf16_bits(to_bf16(acc[r]));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = i * 256 + tid;   // 32 rows x 16 chunks of 16 B
    const int rr = chunk >> 4, cc = chunk & 15;
    const int n = n0 + rr;
    if (n < N) *(i16x8*)(out + ((int64_t)n * H + h) * D_V + cc * 8) = *(const i16x8*)&ot[rr][cc * 8];
  }
}

}  // namespace

hipError_t launch_combine_out(const void* part_o, int part_bf16, const float* part_lse, const int32_t* seg_first,
                              const int32_t* seg_count, int B, int s_q, int H, const uint16_t* w_uv,
                              uint16_t* out, void* o_lat, int o_bf16, float* lse, hipStream_t stream) {
  const int N = B * s_q;
  const dim3 grid(H, (N + CO_ROWS - 1) / CO_ROWS);
  if (part_bf16)
    hipLaunchKernelGGL(combine_out_kernel<true>, grid, dim3(256), 0, stream, part_o, part_lse, seg_first, seg_count,
                       s_q, H, N, w_uv, out, o_lat, o_bf16, lse);
  else
    hipLaunchKernelGGL(combine_out_kernel<false>, grid, dim3(256), 0, stream, part_o, part_lse, seg_first,
                       seg_count, s_q, H, N, w_uv, out, o_lat, o_bf16, lse);
  return hipGetLastError();
}

hipError_t launch_absorb_q(const uint16_t* q, const uint16_t* w_uk, uint16_t* q_lat, int N, int H,
                           hipStream_t stream) {
  const int groups = (N + AQ_ROWS - 1) / AQ_ROWS;
  hipLaunchKernelGGL(absorb_q_kernel, dim3(H * groups, D_C / AQ_COLS), dim3(256), 0, stream, q, w_uk, q_lat, N, H);
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
