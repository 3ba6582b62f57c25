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
  // the transposed product, D^T[column][token] (the weight fragment as the
  // A operand): lane (l32, half) then holds columns 8 g + 4 half .. + 3
  // (g = 0..3) of token l32, four 8-byte runs of its output row
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D_NOPE / 16; ++ks) {
    const int krow = ks * 16 + 8 * half + (jj >> 2);
    const bf16x8 bw = join_tr(ds_read_tr16(wt + aq_off(krow, bcol)), ds_read_tr16(wt + aq_off(krow + 4, bcol)));
    const i16x8 z = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    acc0 = mfma32(bw, __builtin_bit_cast(bf16x8, ok0 ? a0[ks] : z), acc0);
    acc1 = mfma32(bw, __builtin_bit_cast(bf16x8, ok1 ? a1[ks] : z), acc1);
  }
  // stage the 64 x 128 output block in LDS (8-byte runs), then write whole
  // 256-byte rows.  The rows are written with the nontemporal hint: they are
  // read back only by the next kernel, and left as dirty lines in this XCD's
  // L2 they lengthen the end of the launch (measured: 10.3 -> 9.4 us at
  // B = 64, H = 128)
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int col = c0 + 8 * g4 + 4 * half;
    *(uint64_t*)&ot[l32][col] = pack_bf16x4(f32x4{acc0[4 * g4], acc0[4 * g4 + 1], acc0[4 * g4 + 2], acc0[4 * g4 + 3]});
    *(uint64_t*)&ot[l32 + 32][col] =
        pack_bf16x4(f32x4{acc1[4 * g4], acc1[4 * g4 + 1], acc1[4 * g4 + 2], acc1[4 * g4 + 3]});
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int chunk = i * 256 + tid;          // 64 rows x 16 chunks of 16 B
    const int rr = chunk >> 4, cc = chunk & 15;
    const int nn = n0 + rr;
    if (nn < N)
      __builtin_nontemporal_store(*(const i16x8*)&ot[rr][cc * 8],
                                  (i16x8*)(q_lat + ((int64_t)nn * H + h) * ROWW + cblk * AQ_COLS + cc * 8));
  }
  // the rope part of the query rows is carried over unchanged
  if (rope_on) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + rr0 + 32 * i;
      if (n < N) __builtin_nontemporal_store(rope[i], (i16x8*)(q_lat + ((int64_t)n * H + h) * ROWW + D_C + rc * 8));
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
// HBM.  grid (H, ceil(N / 32)), 4 waves; a work-group takes 32 query rows of
// one head, and wave w computes output columns 32 w .. 32 w + 31.  The merge
// arithmetic is the one of the stand-alone merge kernel, term for term (splits
// added in order, the same weights), and the projection accumulates in the
// order of absorb_out, so the bits are the same as the two steps apart.
//
// Two paths, chosen per work-group from the split counts of its rows:
//  * at most four splits per row (the common case): the partials (registers)
//    and W_UV rows (LDS, all of W_UV[h] resident) of the four 128-column
//    chunks are issued chunk by chunk at the start; each chunk is merged,
//    staged as bf16 high (+ low) MFMA operands and projected as soon as its
//    loads are in, so the merge and the projection of one chunk overlap the
//    arrival of the next;
//  * more splits: all 512 columns of a row are merged four splits at a time,
//    then projected through W_UV in four staged chunks.
// ---------------------------------------------------------------------------
constexpr int CO_ROWS = 32;
constexpr int CO_ROWS_NARROW = 8;                 // rows per work-group of a narrow launch
constexpr int kComputeUnits = 256;
constexpr int CO_KC = 128;                        // W_UV rows (latent columns) per chunk
constexpr int CO_NKC = D_C / CO_KC;               // 4 chunks
constexpr int CO_WBYTES = CO_KC * D_V * 2;        // 32 KB: W_UV rows of one chunk
constexpr int CO_W_LOADS = CO_WBYTES / (256 * 16);   // 8 direct loads per thread per chunk
constexpr int CO_SG = 4;                          // splits per load group
constexpr int CO_LDS = 160 * 1024;
// many-split path: [32][512] bf16 operand planes
constexpr int CO_ABYTES = CO_ROWS * D_C * 2;      // 32 KB
static_assert(3 * CO_WBYTES + 2 * CO_ABYTES <= CO_LDS, "LDS budget (many splits)");
// four-split path: [32][128] bf16 operand planes of one chunk, high and low,
// double-buffered over the chunks
constexpr int CF_ABYTES = CO_ROWS * CO_KC * 2;    // 8 KB
static_assert(CO_NKC * CO_WBYTES + 4 * CF_ABYTES <= CO_LDS, "LDS budget (four splits)");

// row-major [32][512] bf16 operand plane; the 16-byte chunk index is XORed
// with the row so that the 32 rows of an MFMA fragment read hit all banks
__device__ __forceinline__ int co_aoff(int r, int k) {
  return r * (D_C * 2) + (((k >> 3) ^ (r & 15)) << 4) + (k & 7) * 2;
}
// [32][128] bf16 plane of one chunk: 16-byte chunk c16 of row r, XORed the same way
__device__ __forceinline__ uint32_t cf_aoff(int r, int c16) {
  return (uint32_t)(r * (CO_KC * 2) + ((c16 ^ (r & 15)) << 4));
}

// W_UV rows kc*128 .. +127 of one head into a 32 KB LDS slot (direct loads,
// chunk index XORed as aq_off expects)
__device__ __forceinline__ void co_issue_w(const uint16_t* wsrc, char* slot, int kc, int wave, int lane) {
  char* dst = slot + wave * 64 * 16;
#pragma unroll
  for (int i = 0; i < CO_W_LOADS; ++i) {
    const int s = i * 256 + wave * 64 + lane;
    const int k = s / AQ_CHUNKS;
    const int cc = (s % AQ_CHUNKS) ^ chunk_swz(k);
    __builtin_amdgcn_global_load_lds((const void*)(wsrc + (int64_t)(kc * CO_KC + k) * D_V + cc * 8),
                                     (lds_void_t*)(dst + i * 256 * 16), 16, 0, 0);
  }
}

// Global loads issued as inline asm, in program order among the direct
// W_UV loads, so that explicit vmcnt waits can count them (the compiler's
// own waits turn into vmcnt(0) while direct-to-LDS loads are in flight).  A
// consumer first calls wait_vm<N>() on the loaded registers: N = loads issued
// after the one waited for.
__device__ __forceinline__ void gload_b128(u32x4& d, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(d) : "v"(p) : "memory");
}
__device__ __forceinline__ void gload_b32(float& d, const void* p) {
  asm volatile("global_load_dword %0, %1, off" : "=v"(d) : "v"(p) : "memory");
}
template <int N, typename... R>
__device__ __forceinline__ void wait_vm(R&... regs) {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
  (touch_reg(regs), ...);
}

// the 32 x 128 output block of the work-group: staged in LDS (wave w wrote
// its columns), then its first ROWS rows written as whole 256-byte rows
template <int ROWS>
__device__ __forceinline__ void co_store_out(const f32x16& acc, char* stage, uint16_t* out, int n0, int N, int H,
                                             int h, int tid, int wave, int half, int l32) {
  uint16_t(*ot)[D_V + 8] = (uint16_t(*)[D_V + 8])stage;
  const int v0 = wave * 32;
#pragma unroll
  for (int r = 0; r < 16; ++r) ot[8 * (r >> 2) + 4 * half + (r & 3)][v0 + l32] = bf16_bits(to_bf16(acc[r]));
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int chunk = i * 256 + tid;   // 32 rows x 16 chunks of 16 B
    const int rr = chunk >> 4, cc = chunk & 15;
    const int n = n0 + rr;
    if (rr < ROWS && n < N) *(i16x8*)(out + ((int64_t)n * H + h) * D_V + cc * 8) = *(const i16x8*)&ot[rr][cc * 8];
  }
}

// Many splits per row: merge all 512 columns (four splits at a time), stage
// them as bf16 high + low operands in LDS, then stream W_UV[h] through LDS in
// four 128-row chunks.  ROWS query rows per work-group (32, or 8 when the
// launch would otherwise leave compute units idle); the products of the
// 32-row MFMA tile past them are computed and not stored.
template <bool PB16, int ROWS, bool EARLY_W>
__device__ __forceinline__ void combine_out_many(char* smem, const void* __restrict__ part_o,
                                                 const float* __restrict__ part_lse,
                                                 const int32_t* __restrict__ seg_first,
                                                 const int32_t* __restrict__ seg_count, int s_q, int H, int N,
                                                 const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
                                                 void* o_lat, int o_bf16, float* lse_out) {
  char* const wt = smem;                              // [3][CO_WBYTES]: W_UV chunks 0-2, then 3 in slot 0
  char* const at = smem + 3 * CO_WBYTES;              // [2][CO_ABYTES]: [hi, lo]
  const int h = blockIdx.x, n0 = blockIdx.y * ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int R = s_q * H;
  const uint16_t* wsrc = w_uv + (int64_t)h * D_C * D_V;

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
    const bool ok = r < ROWS && n < N;
    const int b = ok ? n / s_q : 0;
    const int row = ok ? (n - b * s_q) * H + h : 0;
    const int64_t sb = seg_first[b];
    const int n_split = seg_count[b];
    // splits are taken four at a time with every load of the group in flight
    // together (indices past the last split reload it and get weight 0), and
    // added in split order.  The first group's partials are loaded with the
    // log-sum-exps, before the maximum is known (it only sets their weights).
    auto load_group = [&](int s0, float (&l)[CO_SG], Raw (&d)[CO_SG][NCH]) {
#pragma unroll
      for (int u = 0; u < CO_SG; ++u) {
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
    float l[CO_SG];
    Raw d[CO_SG][NCH];
    load_group(0, l, d);
    // the first three W_UV chunks load behind the first group of partials
    // (so the merge waits only for its own loads) and during the merge
    if constexpr (!EARLY_W) co_issue_w(wsrc, wt, 0, wave, lane);   // else issued at kernel entry
    co_issue_w(wsrc, wt + CO_WBYTES, 1, wave, lane);
    co_issue_w(wsrc, wt + 2 * CO_WBYTES, 2, wave, lane);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < CO_SG; ++u) mx = fmaxf(mx, l[u]);
    for (int s0 = CO_SG; s0 < n_split; s0 += CO_SG) {
#pragma unroll
      for (int u = 0; u < CO_SG; ++u) mx = fmaxf(mx, part_lse[(sb + min(s0 + u, n_split - 1)) * R + row]);
    }
    float wsum = 0.f;
    f32x4 acc[NCH][VW / 4];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto add_group = [&](int s0, const float (&lg)[CO_SG], const Raw (&dg)[CO_SG][NCH]) {
      float w[CO_SG];
#pragma unroll
      for (int u = 0; u < CO_SG; ++u) w[u] = (s0 + u < n_split && lg[u] != -INFINITY) ? exp2f(lg[u] - mx) : 0.f;
#pragma unroll
      for (int u = 0; u < CO_SG; ++u) {
        if (w[u] == 0.f) continue;      // absent or empty split: its partial may hold anything
        wsum += w[u];
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
          for (int j = 0; j < VW / 4; ++j) acc[i][j] += w[u] * vals(dg[u][i], j);
      }
    };
    if constexpr (PB16) {
      // groups in pairs: the next group's loads are in flight while the
      // current one is added (two register buffers, so both stay static)
      float l2[CO_SG];
      Raw d2[CO_SG][NCH];
      for (int s0 = 0; s0 < n_split; s0 += 2 * CO_SG) {
        if (s0 + CO_SG < n_split) load_group(s0 + CO_SG, l2, d2);
        add_group(s0, l, d);
        if (s0 + 2 * CO_SG < n_split) load_group(s0 + 2 * CO_SG, l, d);
        if (s0 + CO_SG < n_split) add_group(s0 + CO_SG, l2, d2);
      }
    } else {
      // fp32 partials: one group's registers are all there is room for
      for (int s0 = 0; s0 < n_split; s0 += CO_SG) {
        if (s0 > 0) load_group(s0, l, d);
        add_group(s0, l, d);
      }
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    if (r >= ROWS) return;
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
        *(uint64_t*)(at + co_aoff(r, k)) = ph;
        *(uint64_t*)(at + CO_ABYTES + co_aoff(r, k)) = pl;
      }
    if (ok && lse_out != nullptr && (tid % TPR) == 0)
      lse_out[(int64_t)n * H + h] = wsum > 0.f ? (mx + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
  };
  {
    const int rows_here = min(ROWS, N - n0);
    if (rows_here > 16) merge(std::integral_constant<int, 8>{});
    else if (rows_here > 8) merge(std::integral_constant<int, 16>{});
    else merge(std::integral_constant<int, 32>{});
  }

  // ---- projection: out[32 rows][32 w ..] over 4 chunks of 128 latent rows
  const int v0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = v0 + grp * 16 + 4 * (jj & 3);
  f32x16 acc = f32x16{};
  for (int kc = 0; kc < CO_NKC; ++kc) {
    // chunk kc of this thread's loads is done once at most the younger
    // chunks' loads are outstanding: chunks 1 and 2 at kc = 0, then one
    // chunk (2, then 3, issued at kc = 1 into the slot chunk 0 used)
    if (kc == 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * CO_W_LOADS) : "memory");
    else if (kc + 1 < CO_NKC)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CO_W_LOADS) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // chunk kc (and the merged operands) visible; chunk kc-1 consumed
    if (kc == 1) co_issue_w(wsrc, wt, 3, wave, lane);
    const char* w = wt + (kc % 3) * CO_WBYTES;
#pragma unroll
    for (int ks = 0; ks < CO_KC / 16; ++ks) {
      const int kg = kc * CO_KC + ks * 16 + half * 8;        // A columns of this lane
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *(const i16x8*)(at + co_aoff(l32, kg)));
      const bf16x8 alo = __builtin_bit_cast(bf16x8, *(const i16x8*)(at + CO_ABYTES + co_aoff(l32, kg)));
      const int krow = ks * 16 + 8 * half + (jj >> 2);
      const bf16x8 bw = join_tr(ds_read_tr16(w + aq_off(krow, bcol)), ds_read_tr16(w + aq_off(krow + 4, bcol)));
      acc = mfma32(ahi, bw, acc);
      if (!o_bf16) acc = mfma32(alo, bw, acc);
    }
  }
  __syncthreads();
  co_store_out<ROWS>(acc, at, out, n0, N, H, h, tid, wave, half, l32);
}

// At most four splits per row: W_UV[h] resident in LDS, the partials of the
// four 128-column chunks streaming behind it (see above).  Thread -> row
// r = tid / 8 and, per chunk, 16 columns: bf16 partials in two 16-byte loads
// (columns 8 (tid % 8) and 64 + 8 (tid % 8)), fp32 in four (columns 4 (tid %
// 8) + 32 i), so the 8 threads of a row read whole 128-byte lines.
// (part_o and part_lse are not __restrict__ here: their loads must not move
// across the compiler barriers that fix the issue order.)
// The four-split path's issue order, per thread (P(c): partials of chunk c,
// CO_SG * 2 loads for bf16 and CO_SG * 4 for fp32; W(c): W_UV rows of chunk
// c, CO_W_LOADS direct loads):
//   bf16:  log-sum-exps, P(0), W(0), P(1), W(1), P(2), W(2), P(3), W(3)
//   fp32:  log-sum-exps, P(0), W(0), P(1), W(1), W(2), W(3); P(2) after the
//          merge of chunk 0 and P(3) after the merge of chunk 1
// co_after() is the number of loads issued after P(kc) (what = 0) or W(kc)
// (what = 1) by the time chunk kc waits for them; global stores issued in
// between only make such a wait stricter.
constexpr int co_after(bool pb16, int what, int kc) {
  if (pb16) return (CO_NKC - 1 - kc) * (CO_SG * 2 + CO_W_LOADS) + (what == 0 ? CO_W_LOADS : 0);
  constexpr int P = CO_SG * 4, Wl = CO_W_LOADS;
  if (what == 0) return kc == 0 ? Wl + P + 3 * Wl : kc == 1 ? 3 * Wl + P : kc == 2 ? P : 0;
  // W(2), W(3) precede P(2): once P(2) is in, so are they
  return kc == 0 ? P + 3 * Wl + P : kc == 1 ? 2 * Wl + 2 * P : kc == 2 ? P : 0;
}

// the same counts when W_UV chunk 0 was issued before everything else (at
// kernel entry): only the merge of chunk 0 has its eight loads fewer behind it
constexpr int co_after_e(bool pb16, bool early_w, int what, int kc) {
  return (early_w && what == 0 && kc == 0) ? co_after(pb16, 0, 0) - CO_W_LOADS : co_after(pb16, what, kc);
}

template <bool PB16, bool OB16, bool EARLY_W>
__device__ __forceinline__ void combine_out_few(char* smem, const void* part_o, const float* part_lse, int64_t sb,
                                                int n_split, int s_q, int H, int N, const uint16_t* w_uv,
                                                uint16_t* out, void* o_lat, float* lse_out) {
  char* const wt = smem;                               // [4][CO_WBYTES]
  char* const at = smem + CO_NKC * CO_WBYTES;          // [2 buffers][hi, lo][CF_ABYTES]
  const int h = blockIdx.x, n0 = blockIdx.y * CO_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int R = s_q * H;
  const uint16_t* wsrc = w_uv + (int64_t)h * D_C * D_V;

  constexpr int NL = PB16 ? 2 : 4;           // 16-byte loads per split and chunk
  constexpr int VW = PB16 ? 8 : 4;           // values per load
  constexpr int NST = PB16 ? 4 : 2;          // chunks of partials in flight
  using Raw = typename std::conditional<PB16, u32x4, f32x4>::type;
  const int r = tid >> 3, cg = tid & 7;
  const int n = n0 + r;
  const bool ok = n < N;
  const int b = ok ? n / s_q : 0;
  const int row = ok ? (n - b * s_q) * H + h : 0;
  auto col = [&](int kc, int i) -> int { return kc * CO_KC + (PB16 ? 8 * cg + 64 * i : 4 * cg + 32 * i); };
  // split s of the group (past the last split: the last one again, weight 0)
  auto src_row = [&](int s) -> int64_t { return ((sb + max(min(s, n_split - 1), 0)) * R + row) * D_C; };
  constexpr int LPC = CO_SG * NL;             // loads per chunk of partials
  u32x4 d[NST][CO_SG][NL];
  auto load_chunk = [&](int kc, u32x4 (&dst)[CO_SG][NL]) {
#pragma unroll
    for (int s = 0; s < CO_SG; ++s) {
      const int64_t base = src_row(s);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if constexpr (PB16) gload_b128(dst[s][i], (const uint16_t*)part_o + base + col(kc, i));
        else gload_b128(dst[s][i], (const float*)part_o + base + col(kc, i));
      }
    }
  };
  // issue order (see co_after): the log-sum-exps, then per chunk its
  // partials (the first NST chunks) and its W_UV rows; the partials of chunk
  // kc + NST follow the merge of chunk kc
  float l[CO_SG];
#pragma unroll
  for (int s = 0; s < CO_SG; ++s) gload_b32(l[s], part_lse + (sb + max(min(s, n_split - 1), 0)) * R + row);
  static_for<0, CO_NKC>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    if constexpr (c < NST) load_chunk(c, d[c]);
    if constexpr (!(EARLY_W && c == 0)) co_issue_w(wsrc, wt + c * CO_WBYTES, c, wave, lane);
  });
  wait_vm<co_after_e(PB16, EARLY_W, 0, 0)>(l[0], l[1], l[2], l[3]);

  // weights of the splits in split order (as the stand-alone merge does)
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < CO_SG; ++s) mx = fmaxf(mx, s < n_split ? l[s] : -INFINITY);
  float w[CO_SG];
  float wsum = 0.f;
#pragma unroll
  for (int s = 0; s < CO_SG; ++s) {
    w[s] = (s < n_split && l[s] != -INFINITY) ? exp2f(l[s] - mx) : 0.f;
    if (w[s] != 0.f) wsum += w[s];
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  auto vals = [&](const Raw& x, int j) -> f32x4 {
    if constexpr (PB16) {
      const uint32_t lo = x[2 * j], hi = x[2 * j + 1];
      return f32x4{__builtin_bit_cast(float, lo << 16), __builtin_bit_cast(float, lo & 0xFFFF0000u),
                   __builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xFFFF0000u)};
    } else {
      return x;
    }
  };

  const int v0 = wave * 32;
  const int grp = (lane >> 4) & 1, jj = lane & 15;
  const int bcol = v0 + grp * 16 + 4 * (jj & 3);
  f32x16 acc_o = f32x16{};
  static_for<0, CO_NKC>([&](auto kcc) {
    constexpr int kc = decltype(kcc)::value;
    constexpr int st = kc % NST;
    // ---- merge chunk kc, once its loads are in
    wait_vm<co_after_e(PB16, EARLY_W, 0, kc)>();
#pragma unroll
    for (int s = 0; s < CO_SG; ++s)
#pragma unroll
      for (int i = 0; i < NL; ++i) touch_reg(d[st][s][i]);
    f32x4 acc[NL][VW / 4];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // an absent or empty split (weight 0) may hold anything: its values are
    // replaced by zeros, which leaves every sum exactly as skipping it does
#pragma unroll
    for (int s = 0; s < CO_SG; ++s) {
      const bool use = w[s] != 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < VW / 4; ++j) {
          const f32x4 x = vals(__builtin_bit_cast(Raw, d[st][s][i]), j);
          acc[i][j] += w[s] * f32x4{use ? x[0] : 0.f, use ? x[1] : 0.f, use ? x[2] : 0.f, use ? x[3] : 0.f};
        }
    }
    // the registers of chunk kc are free: the partials of chunk kc + NST
    if constexpr (kc + NST < CO_NKC) load_chunk(kc + NST, d[st]);
    f32x4 v[NL][VW / 4];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) {
        v[i][j] = acc[i][j] * inv;
        if (!ok) v[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // ---- stage the high (+ low) operand planes of the chunk
    char* const ahi_p = at + (kc & 1) * 2 * CF_ABYTES;
    char* const alo_p = ahi_p + CF_ABYTES;
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int j = 0; j < VW / 4; ++j) {
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 bh = to_bf16(v[i][j][e]);
          hi[e] = bf16_bits(bh);
          lo[e] = OB16 ? (uint16_t)0 : bf16_bits(to_bf16(v[i][j][e] - (float)bh));
        }
        const uint64_t ph = (uint64_t)hi[0] | ((uint64_t)hi[1] << 16) | ((uint64_t)hi[2] << 32) | ((uint64_t)hi[3] << 48);
        const uint64_t pl = (uint64_t)lo[0] | ((uint64_t)lo[1] << 16) | ((uint64_t)lo[2] << 32) | ((uint64_t)lo[3] << 48);
        const int c = col(0, i) + 4 * j;                 // column within the chunk
        const uint32_t off = cf_aoff(r, c >> 3) + (c & 7) * 2;
        *(uint64_t*)(ahi_p + off) = ph;
        *(uint64_t*)(alo_p + off) = pl;
      }
    wait_vm<co_after_e(PB16, EARLY_W, 1, kc)>();   // W_UV rows of chunk kc landed (this thread's share)
    barrier_lds();     // chunk kc's operands visible; the buffer of chunk kc - 2 consumed
    // the latent output, when asked for (stores issued after the W_UV wait)
    if (ok && o_lat != nullptr) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int j = 0; j < VW / 4; ++j)
          part_store(o_lat, ((int64_t)n * H + h) * D_C + col(kc, i) + 4 * j, v[i][j], OB16);
    }
    // ---- projection of chunk kc.  The operand reads are inline asm with
    // exact lgkmcnt waits, one k-step ahead (compiler-issued LDS reads would
    // first wait for every outstanding global load).
    {
      const uint32_t a_base = lds_addr(ahi_p);
      const uint32_t w_base = lds_addr(wt + kc * CO_WBYTES);
      // rows 16 ks + 8 half + jj / 4 (+ 4): the XOR of aq_off depends on
      // the row's low three bits only, so the k-steps are immediate offsets
      const uint32_t b0 = w_base + aq_off(8 * half + (jj >> 2), bcol);
      const uint32_t b1 = w_base + aq_off(8 * half + (jj >> 2) + 4, bcol);
      constexpr int RPK = OB16 ? 3 : 4;              // LDS reads per k-step
      i16x8 ah[2], al[2];
      i16x4 bt[2][2];
      auto issue = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        const uint32_t aa = a_base + cf_aoff(l32, 2 * ks + half);
        lds_read_b128<0>(ah[ks & 1], aa);
        if constexpr (!OB16) lds_read_b128<CF_ABYTES>(al[ks & 1], aa);
        lds_read_tr16<ks * 4096>(bt[ks & 1][0], b0);
        lds_read_tr16<ks * 4096>(bt[ks & 1][1], b1);
      };
      issue(std::integral_constant<int, 0>{});
      static_for<0, CO_KC / 16>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        if constexpr (ks + 1 < CO_KC / 16) issue(std::integral_constant<int, ks + 1>{});
        constexpr int younger = ks + 1 < CO_KC / 16 ? RPK : 0;
        wait_lgkm<younger>(ah[ks & 1], al[ks & 1], bt[ks & 1][0], bt[ks & 1][1]);
        const bf16x8 bw = join_tr(bt[ks & 1][0], bt[ks & 1][1]);
        acc_o = mfma32(__builtin_bit_cast(bf16x8, ah[ks & 1]), bw, acc_o);
        if constexpr (!OB16) acc_o = mfma32(__builtin_bit_cast(bf16x8, al[ks & 1]), bw, acc_o);
      });
    }
  });
  if (ok && lse_out != nullptr && cg == 0)
    lse_out[(int64_t)n * H + h] = wsum > 0.f ? (mx + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
  // chunk 2's operand buffer is free once every wave is past the last barrier
  co_store_out<CO_ROWS>(acc_o, at, out, n0, N, H, h, tid, wave, half, l32);
}

template <bool PB16, bool OB16, int ROWS>
__global__ __launch_bounds__(256) void combine_out_kernel(const void* part_o, const float* part_lse,
                                                          const int32_t* __restrict__ seg_first,
                                                          const int32_t* __restrict__ seg_count,
                                                          int s_q, int H, int N,
                                                          const uint16_t* __restrict__ w_uv,
                                                          uint16_t* __restrict__ out, void* o_lat,
                                                          float* lse_out) {
  __shared__ __attribute__((aligned(1024))) char smem[CO_LDS];
  // with bf16 partials and 32-row blocks, W_UV chunk 0 (which needs only the
  // head) loads into its LDS slot during the split bookkeeping's round trip;
  // both paths keep chunk 0 there
  constexpr bool EARLY_W = PB16 && ROWS == CO_ROWS;
  const int n0 = blockIdx.y * ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // split count and first slot of this thread's row (the four-split path's
  // row mapping); lane l % 32 also fetches the split count of row l % 32, so
  // that every wave sees every count of the work-group's rows itself.
  // The loads are inline asm, counted past the W_UV loads behind them.
  const int r = tid >> 3;
  const int n = n0 + r;
  const int b = n < N ? n / s_q : 0;
  const int rl = lane & 31, nl = n0 + rl;
  const bool okl = rl < ROWS && nl < N;
  float f_first, f_count, f_rl;
  gload_b32(f_first, seg_first + b);
  gload_b32(f_count, seg_count + b);
  gload_b32(f_rl, seg_count + (okl ? nl / s_q : 0));
  if constexpr (EARLY_W) co_issue_w(w_uv + (int64_t)blockIdx.x * D_C * D_V, smem, 0, wave, lane);
  wait_vm<EARLY_W ? CO_W_LOADS : 0>(f_first, f_count, f_rl);
  const int64_t sb = __builtin_bit_cast(int32_t, f_first);
  const int ns = __builtin_bit_cast(int32_t, f_count);
  // a row with more than four splits takes the many-split path (the same
  // answer in every wave)
  const bool many = __builtin_amdgcn_ballot_w64(okl && __builtin_bit_cast(int32_t, f_rl) > CO_SG) != 0;
  if (ROWS == CO_ROWS && !many)
    combine_out_few<PB16, OB16, EARLY_W>(smem, part_o, part_lse, sb, ns, s_q, H, N, w_uv, out, o_lat, lse_out);
  else
    combine_out_many<PB16, ROWS, EARLY_W>(smem, part_o, part_lse, seg_first, seg_count, s_q, H, N, w_uv, out,
                                          o_lat, OB16 ? 1 : 0, lse_out);
}

}  // namespace

hipError_t launch_combine_out(const void* part_o, int part_bf16, const float* part_lse, const int32_t* seg_first,
                              const int32_t* seg_count, int B, int s_q, int H, const uint16_t* w_uv,
                              uint16_t* out, void* o_lat, int o_bf16, float* lse, hipStream_t stream) {
  const int N = B * s_q;
  // 32 query rows per work-group, or 8 when that leaves compute units idle
  // (few query tokens: each work-group then streams a quarter of the rows)
  const bool narrow = (int64_t)H * ((N + CO_ROWS - 1) / CO_ROWS) < kComputeUnits;
  const int rows = narrow ? CO_ROWS_NARROW : CO_ROWS;
  const dim3 grid(H, (N + rows - 1) / rows);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, part_o, part_lse, seg_first, seg_count, s_q, H, N, w_uv, out,
                       o_lat, lse);
  };
  auto pick = [&](auto rc) {
    constexpr int R = decltype(rc)::value;
    if (part_bf16) {
      if (o_bf16) go(combine_out_kernel<true, true, R>);
      else go(combine_out_kernel<true, false, R>);
    } else {
      if (o_bf16) go(combine_out_kernel<false, true, R>);
      else go(combine_out_kernel<false, false, R>);
    }
  };
  if (narrow) pick(std::integral_constant<int, CO_ROWS_NARROW>{});
  else pick(std::integral_constant<int, CO_ROWS>{});
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
