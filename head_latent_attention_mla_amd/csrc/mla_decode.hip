// Split-T latent attention for absorbed MLA decode on gfx950, plus the
// log-sum-exp merge of the splits.
//
// The computation ("MLA, dim by dim", section "MLA Decode"; "Why MLA and MTP
// Fight Each Other", sections 4.2 and 8): every head of every query token
// scores its 576-wide latent query against the same cached rows, softmaxes,
// and averages the rows' 512 latent columns.  All heads share each cached
// row, so one work-group holds 128 query rows (heads x query tokens) and reads
// every 64-row latent tile from HBM once into LDS, where it serves both the
// score contraction (K = 576) and the value contraction (K = 64 rows).
//
// Work-group = 4 waves, one per SIMD.  Per tile:
//   1. scores: wave w computes S^T[t][row] for ITS 32 query rows (MFMA
//      32x32x16, A = tile rows from LDS, B = latent queries held in VGPRs),
//      runs the online softmax for those rows, and writes the bf16
//      probabilities to LDS already laid out as MFMA B fragments;
//   2. values: wave w computes O^T[c][row] for 128 latent columns c and ALL
//      128 query rows (A = tile read transposed from LDS, B = probabilities
//      from LDS), so each transposed tile fragment feeds 4 MFMAs.
// The k-slot order of the value contraction is permuted so that a lane's
// score accumulators are exactly its B fragment; the transposed tile reads
// follow the same permutation.
//
// Softmax reference: each row exponentiates against a reference m (log2
// domain) that only moves when the running maximum exceeds it by more than
// 64, in steps of 64 (probabilities stay <= 2^64, fine in bf16 and fp32).  A
// move is rare; the owning wave signals it to the other waves in the sign bits
// of three of the row's probabilities (always >= 0 otherwise), and every wave
// multiplies that row's accumulators by 2^(-64 k).
//
// The cache is split along T into n_split ranges; each (sequence, range, row
// group) is one work-group writing a normalised partial output ([c][row]
// major, so stores are row-contiguous) and its log2-domain log-sum-exp.  The
// combine kernel merges the ranges.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int KT = 64;                        // cached rows per LDS tile
constexpr int CHUNKS = ROWW * 2 / 16;         // 72 16-byte chunks per bf16 row
constexpr int TILE_BYTES = KT * ROWW * 2;     // 73,728
constexpr int P_BYTES = 128 * KT * 2;         // bf16 probabilities of 128 rows x 64 t
constexpr int NTHREADS = 256;
constexpr int LOADS_PER_WAVE = KT / 4 * CHUNKS / 64;  // 18: each wave loads 16 rows
constexpr float REF_STEP = 64.0f;             // reference moves in steps of 2^64
static_assert(2 * TILE_BYTES + P_BYTES <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int lds_off(int t, int elem) {
  const int c = elem >> 3;
  return (t * CHUNKS + (c ^ chunk_swz(t))) * 16 + (elem & 7) * 2;
}

// Work-group barriers that wait only for what the barrier publishes.
// __syncthreads() would also wait for the prefetch of the next tile (vmcnt).
__device__ __forceinline__ void barrier_tile_ready() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc *= alpha on an accumulator that lives in AGPRs, one register at a time
// (a plain vector multiply makes the register allocator move the whole block
// through VGPRs).
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = acc[i];
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t) : "v"(alpha));
    acc[i] = x;
  }
}

// lanes l and l ^ 32 hold the same query row: combine their values.
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another, so swapping x with a copy of x leaves {x[l], x[l ^ 32]} in
// the two registers of every lane.  Issued as inline asm: the compiler's own
// builtin is treated as returning two equal values and one gets folded away.
// The s_nop padding covers the VALU-write -> permlane-read hazard and the
// permlane-write -> VALU-read hazard.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

// keep a value opaque to the optimiser (stops loop-invariant hoisting of
// per-lane address arithmetic that would otherwise pin registers)
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <bool PAGED>
__global__ __launch_bounds__(NTHREADS, 1) void decode_split_bf16_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE_BYTES + P_BYTES];
  char* const pbuf = smem + 2 * TILE_BYTES;
  const uint32_t smem_a = lds_addr(smem);
  const uint32_t pbuf_a = smem_a + 2 * TILE_BYTES;

  // blockIdx -> work item: consecutive work items (the row groups and splits
  // of one sequence) go to the same XCD, whose L2 they share.
  const int xcd = blockIdx.x % 8;
  const int w_item = xcd * p.work_per_xcd + blockIdx.x / 8;
  if (w_item >= p.n_work) return;
  const int g = w_item % p.n_groups;
  const int bsplit = w_item / p.n_groups;
  const int split = bsplit % p.n_split;
  const int b = bsplit / p.n_split;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int T = p.seqlens[b];
  const int t_begin = split * p.split_rows;
  const int t_end = min(T, t_begin + p.split_rows);
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + KT - 1) / KT : 0;

  // ---- rows owned by this wave for the score phase
  const int own_r = g * 128 + wave * 32 + l32;
  const bool own_ok = own_r < p.R;
  const bool wave_on = g * 128 + wave * 32 < p.R;
  const int jq = own_ok ? own_r / p.H : 0;
  const int visible = p.causal ? (T - p.s_q + jq + 1) : T;
  const int lim = min(visible, t_end);

  bf16x8 qf[ROWW / 16];
  {
    const uint16_t* qrow = p.q_lat + ((int64_t)b * p.R + (own_ok ? own_r : 0)) * ROWW + half * 8;
#pragma unroll
    for (int ks = 0; ks < ROWW / 16; ++ks) {
      i16x8 v = *(const i16x8*)(qrow + ks * 16);
      if (!own_ok) v = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tile loader.  Wave w copies rows 16w..16w+15 of the tile: 18 loads
  // of 64 lanes x 16 B, each filling 1 KB of LDS in order.  The chunk that
  // lane l fetches for LDS slot 64 k + l follows the XOR swizzle; the pattern
  // repeats every 8 rows (9 loads), so 9 per-lane byte offsets (< 2^14,
  // packed two per register) cover all 18 loads.  The buffer window of a tile
  // ends at the sequence's last row, so rows past it read as zero.
  uint32_t loff[5] = {0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int s = 64 * k + lane;
    const int tl = s / CHUNKS;
    const int c = (s - tl * CHUNKS) ^ chunk_swz(tl);
    loff[k >> 1] |= (uint32_t)(tl * ROWW * 2 + c * 16) << (16 * (k & 1));
  }
  const char* rows = (const char*)p.rows;
  // per-tile load state: buffer window over the tile's rows and LDS target
  auto tile_rsrc = [&](int tile) {
    const int ts = t_begin + tile * KT;
    const char* base;
    if (PAGED) {
      const int blk = p.block_table[(int64_t)b * p.max_blocks + (ts >> 6)];
      base = rows + (int64_t)blk * KT * ROWW * 2;
    } else {
      base = rows + ((int64_t)b * p.T_stride + ts) * ROWW * 2;
    }
    const int valid = min(KT, T - ts);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, valid * ROWW * 2, 0x00020000);
  };
  const int soff = wave * (16 * ROWW * 2);
  auto issue_load = [&](__amdgpu_buffer_rsrc_t rsrc, int buf, auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int k9 = k % 9;
    const uint32_t vo = (loff[k9 >> 1] >> (16 * (k9 & 1))) & 0xFFFFu;
    char* dst = smem + buf * TILE_BYTES + wave * (16 * ROWW * 2) + k * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, vo,
                                             soff + (k >= 9 ? 8 * ROWW * 2 : 0), 0, 0);
  };
  auto issue_tile = [&](int tile, int buf) {
    const auto rsrc = tile_rsrc(tile);
    static_for<0, 18>([&](auto kc) { issue_load(rsrc, buf, kc); });
  };

  // O^T accumulators: columns 128*wave + 32*cb + ..., rows 32*rb + l32
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  float m_ref = -INFINITY;   // softmax reference of the owned row (log2 domain)
  float l_sum = 0.f;         // sum of the owned row's (rounded) probabilities

  // score-phase read geometry: row l32 (and l32 + 32), chunk 2 ks + half; the
  // XOR pattern only touches the low 3 chunk bits, so 4 lane offsets cover all
  // 36 k-steps (the rest is an immediate offset)
  uint32_t qoff[4];
  {
    const int sw = chunk_swz(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i) qoff[i] = l32 * (CHUNKS * 16) + 16 * ((2 * i + half) ^ sw);
  }
  // value-phase transposed-read geometry: lane reads row 16 kap + 4 half +
  // rsel (+8), columns 128 wave + 32 cb + 16 grp + csel; the XOR pattern of
  // that row is lane-constant and only the parity of cb changes the swizzled
  // chunk, so two lane offsets cover every read
  uint32_t pvoff[2];
  {
    const int grp = (lane >> 4) & 1;
    const int rsel = (lane & 15) >> 2;
    const int csel = 4 * (lane & 3);
    const int trow = 4 * half + rsel;
    const int sw = chunk_swz(trow);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chunk = 16 * wave + 4 * i + 2 * grp + (csel >> 3);
      pvoff[i] = trow * (CHUNKS * 16) + 16 * (chunk ^ sw) + (csel & 7) * 2;
    }
  }
  const uint32_t pb_lane = pbuf_a + lane * 16;

  // zero both tile buffers once (LDS of rows past a sequence end stays finite)
  for (int i = tid; i < 2 * TILE_BYTES / 16; i += NTHREADS) ((i16x8*)smem)[i] = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
  barrier_lds();

  if (n_tiles > 0) issue_tile(0, 0);

  for (int tile = 0; tile < n_tiles; ++tile) {
    barrier_tile_ready();   // tile ready; every wave is past the previous value phase
    const bool has_next = tile + 1 < n_tiles;
    const auto next = tile_rsrc(has_next ? tile + 1 : tile);
    const int next_buf = (tile + 1) & 1;
    const uint32_t tb_a = smem_a + (tile & 1) * TILE_BYTES;
    const int ts = t_begin + tile * KT;

    // ================= score phase (owned rows) =================
    bf16x8 pk[2][2];
    if (wave_on) {
      f32x16 s0, s1;
      uint32_t qa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qa[i] = tb_a + qoff[i];
      i16x8 ra[4][2];
      auto issue_qk = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        lds_read_b128<128 * (ks >> 2)>(ra[ks & 3][0], qa[ks & 3]);
        lds_read_b128<128 * (ks >> 2) + 32 * CHUNKS * 16>(ra[ks & 3][1], qa[ks & 3]);
      };
      static_for<0, 3>(issue_qk);
      static_for<0, ROWW / 16>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int ahead = (ROWW / 16 - 1 - ks) < 3 ? (ROWW / 16 - 1 - ks) : 3;
        if constexpr (ks + 3 < ROWW / 16) issue_qk(std::integral_constant<int, ks + 3>{});
        // the next tile's loads ride along, one per two k-steps
        if constexpr (ks % 2 == 0) {
          if (has_next) issue_load(next, next_buf, std::integral_constant<int, ks / 2>{});
        }
        wait_lgkm<2 * ahead>(ra[ks & 3][0], ra[ks & 3][1]);
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra[ks & 3][0]);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra[ks & 3][1]);
        if constexpr (ks == 0) {
          mfma32_v0(s0, a0, qf[ks]);
          mfma32_v0(s1, a1, qf[ks]);
        } else {
          mfma32_v(s0, a0, qf[ks]);
          mfma32_v(s1, a1, qf[ks]);
        }
      });
      mfma_v_drain(s0, s1);

      // mask only where the tile reaches past a row's last visible row
      if (__builtin_amdgcn_ballot_w64(ts + KT > lim) != 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = ts + 8 * (r >> 2) + 4 * half + (r & 3);
          s0[r] = (t < lim) ? s0[r] : -INFINITY;
          s1[r] = (t + 32 < lim) ? s1[r] : -INFINITY;
        }
      }
      // running maximum on raw scores (the scale is positive)
      float mraw = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, fmaxf(s0[r], s1[r]));
      const float mx = max_halves(mraw) * p.scale_log2;
      int kstep = 0;
      if (m_ref == -INFINITY) {
        m_ref = mx;   // first visible scores: accumulators are still zero
      } else if (mx > m_ref + REF_STEP) {
        kstep = (int)ceilf((mx - m_ref - REF_STEP) * (1.0f / REF_STEP));
        if (kstep >= 7) {
          kstep = 7;          // everything so far is below 2^-448 of the new scale
          m_ref = mx;
          l_sum = 0.f;
        } else {
          m_ref += REF_STEP * kstep;
          l_sum *= __builtin_amdgcn_exp2f(-REF_STEP * kstep);
        }
      }
      const float nbase = (m_ref == -INFINITY) ? 0.f : -m_ref;
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const __bf16 p00 = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, nbase)));
        const __bf16 p01 = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], p.scale_log2, nbase)));
        const __bf16 p10 = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, nbase)));
        const __bf16 p11 = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], p.scale_log2, nbase)));
        pk[0][r >> 3][r & 7] = p00;
        pk[0][r >> 3][(r & 7) + 1] = p01;
        pk[1][r >> 3][r & 7] = p10;
        pk[1][r >> 3][(r & 7) + 1] = p11;
        ls += ((float)p00 + (float)p01) + ((float)p10 + (float)p11);
      }
      l_sum += sum_halves(ls);
      if (kstep != 0) {
        // sign bits of the fragment's first three probabilities carry the
        // reference step (both lane halves, so every reader lane sees it)
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (kstep & (1 << e)) pk[0][0][e] = -pk[0][0][e];
      }
    } else {
      if (has_next) static_for<0, 18>([&](auto kc) { issue_load(next, next_buf, kc); });
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) pk[i][j] = bf16x8{};
    }
    // P fragment (row block = wave, kappa = 2 sb + j) for lane
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        *(bf16x8*)(pbuf + ((wave * 4 + 2 * sb + j) * 64 + lane) * 16) = pk[sb][j];

    barrier_lds();   // probabilities of all 128 rows visible

    // ================= value phase (128 columns x all rows) =================
    {
      const uint32_t pa0 = tb_a + pvoff[0];
      const uint32_t pa1 = tb_a + pvoff[1];
      i16x8 bq[2][4];
      i16x4 tr[2][4][2];
      auto issue_pv = [&](auto kc) {
        constexpr int kap = decltype(kc)::value;
        constexpr int slot = kap & 1;
        static_for<0, 4>([&](auto rbc) {
          constexpr int rb = decltype(rbc)::value;
          lds_read_b128<(rb * 4 + kap) * 1024>(bq[slot][rb], pb_lane);
        });
        static_for<0, 4>([&](auto cbc) {
          constexpr int cb = decltype(cbc)::value;
          constexpr int off = 16 * kap * (CHUNKS * 16) + 128 * (cb >> 1);
          const uint32_t a = (cb & 1) ? pa1 : pa0;
          lds_read_tr16<off>(tr[slot][cb][0], a);
          lds_read_tr16<off + 8 * CHUNKS * 16>(tr[slot][cb][1], a);
        });
      };
      issue_pv(std::integral_constant<int, 0>{});
      static_for<0, 4>([&](auto kc) {
        constexpr int kap = decltype(kc)::value;
        constexpr int slot = kap & 1;
        wait_lgkm<0>(bq[slot][0], bq[slot][1], bq[slot][2], bq[slot][3],
                     tr[slot][0][0], tr[slot][0][1], tr[slot][1][0], tr[slot][1][1],
                     tr[slot][2][0], tr[slot][2][1], tr[slot][3][0], tr[slot][3][1]);
        if constexpr (kap + 1 < 4) issue_pv(std::integral_constant<int, kap + 1>{});
        if constexpr (kap == 0) {
          // reference steps of rows 32 rb + l32, carried in the sign bits of
          // the first three probabilities of the kappa = 0 fragment
          float alpha[4];
          bool any_step = false;
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            const uint32_t d0 = (uint32_t)__builtin_bit_cast(u32x4, bq[0][rb])[0];
            const uint32_t d1 = (uint32_t)__builtin_bit_cast(u32x4, bq[0][rb])[1];
            const int code = (int)(((d0 >> 15) & 1u) | ((d0 >> 30) & 2u) | ((d1 >> 13) & 4u));
            alpha[rb] = code == 0 ? 1.0f : (code == 7 ? 0.0f : __builtin_amdgcn_exp2f(-REF_STEP * code));
            any_step |= code != 0;
          }
          if (__builtin_amdgcn_ballot_w64(any_step) != 0) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
              for (int rb = 0; rb < 4; ++rb) scale_acc(acc[cb][rb], alpha[rb]);
          }
        }
        bf16x8 bb[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          u32x4 v = __builtin_bit_cast(u32x4, bq[slot][rb]);
          v &= 0x7FFF7FFFu;
          bb[rb] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const bf16x8 a = join_tr(tr[slot][cb][0], tr[slot][cb][1]);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) acc[cb][rb] = mfma32(a, bb[rb], acc[cb][rb]);
        }
      });
    }
  }

  // ---- epilogue: share each row's normaliser, write the normalised partials
  barrier_lds();
  float* const lsh = (float*)pbuf;          // [128] l_sum
  if (half == 0) lsh[wave * 32 + l32] = l_sum;
  barrier_lds();

  const int64_t pbase = ((int64_t)b * p.n_split + split) * D_C;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = g * 128 + rb * 32 + l32;
    if (row >= p.R) continue;
    const float l = lsh[rb * 32 + l32];
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = wave * 128 + cb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        p.part_o[(pbase + c) * p.R + row] = acc[cb][rb][r] * inv;
      }
    }
  }
  if (half == 0 && own_ok)
    p.part_lse[((int64_t)b * p.n_split + split) * p.R + own_r] =
        l_sum > 0.f ? m_ref + log2f(l_sum) : -INFINITY;
}

// Merge the split partials.  Work-group = 64 query rows x 64 latent columns
// of one sequence; thread (row, 16-column slice).  Weights 2^(lse_s - max).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      int B, int R, int n_split,
                                                      void* o_lat, int o_bf16, float* lse_out) {
  const int b = blockIdx.z;
  const int row = blockIdx.x * 64 + (threadIdx.x & 63);
  const int c0 = blockIdx.y * 64 + (threadIdx.x >> 6) * 16;
  if (row >= R) return;
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s)
    mx = fmaxf(mx, part_lse[((int64_t)b * n_split + s) * R + row]);
  float wsum = 0.f;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ls = part_lse[((int64_t)b * n_split + s) * R + row];
    if (ls == -INFINITY) continue;
    const float w = exp2f(ls - mx);
    wsum += w;
    const float* src = part_o + (((int64_t)b * n_split + s) * D_C + c0) * R + row;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += w * src[(int64_t)i * R];
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  const int64_t orow = (int64_t)b * R + row;
  if (o_bf16) {
    uint16_t* o = (uint16_t*)o_lat + orow * D_C + c0;
    i16x8 v0, v1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v0[i] = (short)bf16_bits(to_bf16(acc[i] * inv));
      v1[i] = (short)bf16_bits(to_bf16(acc[i + 8] * inv));
    }
    *(i16x8*)o = v0;
    *(i16x8*)(o + 8) = v1;
  } else {
    float* o = (float*)o_lat + orow * D_C + c0;
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *(f32x4*)(o + i) = f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
  }
  if (lse_out != nullptr && blockIdx.y == 0 && threadIdx.x < 64)
    lse_out[orow] = wsum > 0.f ? (mx + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_decode_split(const DecodeParams& p, hipStream_t stream) {
  const int grid = 8 * p.work_per_xcd;
  if (p.paged)
    hipLaunchKernelGGL(decode_split_bf16_kernel<true>, dim3(grid), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_bf16_kernel<false>, dim3(grid), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, int B, int R, int n_split,
                          void* o_lat, int o_bf16, float* lse, hipStream_t stream) {
  dim3 grid((R + 63) / 64, D_C / 64, B);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, part_o, part_lse, B, R, n_split,
                     o_lat, o_bf16, lse);
  return hipGetLastError();
}

}  // namespace mla
