// Split-T latent attention for absorbed MLA decode on gfx950, bf16 caches:
// score waves and value waves.
//
// The computation is that of decode_split_kernel ("MLA, dim by dim", section
// "MLA Decode"; "Why MLA and MTP Fight Each Other", sections 4.2 and 8): every
// query row (head x query token) scores its 576-wide latent query against the
// shared cached rows, softmaxes, and averages the rows' 512 latent columns.
// Each 32-row latent tile is read once from memory into LDS, where it serves
// both contractions for the 64 query rows of the work-group.
//
// Why two kinds of waves.  The latent queries of a row group (64 rows x 576
// bf16, 72 KB) and the fp32 output accumulators (64 rows x 512, 128 KB) fit
// the register file of a compute unit with room for two waves per SIMD, so
// that one wave's softmax arithmetic runs while the other wave's matrix
// products keep the matrix cores busy:
//   waves 0-3, score waves: wave s holds the latent queries of rows
//     32 (s & 1) .. +31 and scores them against tile rows 16 (s >> 1) .. +15
//     (MFMA 16x16x32, the tile fragment from LDS, the queries in registers),
//     runs the softmax of those scores and writes the bf16 probabilities to
//     LDS in the value product's operand layout;
//   waves 4-7, value waves: wave v accumulates O^T for latent columns
//     128 v .. +127 and all 64 rows (MFMA 32x32x16, the tile read transposed
//     from LDS, the probabilities from LDS) and issues the tile loads.
// The two kinds work one tile apart between barriers: in interval k the score
// waves take tile k + 1 while the value waves take tile k, and the loads of
// tile k + 3 are issued; a ring of four tile buffers gives each tile two
// intervals in flight.
//
// Softmax references.  Each row's probabilities of a tile are taken against a
// reference 64 K (log2 units, K an integer) that only rises: it is set from
// the first visible scores (K = ceil(max / 64), so the largest probability is
// in (2^-64, 1]) and raised when a tile's maximum passes 64 K + 64.  The two
// score waves of a row (the two halves of each tile) take the larger of their
// own and the other's last K, so they agree after a change within one tile.
// Every (row, tile half) publishes its K beside the probabilities; a value
// wave holding a smaller K for the row rescales its accumulators by 2^(-64 d),
// and probabilities published with a smaller K than the accumulators' are
// scaled down by 2^(-64 d) before the product.  K can move by several steps
// at once (the maximum only has to pass the next multiple of 64), so these
// powers of two are applied to the values with ldexp: 2^-128 itself is an
// fp32 denormal and would flush to zero.  Each score wave sums its own
// rounded probabilities per row; the sums of the two halves are brought to
// the accumulators' K at the end.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_plan.h"

namespace mla {

namespace {

constexpr int NT = 512;                        // threads: 4 score waves + 4 value waves
constexpr int G = 64;                          // query rows per work-group
constexpr int KT = 32;                         // cached rows per LDS tile
constexpr int NB = 4;                          // tile buffers (ring)
constexpr int CHUNKS = ROWW * 2 / 16;          // 72 16-byte chunks per bf16 row
constexpr int ROWB = ROWW * 2;                 // 1152 bytes per row
constexpr int TILE_BYTES = KT * ROWB;          // 36,864
constexpr int P_BYTES = G * KT * 2;            // 4 KB: bf16 probabilities of one tile
constexpr int CODE_BYTES = 2 * G * 4;          // int32 K per (tile half, row)
constexpr int P_OFF = NB * TILE_BYTES;
constexpr int CODE_OFF = P_OFF + 2 * P_BYTES;
constexpr int SMEM_BYTES = CODE_OFF + 2 * CODE_BYTES;
constexpr int LOADS = 9;                       // 1 KB loads per value wave per tile (8 rows)
constexpr int K_NONE = -(1 << 24);             // no visible score yet
constexpr float REF_STEP = 64.0f;
constexpr int REF_SHIFT = 64;                  // the same step as a power of two
constexpr int STAGE_PITCH_B16 = D_C * 2 + 16;  // staged partial row (bf16), padded
constexpr int STAGE_PITCH_F32 = D_C * 4 + 16;  // staged partial row (fp32), padded
static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget");
static_assert((2 * NT + 4) * 8 <= P_OFF, "plan scratch fits the tile buffers");
static_assert(G * STAGE_PITCH_F32 <= P_OFF, "partial staging fits the tile buffers");

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Score product, accumulated in registers the softmax reads right after.
// (This file is compiled with every MFMA operand in VGPRs: one pool of 256
// registers per wave holds either the score waves' latent queries or the
// value waves' accumulators.)  The hazard recognizer does not see inside
// inline asm: after the last of these, drain16() before any other
// instruction reads the accumulators.  Back-to-back MFMAs into the same
// accumulator need no wait states.
__device__ __forceinline__ void mfma16_v0(f32x4_t& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v(f32x4_t& c, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void drain16(f32x4_t& c0, f32x4_t& c1) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}

// lanes l, l ^ 16, l ^ 32 and l ^ 48 hold the same query row: reduce over
// them.  v_permlane16_swap exchanges the odd 16-lane rows of one register with
// the even rows of another, v_permlane32_swap the upper half with the lower;
// swapping a value with a copy of itself leaves {x[l], x[l ^ 16]} (then
// {x[l], x[l ^ 32]}) in the two registers.  s_nop: VALU-write ->
// permlane-read and permlane-write -> VALU-read hazards.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max4rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum4rows(float x) {
  float a = x, b = x;
  swap16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap32(a, b);
  return a + b;
}

// acc *= 2^n.  The references move in whole steps of 2^64 and may move by
// several at once: a factor of 2^-128 is an fp32 denormal (flushed to 0),
// while the scaled values are not, so the exponent is applied to each value
// (v_ldexp_f32).
__device__ __forceinline__ void ldexp_acc(f32x16& acc, int n) {
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_ldexpf(acc[i], n);
}

__device__ __forceinline__ int lds_read_i32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

template <bool PAGED>
__global__ __launch_bounds__(NT, 1) void decode_sv_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  const uint32_t smem_a = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int b, j, parts, sl, g;
  if (!plan_work_t<NT>(p, (int64_t*)smem, b, j, parts, sl, g)) return;   // surplus work-group
  const int T = p.seqlens[b];
  const int nt_b = (T + PLAN_TILE - 1) / PLAN_TILE;
  const int t_begin = (int)floor_div((int64_t)j * nt_b, parts) * PLAN_TILE;
  const int t_end = min(T, (int)floor_div((int64_t)(j + 1) * nt_b, parts) * PLAN_TILE);
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + KT - 1) / KT : 0;

  int* const codes = (int*)(smem + CODE_OFF);     // [2 slots][2 halves][64 rows]
  for (int i = tid; i < 2 * 2 * G; i += NT) codes[i] = K_NONE;

  const bool is_score = wave < 4;
  const char* rows = (const char*)p.rows;

  if (is_score) {
    // ======================= score waves =======================
    const int s_rb = wave & 1, s_th = wave >> 1;
    const int q4 = lane >> 4, l16 = lane & 15;
    int lim[2];
    bf16x8 qf[ROWW / 32][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = g * G + s_rb * 32 + nb * 16 + l16;
      const bool ok = r < p.R;
      const int jq = ok ? r / p.H : 0;
      lim[nb] = ok ? min(p.causal ? T - p.s_q + jq + 1 : T, t_end) : 0;
      const uint16_t* qrow = p.q_lat + ((int64_t)b * p.R + (ok ? r : 0)) * ROWW + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < ROWW / 32; ++ks) {
        i16x8 v = *(const i16x8*)(qrow + 32 * ks);
        if (!ok) v = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
        qf[ks][nb] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // score fragment reads: tile row 16 th + l16, logical chunk 4 ks + q4.
    // The XOR swizzle only touches the low 3 chunk bits, so k-steps 2m and
    // 2m + 1 use two lane offsets and m is an immediate (128 m bytes).
    const int t_s = s_th * 16 + l16;
    uint32_t aoff[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) aoff[bb] = t_s * ROWB + 16 * ((4 * bb + q4) ^ tile_swz(t_s));
    // probability writes: this lane's 4 scores of row nb * 16 + l16 (tile
    // rows 16 th + 4 q4 + e) go to the value product's B fragment of (half th,
    // row block rb): lane (row % 32) + 32 (q4 & 1), elements 4 (q4 >> 1) + e
    const uint32_t pw_off = (uint32_t)(((s_th * 2 + s_rb) * 64 + l16 + 32 * (q4 & 1)) * 16 + 8 * (q4 >> 1));
    const uint32_t p_base = smem_a + P_OFF;
    const uint32_t code_base = smem_a + CODE_OFF;
    int k_own[2] = {K_NONE, K_NONE};
    float l_own[2] = {0.f, 0.f};
    // every real row sees at least its first lim_lo rows (rows past the
    // query count never reach the output, so they need no mask)
    const int lim_lo = min(p.causal ? T - p.s_q + 1 : T, t_end);
    __syncthreads();                              // codes initialised; tile 0 issued by the value waves
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // latent queries in registers
    __syncthreads();                              // tile 0 in LDS
    for (int i = 0; i <= n_tiles; ++i) {          // interval i - 1: tile i
      if (i < n_tiles) {
        const uint32_t tb_a = smem_a + (i & (NB - 1)) * TILE_BYTES;
        // the other half's K for these rows at the previous tile
        const uint32_t cprev = code_base + ((i + 1) & 1) * CODE_BYTES + (1 - s_th) * G * 4;
        const int kp0 = lds_read_i32(cprev + (s_rb * 32 + l16) * 4);
        const int kp1 = lds_read_i32(cprev + (s_rb * 32 + 16 + l16) * 4);
        f32x4_t sc[2];
        // a k-step is two 16-cycle products: keep seven fragment reads in
        // flight to cover the LDS latency
        constexpr int AHEAD = 7;
        i16x8 ra[AHEAD + 1];
        auto issue = [&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          lds_read_b128<128 * (ks >> 1)>(ra[ks % (AHEAD + 1)], tb_a + aoff[ks & 1]);
        };
        static_for<0, AHEAD>(issue);
        static_for<0, ROWW / 32>([&](auto kc) {
          constexpr int ks = decltype(kc)::value;
          constexpr int ahead = (ROWW / 32 - 1 - ks) < AHEAD ? (ROWW / 32 - 1 - ks) : AHEAD;
          if constexpr (ks + AHEAD < ROWW / 32) issue(std::integral_constant<int, ks + AHEAD>{});
          wait_lgkm<ahead>(ra[ks % (AHEAD + 1)]);
          const bf16x8 a = __builtin_bit_cast(bf16x8, ra[ks % (AHEAD + 1)]);
          if constexpr (ks == 0) {
            mfma16_v0(sc[0], a, qf[ks][0]);
            mfma16_v0(sc[1], a, qf[ks][1]);
          } else {
            mfma16_v(sc[0], a, qf[ks][0]);
            mfma16_v(sc[1], a, qf[ks][1]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        drain16(sc[0], sc[1]);
        // mask (only where the tile reaches past the first row's last
        // visible position), reference, probabilities
        int kp[2] = {kp0, kp1};
        wait_lgkm<0>(kp[0], kp[1]);                 // (complete already: the last k-step waited for all)
        const int ts = t_begin + i * KT;
        if (ts + KT > lim_lo) {
          const int t0 = ts + s_th * 16 + 4 * q4;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[nb][e] = (t0 + e < lim[nb]) ? sc[nb][e] : -INFINITY;
        }
        uint64_t pw[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          // the reference moves only when a score passes 64 (K + 1) (or on
          // the first visible score): a per-lane test, then the row maximum
          // across the four lanes of the row in the rare case it is needed
          int k = max(k_own[nb], kp[nb]);
          const float ml = fmaxf(fmaxf(sc[nb][0], sc[nb][1]), fmaxf(sc[nb][2], sc[nb][3])) * p.scale_log2;
          const bool move = ml > -INFINITY && (k == K_NONE || ml > REF_STEP * (float)k + REF_STEP);
          if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m = max4rows(ml);
            if (m > -INFINITY && (k == K_NONE || m > REF_STEP * (float)k + REF_STEP))
              k = (int)ceilf(m * (1.0f / REF_STEP));
          }
          if (k != k_own[nb]) {
            l_own[nb] = k_own[nb] == K_NONE ? 0.f : __builtin_amdgcn_ldexpf(l_own[nb], -REF_SHIFT * (k - k_own[nb]));
            k_own[nb] = k;
          }
          const float nbase = k == K_NONE ? 0.f : -REF_STEP * (float)k;
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[nb][e], p.scale_log2, nbase));
          pw[nb] = pack_bf16x4(pv);
          // sum of the rounded probabilities, two at a time
          const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
          l_own[nb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)pw[nb]), ones, l_own[nb], false);
          l_own[nb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, (uint32_t)(pw[nb] >> 32)), ones, l_own[nb], false);
        }
        const uint32_t pslot = p_base + (i & 1) * P_BYTES + pw_off;
        asm volatile("ds_write_b64 %0, %1" ::"v"(pslot), "v"(pw[0]) : "memory");
        asm volatile("ds_write_b64 %0, %1 offset:256" ::"v"(pslot), "v"(pw[1]) : "memory");
        if (q4 == 0) {
          const uint32_t cw = code_base + (i & 1) * CODE_BYTES + s_th * G * 4 + (s_rb * 32 + l16) * 4;
          asm volatile("ds_write_b32 %0, %1" ::"v"(cw), "v"(k_own[0]) : "memory");
          asm volatile("ds_write_b32 %0, %1 offset:64" ::"v"(cw), "v"(k_own[1]) : "memory");
        }
      }
      barrier_lds();
    }
    // epilogue: per-row sums of the rounded probabilities of this half, and
    // the K they are counted against
    barrier_tile_ready();
    float* const lsh = (float*)(smem + P_OFF);    // [2 halves][64 rows] sums
    int* const ksh = (int*)(smem + P_OFF + 2 * G * 4);   // [2 halves][64 rows] K
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float l = sum4rows(l_own[nb]);
      if (q4 == 0) {
        lsh[s_th * G + s_rb * 32 + nb * 16 + l16] = l;
        ksh[s_th * G + s_rb * 32 + nb * 16 + l16] = k_own[nb];
      }
    }
    barrier_lds();
    barrier_lds();                                // value waves stage the partial rows
  } else {
    // ======================= value waves =======================
    const int v = wave - 4;
    // ---- tile loads: value wave v copies tile rows 8 v .. 8 v + 7, 9 loads
    // of 64 lanes x 16 B, each filling 1 KB of LDS in order; the chunk lane l
    // fetches for LDS slot 64 k + l follows the XOR swizzle of its row.
    uint32_t loff[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int s = 64 * k + lane;
      const int tl = s / CHUNKS;
      const int c = (s - tl * CHUNKS) ^ tile_swz(8 * v + tl);
      loff[k >> 1] |= (uint32_t)(tl * ROWB + c * 16) << (16 * (k & 1));
    }
    const int soff = v * 8 * ROWB;
    auto tile_rsrc = [&](int tile) {
      const int ts = t_begin + tile * KT;
      const bool live = tile < n_tiles;
      const int valid = live ? min(KT, T - ts) : 0;
      int64_t base;
      if (PAGED) base = live ? (int64_t)p.block_table[(int64_t)b * p.max_blocks + (ts >> 6)] * PLAN_TILE + (ts & 63) : 0;
      else base = (int64_t)b * p.T_stride + (live ? ts : 0);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(rows + base * ROWB), (short)0, valid * ROWB, 0x00020000);
    };
    // (the buffer resource is passed by value: the host pass cannot form a
    // reference to it)
    auto issue_load = [&](__amdgpu_buffer_rsrc_t rsrc, char* dst, auto kc) {
      constexpr int k = decltype(kc)::value;
      const uint32_t vo = (loff[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + k * 1024), 16, vo, soff, 0, 0);
    };
    auto issue_tile = [&](int tile) {
      const auto rsrc = tile_rsrc(tile);
      char* const dst = smem + (tile & (NB - 1)) * TILE_BYTES + soff;
      static_for<0, LOADS>([&](auto kc) { issue_load(rsrc, dst, kc); });
    };
    // ---- transposed reads of the value product: lane reads tile row
    // 16 kap + 4 half + rsel (+ 8), columns 128 v + 32 cb + 16 grp + csel; only
    // the parity of cb changes the swizzled chunk, so four lane offsets cover
    // every read (cb >> 1 is an immediate of 128 bytes)
    uint32_t pvoff[2][2];
    {
      const int half = lane >> 5, grp = (lane >> 4) & 1;
      const int rsel = (lane & 15) >> 2, csel = 4 * (lane & 3);
      const int trow = 4 * half + rsel;
#pragma unroll
      for (int r8 = 0; r8 < 2; ++r8) {
        const int sw = tile_swz(trow + 8 * r8);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int chunk = 16 * v + 4 * i + 2 * grp + (csel >> 3);
          pvoff[r8][i] = trow * ROWB + 16 * (chunk ^ sw) + (csel & 7) * 2;
        }
      }
    }
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 2; ++r) acc[i][r] = f32x16{};
    int k_acc[2] = {K_NONE, K_NONE};             // accumulators' K for rows 32 rb + lane % 32
    const uint32_t p_base = smem_a + P_OFF + lane * 16;
    const uint32_t code_base = smem_a + CODE_OFF + (lane & 31) * 4;

    issue_tile(0);
    issue_tile(1);
    __syncthreads();                              // codes initialised
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");   // tile 0 (tile 1 in flight)
    __syncthreads();                              // tile 0 in LDS
    for (int i = 0; i <= n_tiles; ++i) {          // interval i - 1: values of tile i - 1
      issue_tile(i + 2);
      const int k = i - 1;
      if (k >= 0) {
        const uint32_t tb_a = smem_a + (k & (NB - 1)) * TILE_BYTES;
        const uint32_t pb = p_base + (k & 1) * P_BYTES;
        const uint32_t cb_a = code_base + (k & 1) * CODE_BYTES;
        i16x8 bq[2][2];
        int cd[2][2];
        static_for<0, 2>([&](auto kc) {
          constexpr int kap = decltype(kc)::value;
          static_for<0, 2>([&](auto rc) {
            constexpr int rb = decltype(rc)::value;
            lds_read_b128<(kap * 2 + rb) * 1024>(bq[kap][rb], pb);
          });
        });
#pragma unroll
        for (int kap = 0; kap < 2; ++kap)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) cd[kap][rb] = lds_read_i32(cb_a + kap * G * 4 + rb * 128);
        constexpr int TR = 4;                     // transposed fragments in a ring, TR - 1 ahead
        i16x4 tr[TR][2];
        auto issue_a = [&](auto uc) {
          constexpr int u = decltype(uc)::value;
          constexpr int kap = u >> 2, cb = u & 3;
          constexpr int off = 16 * kap * ROWB + 128 * (cb >> 1);
          lds_read_tr16<off>(tr[u % TR][0], tb_a + pvoff[0][cb & 1]);
          lds_read_tr16<off + 8 * ROWB>(tr[u % TR][1], tb_a + pvoff[1][cb & 1]);
        };
        static_for<0, TR - 1>([&](auto uc) { issue_a(uc); });
        // everything above is in flight: the probability and K reads (4 + 4)
        // are older than the first fragments' (2 (TR - 1))
        wait_lgkm<2 * (TR - 1)>(bq[0][0], bq[0][1], bq[1][0], bq[1][1], cd[0][0], cd[0][1], cd[1][0], cd[1][1]);
        // softmax references (rare: the first tile and when scores jump):
        // the accumulators move to the largest K published for the row, and
        // a half published with a smaller K is scaled down to it
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int c0 = cd[0][rb], c1 = cd[1][rb];
          int kn = k_acc[rb];
          if (c0 != K_NONE) kn = max(kn, c0);
          if (c1 != K_NONE) kn = max(kn, c1);
          const bool need = kn != k_acc[rb] || (c0 != K_NONE && c0 != kn) || (c1 != K_NONE && c1 != kn);
          if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const int na = (k_acc[rb] == K_NONE) ? 0 : -REF_SHIFT * (kn - k_acc[rb]);
#pragma unroll
            for (int cbi = 0; cbi < 4; ++cbi) ldexp_acc(acc[cbi][rb], na);
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
              const int c = cd[kap][rb];
              const int nbeta = (c == K_NONE) ? 0 : -REF_SHIFT * (kn - c);
              bf16x8 pb8 = __builtin_bit_cast(bf16x8, bq[kap][rb]);
#pragma unroll
              for (int e = 0; e < 8; ++e) pb8[e] = to_bf16(__builtin_amdgcn_ldexpf((float)pb8[e], nbeta));
              bq[kap][rb] = __builtin_bit_cast(i16x8, pb8);
            }
            k_acc[rb] = kn;
          }
        }
        static_for<0, 8>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          constexpr int kap = u >> 2, cb = u & 3;
          // fragments issued after this one: min(TR - 2, 7 - u) units
          constexpr int younger = (7 - u) < (TR - 2) ? (7 - u) : (TR - 2);
          wait_lgkm<2 * younger>(tr[u % TR][0], tr[u % TR][1]);
          if constexpr (u + TR - 1 < 8) issue_a(std::integral_constant<int, u + TR - 1>{});
          const bf16x8 a = join_tr(tr[u % TR][0], tr[u % TR][1]);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[cb][rb] = mfma32(a, __builtin_bit_cast(bf16x8, bq[kap][rb]), acc[cb][rb]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // tile i + 1 landed (the 9 loads of tile i + 2 may still be in flight)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      barrier_lds();
    }
    barrier_tile_ready();                         // every load landed: the tile buffers are free
    barrier_lds();                                // the score waves' sums and K are in LDS
    const float* const lsh = (const float*)(smem + P_OFF);
    const int* const ksh = (const int*)(smem + P_OFF + 2 * G * 4);
    const bool pb16 = p.part_bf16 != 0;
    const int pitch = pb16 ? STAGE_PITCH_B16 : STAGE_PITCH_F32;
    const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = rb * 32 + l32;
      float l = 0.f;
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int kt = ksh[th * G + r];
        const float lt = lsh[th * G + r];
        if (kt != K_NONE && lt > 0.f) l += __builtin_amdgcn_ldexpf(lt, REF_SHIFT * (kt - k_acc[rb]));
      }
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      char* const srow = smem + r * pitch;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = v * 128 + cb * 32 + 8 * q + 4 * half;
          const f32x4 val = {acc[cb][rb][4 * q] * inv, acc[cb][rb][4 * q + 1] * inv, acc[cb][rb][4 * q + 2] * inv,
                             acc[cb][rb][4 * q + 3] * inv};
          if (pb16) *(uint64_t*)(srow + col * 2) = pack_bf16x4(val);
          else *(f32x4*)(srow + col * 4) = val;
        }
      const int row = g * G + r;
      if (v == 0 && half == 0 && row < p.R)
        p.part_lse[(int64_t)sl * p.R + row] = l > 0.f ? REF_STEP * (float)k_acc[rb] + log2f(l) : -INFINITY;
    }
    barrier_lds();
  }
  // ---- every wave writes whole staged partial rows: wave w rows w, w + 8, ...
  const bool pb16 = p.part_bf16 != 0;
  const int n_rows = min(G, p.R - g * G);
  const int64_t prow0 = (int64_t)sl * p.R + g * G;
  if (pb16) {
    uint16_t* const dst = (uint16_t*)p.part_o + prow0 * D_C + lane * 8;
    for (int r = wave; r < n_rows; r += 8) {
      const u32x4 val = *(const u32x4*)(smem + r * STAGE_PITCH_B16 + lane * 16);
      *(u32x4*)(dst + (int64_t)r * D_C) = val;
    }
  } else {
    float* const dst = (float*)p.part_o + prow0 * D_C + lane * 4;
    for (int r = wave; r < n_rows; r += 8) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 val = *(const u32x4*)(smem + r * STAGE_PITCH_F32 + h2 * 1024 + lane * 16);
        *(u32x4*)(dst + (int64_t)r * D_C + h2 * 256) = val;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_sv(const DecodeParams& p, hipStream_t stream) {
  const int grid = 8 * p.work_per_xcd;
  if (p.paged)
    hipLaunchKernelGGL((decode_sv_kernel<true>), dim3(grid), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_sv_kernel<false>), dim3(grid), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
