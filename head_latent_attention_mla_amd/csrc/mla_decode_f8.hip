// Split-T latent attention with FP8 arithmetic for an FP8 (E4M3) latent
// cache: the cached codes feed the matrix cores directly, the latent queries
// and the probabilities are quantised to E4M3 too, and the per-row scales are
// applied outside the products ("Decode attention intensity is fixed at the
// query-to-KV head ratio...", "A strong answer" and "What interviewers probe
// next": FP8 halves the cache bytes, and with FP8 arithmetic the path is
// priced against the FP8 ridge instead of the bf16 one).
//
// Same work plan, tiling and partial-output format as decode_split_kernel
// (the merge kernels are shared).  Per 64-row tile, on the MFMA
// v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate):
//   scores   S8^T[t][row] = sum_k code_t[k] * q8_row[k]   (9 k-steps of 64)
//            s = S8 * sigma_t * qscale_row * softmax_scale
//   values   O^T[c][row] += sum_t code_t[c] * w8[t][row], one k-step of 64 rows
//            w = p * sigma_t * 2^-e, quantised to E4M3; the row normaliser sums
//            the weights actually used, dequant(w8) / (sigma_t 2^-e), so a row
//            of few cached rows stays normalised
// A query row whose largest probability is more than 1/32 of its total (few
// rows, or a peaked softmax) does not average out the E4M3 rounding of its
// weights and query: each part records its rows' maximum scores, and the
// bf16-arithmetic scan then recomputes the (sequence, row group) pairs that
// hold such a row.
// q8 = E4M3(q_lat / qscale_row), qscale_row = amax|q_lat row| / 448.  The
// exponent e is this work-group's running max of ceil(log2 sigma), so w <= 2^8
// (the softmax reference moves in steps of 2^8 here); when it grows the
// accumulators are rescaled by the exact power of two.  The epilogue
// multiplies by 2^e before normalising.
//
// LDS tile layout: 64 rows x 36 chunks of 16 B (576 B rows), written by
// direct loads with the chunk index XOR-swizzled per row so that both the
// score reads (128-bit reads, 16 lanes = 16 rows per pass over 64 banks of
// 256 B) and the transposed 8-bit reads of the value product
// (ds_read_b64_tr_b8: 32 lanes per pass read 2 chunks of rows b .. b + 3 and
// b + 8 .. b + 11) hit distinct banks.  A 576-byte row starts 64 B further
// into the 256-byte bank row than the one before; the swizzle compensates.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_split_store.h"
#include "mla_plan.h"

namespace mla {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int KT = 64;                         // cached rows per tile
constexpr int NTHREADS = 256;
constexpr int STAGE = KT * ROWW;               // 36,864: e4m3 codes of one tile
constexpr int PB_BYTES = 4 * 64 * 32;          // e4m3 probability fragments of 128 rows
constexpr int SC_BYTES = 2 * KT * 4;           // row scales of one tile and their reciprocals
constexpr float REF_STEP = 8.0f;               // probabilities stay <= 2^8 (E4M3 max 448)
constexpr int E_NONE = -100000;                // no scale seen yet
static_assert(PB_BYTES >= PLAN_SCRATCH_BYTES, "plan scratch");
constexpr int MAIN_BYTES = 2 * STAGE + PB_BYTES + 2 * SC_BYTES;
// the partial rows are staged over the whole buffer at the end, with the
// row normalisers past them
constexpr int SMEM_BYTES = MAIN_BYTES > SPLIT_STAGE_BYTES + 512 ? MAIN_BYTES : SPLIT_STAGE_BYTES + 512;
static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget");

// chunk XOR pattern of tile row t: the 16-byte bank slot of (row t, physical
// chunk p) is 4 (t & 3) + p (mod 16), so rows t .. t + 3 already fall in
// different quarters and the XOR (t >> 2) & 3 separates the four such groups
// of an aligned run of 16 rows (score reads); for the transposed reads rows
// b .. b + 3 and b + 8 .. b + 11 differ in XOR bit 1.  Period 16, so row
// offsets of 16 and 32 are immediates.
__device__ __forceinline__ int f8_swz(int t) { return (t >> 2) & 3; }
// logical -> physical chunk of row t (an involution per row); the four rope
// chunks 32..35 stay among themselves
__device__ __forceinline__ int f8_chunk(int t, int c) {
  return c < 32 ? (c ^ f8_swz(t)) : 32 + ((c - 32) ^ (f8_swz(t) & 3));
}

__device__ __forceinline__ f32x16 mfma8(v8i a, v8i b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int OFF>
__device__ __forceinline__ void lds_read_tr8(v2i& d, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "i"(OFF));
}

// four non-negative values (<= 448) -> four E4M3 codes, round to nearest even
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <bool PAGED>
__global__ __launch_bounds__(NTHREADS, 1) void decode_split_f8_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
  char* const pbuf = smem + 2 * STAGE;
  float* const scl = (float*)(smem + 2 * STAGE + PB_BYTES);   // per buffer: 64 scales, then 64 reciprocals
  const uint32_t smem_a = lds_addr(smem);
  const uint32_t pbuf_a = smem_a + 2 * STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int b, j, parts, sl, g;
  if (!plan_work(p, (int64_t*)pbuf, b, j, parts, sl, g)) return;   // surplus work-group
  const int nt_b = (p.seqlens[b] + KT - 1) / KT;
  // (all uniform: kept in scalar registers, as the tile loads' buffer
  // windows must be)
  const int T = __builtin_amdgcn_readfirstlane(p.seqlens[b]);
  const int t_begin = __builtin_amdgcn_readfirstlane((int)floor_div((int64_t)j * nt_b, parts) * KT);
  const int t_end = __builtin_amdgcn_readfirstlane(min(T, (int)floor_div((int64_t)(j + 1) * nt_b, parts) * KT));
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + KT - 1) / KT : 0;

  // ---- own query row; its latent query quantised to E4M3 with a row scale
  const int own_r = g * 128 + wave * 32 + l32;
  const bool own_ok = own_r < p.R;
  const bool wave_on = g * 128 + wave * 32 < p.R;
  const int jq = own_ok ? own_r / p.H : 0;
  const int visible = p.causal ? (T - p.s_q + jq + 1) : T;
  const int lim = min(visible, t_end);

  v8i q8[ROWW / 64];
  float c_row;          // qscale * softmax_scale * log2(e)
  {
    // lane (row, half h) holds k = 64 ks + 32 h + e, e < 32, of each k-step
    const uint16_t* qrow = p.q_lat + ((int64_t)b * p.R + (own_ok ? own_r : 0)) * ROWW + 32 * half;
    float amax = 0.f;
    for (int ks = 0; ks < ROWW / 64; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i16x8 v = *(const i16x8*)(qrow + 64 * ks + 8 * u);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf16_bits_to_float((uint16_t)v[e])));
      }
    amax = own_ok ? fmaxf(amax, __shfl_xor(amax, 32, 64)) : 0.f;
    const float qs = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
    const float inv = 1.0f / qs;
    c_row = qs * p.scale_log2;
#pragma unroll
    for (int ks = 0; ks < ROWW / 64; ++ks) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i16x8 v = *(const i16x8*)(qrow + 64 * ks + 8 * u);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = own_ok ? bf16_bits_to_float((uint16_t)v[e]) * inv : 0.f;
          f[e] = fminf(fmaxf(x, -448.0f), 448.0f);
        }
        // signed values: the conversion keeps the sign
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
        q8[ks][2 * u] = w0;
        q8[ks][2 * u + 1] = w1;
      }
    }
  }

  // ---- tile loader: wave w copies rows 16 w .. 16 w + 15 (9 KB, 9 loads of
  // 1 KB); LDS slot 64 k + lane holds the swizzled chunk this lane fetches
  uint32_t loff[5] = {0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int s = 64 * k + lane;
    const int tl = s / 36;
    const int c = f8_chunk(tl, s - tl * 36);
    loff[k >> 1] |= (uint32_t)(tl * ROWW + c * 16) << (16 * (k & 1));
  }
  const char* rows = (const char*)p.rows;
  auto tile_base = [&](int tile) -> int64_t {   // row index of the tile's first row
    const int ts = t_begin + tile * KT;
    // (the table entry moved to a scalar register: a buffer resource must be uniform)
    if (PAGED) return (int64_t)__builtin_amdgcn_readfirstlane(p.block_table[(int64_t)b * p.max_blocks + (ts >> 6)]) * KT;
    return (int64_t)b * p.T_stride + ts;
  };
  const int soff = wave * (16 * ROWW);
  // the buffer window of a tile; past the last tile an empty window, so its
  // loads fetch nothing (they write zeros into the idle buffer)
  auto tile_rsrc = [&](int tile, bool real) {
    const int ts = t_begin + tile * KT;
    const int valid = real ? __builtin_amdgcn_readfirstlane(min(KT, T - ts)) : 0;
    const int64_t base = real ? tile_base(tile) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(rows + base * ROWW), (short)0, valid * ROWW, 0x00020000);
  };
  auto issue_load = [&](__amdgpu_buffer_rsrc_t rsrc, int buf, auto kc) {   // load k of this wave's nine
    constexpr int k = decltype(kc)::value;
    const uint32_t vo = (loff[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
    char* dst = smem + buf * STAGE + wave * (16 * ROWW);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + k * 1024), 16, vo, soff, 0, 0);
  };
  auto issue_tile = [&](int tile, int buf) {
    const auto rsrc = tile_rsrc(tile, true);
    static_for<0, 9>([&](auto kc) { issue_load(rsrc, buf, kc); });
  };
  auto load_scale = [&](int tile) -> float {   // threads 0..63: the scale of tile row tid
    const int ts = t_begin + tile * KT;
    return (tid < KT && ts + tid < T) ? p.row_scale[tile_base(tile) + tid] : 0.f;
  };

  // ---- read geometry.  Scores: row l32 (+ 32), logical chunks 4 ks + 2 h + u.
  const int swz_r = f8_swz(l32);
  uint32_t so[2][2], sr[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int u = 0; u < 2; ++u) so[a][u] = l32 * ROWW + 16 * ((4 * a + 2 * half + u) ^ swz_r);
#pragma unroll
  for (int u = 0; u < 2; ++u) sr[u] = l32 * ROWW + 16 * (32 + ((2 * half + u) ^ (swz_r & 3)));
  // values: lane (16-lane group: s = lane % 16, grp = lane / 16 % 2) points at
  // row 8 (e / 4) + 4 h + e % 4 (e = s / 2), bytes 8 (s % 2) of logical chunk
  // 8 wave + 2 cb + grp; read j adds 16 j rows.  Lane c then receives column
  // 32 cb + c of the rows t = 16 j + 8 (i / 4) + 4 h + i % 4, i = byte 0..7,
  // which is the k order of its probability fragment
  uint32_t tro[4];
  {
    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    const int e = s16 >> 1;
    const int rl = 8 * (e >> 2) + 4 * half + (e & 3);
    const int sw = f8_swz(rl);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
      tro[cb] = rl * ROWW + 16 * (8 * wave + ((2 * cb + grp) ^ sw)) + 8 * (s16 & 1);
  }
  const uint32_t pb_lane = pbuf_a + lane * 32;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] = f32x16{};
  float m_ref = -INFINITY;
  float l_sum = 0.f;
  float m_run = -INFINITY;   // running maximum of the row's scaled scores (log2 domain)
  int e_cur = E_NONE;

  float sc_next = 0.f;
  if (n_tiles > 0) {
    issue_tile(0, 0);
    const float s0v = load_scale(0);
    if (tid < KT) {
      scl[tid] = s0v;
      scl[KT + tid] = s0v > 0.f ? 1.0f / s0v : 0.f;
    }
  }

  for (int tile = 0; tile < n_tiles; ++tile) {
    barrier_tile_ready();   // codes and scales of this tile in LDS; the other buffers are free
    const bool has_next = tile + 1 < n_tiles;
    // the next tile's scales now, its codes one load per score k-step below
    // (a burst of direct loads stalls the issuing wave)
    if (has_next) sc_next = load_scale(tile + 1);
    const auto next = tile_rsrc(tile + 1, has_next);
    const int next_buf = (tile + 1) & 1;
    const uint32_t tb = smem_a + (tile & 1) * STAGE;
    const float* sct = scl + (tile & 1) * 2 * KT;
    const int ts = t_begin + tile * KT;

    // this lane's 32 row scales (rows 32 sb + 8 gq + 4 h + i): read now, used
    // after the score products are issued
    f32x4 sig[2][4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) sig[sb][gq] = *(const f32x4*)(sct + 32 * sb + 8 * gq + 4 * half);

    // ================= score phase (owned rows) =================
    uint32_t pw[8];                        // this lane's 32 E4M3 weights (fragment bytes)
    f32x16 s0 = {}, s1 = {};
    float smax = 0.f;                      // the tile's largest row scale (every lane alike)
    if (wave_on) {
      constexpr int QK_AHEAD = 2;
      i16x8 ra[QK_AHEAD + 1][4];
      auto issue_qk = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int slot = ks % (QK_AHEAD + 1);
        if constexpr (ks < 8) {
          constexpr int off = 128 * (ks >> 1);
          lds_read_b128<off>(ra[slot][0], tb + so[ks & 1][0]);
          lds_read_b128<off>(ra[slot][1], tb + so[ks & 1][1]);
          lds_read_b128<off + 32 * ROWW>(ra[slot][2], tb + so[ks & 1][0]);
          lds_read_b128<off + 32 * ROWW>(ra[slot][3], tb + so[ks & 1][1]);
        } else {
          lds_read_b128<0>(ra[slot][0], tb + sr[0]);
          lds_read_b128<0>(ra[slot][1], tb + sr[1]);
          lds_read_b128<32 * ROWW>(ra[slot][2], tb + sr[0]);
          lds_read_b128<32 * ROWW>(ra[slot][3], tb + sr[1]);
        }
      };
      static_for<0, QK_AHEAD>(issue_qk);
      static_for<0, ROWW / 64>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int NS = ROWW / 64;
        constexpr int ahead = (NS - 1 - ks) < QK_AHEAD ? (NS - 1 - ks) : QK_AHEAD;
        if constexpr (ks + QK_AHEAD < NS) issue_qk(std::integral_constant<int, ks + QK_AHEAD>{});
        issue_load(next, next_buf, std::integral_constant<int, ks>{});
        constexpr int slot = ks % (QK_AHEAD + 1);
        wait_lgkm<4 * ahead>(ra[slot][0], ra[slot][1], ra[slot][2], ra[slot][3]);
        const u32x4 x0 = __builtin_bit_cast(u32x4, ra[slot][0]), x1 = __builtin_bit_cast(u32x4, ra[slot][1]);
        const u32x4 y0 = __builtin_bit_cast(u32x4, ra[slot][2]), y1 = __builtin_bit_cast(u32x4, ra[slot][3]);
        const v8i a0 = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        const v8i a1 = {(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
        s0 = mfma8(a0, q8[ks], s0);
        s1 = mfma8(a1, q8[ks], s1);
        // one group of row scales per k-step, between the products
        if constexpr (ks < 8) {
          const f32x4 sg = sig[ks >> 2][ks & 3];
          smax = max3f(smax, max3f(sg[0], sg[1], sg[2]), sg[3]);
        }
      });
    } else {
      static_for<0, 9>([&](auto kc) { issue_load(next, next_buf, kc); });
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          smax = max3f(smax, max3f(sig[sb][gq][0], sig[sb][gq][1], sig[sb][gq][2]), sig[sb][gq][3]);
    }

    // the exponent e from the tile's largest row scale
    {
      smax = max_halves(smax);
      if (smax > 0.f) {
        const int e_tile = (int)((__builtin_bit_cast(uint32_t, smax) >> 23) & 0xFF) - 126;   // smax < 2^e_tile
        const int e_new = __builtin_amdgcn_readfirstlane(max(e_cur, e_tile));
        if (e_new != e_cur) {
          if (e_cur != E_NONE) {
            const float f = __builtin_ldexpf(1.0f, e_cur - e_new);
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
              for (int rb = 0; rb < 4; ++rb) scale_acc(acc[c2][rb], f);
          }
          e_cur = e_new;
        }
      }
    }

    if (wave_on) {
      // scores in the log2 domain before the row constant: x = S8 * sigma
      float x0[16], x1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x0[r] = s0[r] * sig[0][r >> 2][r & 3];
        x1[r] = s1[r] * sig[1][r >> 2][r & 3];
      }
      if (__builtin_amdgcn_ballot_w64(ts + KT > lim) != 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = ts + 8 * (r >> 2) + 4 * half + (r & 3);
          x0[r] = (t < lim) ? x0[r] : -INFINITY;
          x1[r] = (t + 32 < lim) ? x1[r] : -INFINITY;
        }
      }
      float mq[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * c;
        mq[c] = max3f(max3f(x0[r], x0[r + 1], x0[r + 2]), max3f(x0[r + 3], x1[r], x1[r + 1]),
                      max3f(x1[r + 2], x1[r + 3], x1[r + 3]));
      }
      const float mx = max_halves(max3f(max3f(mq[0], mq[1], mq[2]), mq[3], mq[3])) * c_row;
      m_run = fmaxf(m_run, mx);
      const bool first = m_ref == -INFINITY;
      const float over = (mx - m_ref - REF_STEP) * (1.0f / REF_STEP);
      const int kraw = (!first && over > 0.f) ? (int)ceilf(over) : 0;
      const int kstep = kraw > 7 ? 7 : kraw;
      l_sum = kstep == 7 ? 0.f : l_sum * __builtin_amdgcn_exp2f(-REF_STEP * kstep);
      m_ref = (first || kstep == 7) ? mx : m_ref + REF_STEP * kstep;
      // w = p sigma 2^-e: the exact power of two rides in the exponent
      // (no scale seen yet: every sigma of the tile is 0 and so is every weight)
      const float nbase = ((m_ref == -INFINITY) ? 0.f : -m_ref) - (e_cur == E_NONE ? 0.f : (float)e_cur);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float pa[4], pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pa[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x0[4 * gq + i], c_row, nbase));
          pb[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x1[4 * gq + i], c_row, nbase));
        }
        const f32x4 sa = sig[0][gq], sbv = sig[1][gq];
        // no clamp to the E4M3 maximum is needed: p <= 2^8 (the reference
        // rule) and sigma 2^-e < 1 (the choice of e), so every weight is <= 256
        pw[gq] = e4m3x4(pa[0] * sa[0], pa[1] * sa[1], pa[2] * sa[2], pa[3] * sa[3]);
        pw[4 + gq] = e4m3x4(pb[0] * sbv[0], pb[1] * sbv[1], pb[2] * sbv[2], pb[3] * sbv[3]);
      }
      // (the tile's share of the normaliser is summed in the value phase)
      // the reference step of the row rides in the sign bits of bytes 0..2
      // (weights are >= 0), in both lane halves
      pw[0] |= ((kstep & 1) ? 0x80u : 0u) | ((kstep & 2) ? 0x8000u : 0u) | ((kstep & 4) ? 0x800000u : 0u);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pw[i] = 0u;
    }
    *(u32x4*)(pbuf + ((wave * 64 + lane) * 32)) = u32x4{pw[0], pw[1], pw[2], pw[3]};
    *(u32x4*)(pbuf + ((wave * 64 + lane) * 32) + 16) = u32x4{pw[4], pw[5], pw[6], pw[7]};

    // ================= value phase (128 columns x all 128 rows) =================
    // the transposed code fragments of the four column blocks only need the tile
    v8i av[4];
    {
      v2i tr[4][4];
      static_for<0, 4>([&](auto cbc) {
        constexpr int cb = decltype(cbc)::value;
        lds_read_tr8<0>(tr[cb][0], tb + tro[cb]);
        lds_read_tr8<16 * ROWW>(tr[cb][1], tb + tro[cb]);
        lds_read_tr8<32 * ROWW>(tr[cb][2], tb + tro[cb]);
        lds_read_tr8<48 * ROWW>(tr[cb][3], tb + tro[cb]);
      });
      barrier_lds();   // probability fragments of all 128 rows visible (waits for the reads above too)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        av[cb] = v8i{tr[cb][0][0], tr[cb][0][1], tr[cb][1][0], tr[cb][1][1],
                     tr[cb][2][0], tr[cb][2][1], tr[cb][3][0], tr[cb][3][1]};
    }
    i16x8 bq[4][2];
    float lq[4];
    static_for<0, 4>([&](auto rbc) {
      constexpr int rb = decltype(rbc)::value;
      lds_read_b128<rb * 64 * 32>(bq[rb][0], pb_lane);
      lds_read_b128<rb * 64 * 32 + 16>(bq[rb][1], pb_lane);
    });
    // row block by row block as its probability fragments land: the reference
    // step of rows 32 rb + l32 (sign bits of bytes 0..2) rescales that block's
    // accumulators first, then its four products
    static_for<0, 4>([&](auto rbc) {
      constexpr int rb = decltype(rbc)::value;
      wait_lgkm<2 * (3 - rb)>(bq[rb][0], bq[rb][1]);
      u32x4 y0 = __builtin_bit_cast(u32x4, bq[rb][0]);
      const u32x4 y1 = __builtin_bit_cast(u32x4, bq[rb][1]);
      const uint32_t d0 = y0[0];
      const int code = (int)(((d0 >> 7) & 1u) | ((d0 >> 14) & 2u) | ((d0 >> 21) & 4u));
      if (__builtin_amdgcn_ballot_w64(code != 0) != 0) {
        const float alpha = code == 0 ? 1.0f : (code == 7 ? 0.0f : __builtin_amdgcn_exp2f(-REF_STEP * code));
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) scale_acc(acc[c2][rb], alpha);
      }
      y0[0] &= 0xFF7F7F7Fu;
      const v8i bv = {(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3], (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb][rb] = mfma8(av[cb], bv, acc[cb][rb]);
      // under the products: this lane's share of the normaliser, the
      // probabilities the value product actually uses, dequant(w8) / sigma
      // (times 2^e below), for its weight group rb (the step bits of word 0
      // masked off)
      {
        constexpr int gq = rb;
        const uint32_t wa = gq == 0 ? (pw[0] & 0xFF7F7F7Fu) : pw[gq];
        const f32x4 ra = *(const f32x4*)(sct + KT + 8 * gq + 4 * half);
        const f32x4 rbv = *(const f32x4*)(sct + KT + 32 + 8 * gq + 4 * half);
        const auto qa0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wa, false);
        const auto qa1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wa, true);
        const auto qb0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[4 + gq], false);
        const auto qb1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[4 + gq], true);
        lq[gq] = ((qa0[0] * ra[0] + qa0[1] * ra[1]) + (qa1[0] * ra[2] + qa1[1] * ra[3])) +
                 ((qb0[0] * rbv[0] + qb0[1] * rbv[1]) + (qb1[0] * rbv[2] + qb1[1] * rbv[3]));
      }
    });
    l_sum += sum_halves((lq[0] + lq[1]) + (lq[2] + lq[3])) * (e_cur == E_NONE ? 0.f : __builtin_ldexpf(1.0f, e_cur));
    // the next tile's scales go to the buffer the previous tile used
    if (has_next && tid < KT) {
      scl[((tile + 1) & 1) * 2 * KT + tid] = sc_next;
      scl[((tile + 1) & 1) * 2 * KT + KT + tid] = sc_next > 0.f ? 1.0f / sc_next : 0.f;
    }
  }

  // ---- epilogue: share each row's normaliser, write the normalised partials.
  // The partials are staged over the tile buffers: the loads issued past the
  // last tile must have landed first.
  barrier_tile_ready();
  float* const lsh = (float*)(smem + SPLIT_STAGE_BYTES);   // [128] l_sum
  if (half == 0) lsh[wave * 32 + l32] = l_sum;
  barrier_lds();
  const float unscale = e_cur == E_NONE ? 1.0f : __builtin_ldexpf(1.0f, e_cur);
  const int64_t pbase = (int64_t)sl * p.R;
  store_split_partials(p, acc, lsh, smem, pbase, g, wave, lane, unscale);
  if (half == 0 && own_ok) p.part_lse[pbase + own_r] = l_sum > 0.f ? m_ref + log2f(l_sum) : -INFINITY;
  // the part's maximum score, for the accuracy check of the fix-up scan
  if (half == 0 && own_ok && p.part_mrun != nullptr) p.part_mrun[pbase + own_r] = m_run;
}

}  // namespace

hipError_t launch_decode_split_f8(const DecodeParams& p, hipStream_t stream) {
  const int grid = 8 * p.work_per_xcd;
  if (p.paged)
    hipLaunchKernelGGL((decode_split_f8_kernel<true>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_f8_kernel<false>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
