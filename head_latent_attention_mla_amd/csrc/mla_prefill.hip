// Prefill by expansion: the other bracketing of the same attention
// ("Why MLA and MTP Fight Each Other", sections 5.5 and 5.6: with many query
// tokens per cached row the per-row expansion is shared by all of them and the
// narrower per-pair contraction wins; "MLA, dim by dim", "MLA Prefill": form
// K = C W_UK and V = C W_UV once, then run ordinary attention over them).
//
// The expansion writes K_nope and V token-major, [B, T_pad, H * 128 + 64]
// bf16 (head h at h * 128 of a row; the pad keeps one head's rows from being
// a power of two apart): expand_kv_kernel, one persistent work-group per
// (head, K or V) that holds that half of the head's weights in LDS and
// streams every cached row (contiguous or paged, bf16 or dequantised E4M3)
// through MFMA, rows past a sequence's end written as 0.
//   copy_rope_kernel copies the rows' rope keys to [B, T_pad, 64].
// Rows past a sequence's end are masked in the attention.  Then one
// attention kernel:
//   prefill_attn_kernel  per (128 query rows, head, sequence): causal flash
//       attention.  Each wave owns 32 query rows: S^T = K Q^T (the K tile from
//       LDS, the query rows held in registers), an online softmax per row,
//       and O^T += V^T P^T with the probabilities kept in registers (the
//       score accumulator layout is already the value product's B operand,
//       up to a fixed permutation of the 16 rows of each k-step that the
//       transposed V reads follow).  K, rope key and V tiles of 64 rows reach
//       LDS by direct loads, double-buffered; 80 KB of LDS lets two
//       work-groups share a compute unit, so one's softmax overlaps the
//       other's matrix products.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int KT = 64;                        // cached rows per attention tile
constexpr int QT = 128;                       // query rows per attention work-group
constexpr int ET = 128;                       // cached rows per expansion work-group
constexpr int KN_BYTES = KT * D_NOPE * 2;     // 16 KB: K_nope tile
constexpr int KR_BYTES = KT * D_ROPE * 2;     // 8 KB: rope key tile
constexpr int V_BYTES = KT * D_V * 2;         // 16 KB: V tile
constexpr int BUF_BYTES = KN_BYTES + KR_BYTES + V_BYTES;
constexpr float REF_STEP = 8.0f;              // softmax reference moves when the max passes it by 2^8

__device__ __forceinline__ i16x8 ld16(const void* p) { return *(const i16x8*)p; }

// the row of sequence b at position t in the cache (element index of its first value)
__device__ __forceinline__ int64_t cache_row(const PrefillParams& p, int b, int t) {
  if (p.block_table != nullptr) return (int64_t)p.block_table[(int64_t)b * p.max_blocks + (t >> 6)] * 64 + (t & 63);
  return (int64_t)b * p.T_stride + t;
}

// 16 consecutive e4m3 codes times the row scale -> two bf16x8 fragments
__device__ __forceinline__ void dequant16(u32x4 w, float s, i16x8& lo, i16x8& hi) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
    i16x8& o = d < 2 ? lo : hi;
    const int e = 4 * (d & 1);
    o[e + 0] = (short)bf16_bits(to_bf16(a[0] * s));
    o[e + 1] = (short)bf16_bits(to_bf16(a[1] * s));
    o[e + 2] = (short)bf16_bits(to_bf16(c[0] * s));
    o[e + 3] = (short)bf16_bits(to_bf16(c[1] * s));
  }
}

// ---------------------------------------------------------------------------
// expansion: one persistent work-group per (head, K or V) keeps that half of
// the head's weights -- W_UK[h] or W_UV[h]^T, 128 rows x 512 -- in LDS (128
// KB, 16-byte chunks XOR row & 7) and walks every 128-row tile of every
// sequence: D[n][t] = sum_c W[n][c] C[t][c], K = 512 in 8 chunks of 64.  Wave
// (nq, tq) = (w & 1, w >> 1) owns outputs 64 nq .. + 63 and tile rows 64 tq ..
// + 63 (2 x 2 blocks of 32 x 32).  The cached-row fragments go straight to
// registers, three chunks ahead across tile boundaries; within a chunk the k
// order is permuted alike for both operands (lane half h holds c = 32 h ..
// 32 h + 31, MFMA j takes 8 j .. 8 j + 7), so a lane reads 64 contiguous bytes.
// ---------------------------------------------------------------------------
constexpr int E_AHEAD = 3;                      // chunks of cached-row fragments in flight
constexpr int E_NCH = D_C / 64;                 // 8 chunks of 64 per tile

template <bool FP8>
__global__ __launch_bounds__(256) void expand_kv_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char wl[D_NOPE * D_C * 2];   // 128 KB
  const int h = blockIdx.x >> 1, part = blockIdx.x & 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int nq = wave & 1, tq = wave >> 1;
  const uint32_t wl_a = lds_addr(wl);

  // the weight half: row L of 1 KB is load L (wave w: rows 32 w .. + 31);
  // slot lane holds logical chunk lane ^ (L & 7)
  {
    const uint16_t* W = (part ? p.w_uvt : p.w_uk) + (int64_t)h * D_NOPE * D_C;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      const int L = 32 * wave + i;
      __builtin_amdgcn_global_load_lds((const void*)(W + (int64_t)L * D_C + 8 * (lane ^ (L & 7))),
                                       (lds_void_t*)(wl + L * 1024), 16, 0, 0);
    }
  }
  // A-fragment reads: row 64 nq + 32 nb + l32, logical chunk 8 ch + 4 half + j
  uint32_t wo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wo[j] = wl_a + (64 * nq + l32) * 1024 + 16 * ((4 * half + j) ^ (l32 & 7));

  const int n_tt = p.T_pad / ET;
  const int n_steps = p.B * n_tt * E_NCH;
  constexpr int elem = FP8 ? 1 : 2;
  // the cached row behind fragment (step s, t-block tb) of this lane; rows
  // past a sequence's end reuse its last row (their outputs are stored as 0)
  auto frag_src = [&](int s, int tb, float& sc) -> const char* {
    const int tile = s / E_NCH, ch = s % E_NCH;
    const int b = tile / n_tt, tt = tile % n_tt;
    const int T = p.seqlens[b];
    const int t = min(tt * ET + 64 * tq + 32 * tb + l32, T - 1);
    const int64_t r = cache_row(p, b, t);
    sc = FP8 ? p.row_scale[r] : 1.0f;
    return (const char*)p.rows + (r * ROWW + ch * 64 + 32 * half) * elem;
  };
  // ring of fragments (bf16 rows) or raw codes and scales (e4m3 rows)
  i16x8 cf[E_AHEAD + 1][2][FP8 ? 1 : 4];
  float csc[E_AHEAD + 1][2];
  uint32_t c8[E_AHEAD + 1][2][FP8 ? 8 : 1];
  auto issue = [&](int s, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const char* src = frag_src(s, tb, csc[slot][tb]);
      if constexpr (FP8) {
        const u32x4 a = *(const u32x4*)src, c = *(const u32x4*)(src + 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c8[slot][tb][q] = a[q];
          c8[slot][tb][4 + q] = c[q];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) cf[slot][tb][j] = *(const i16x8*)(src + 16 * j);
      }
    }
  };
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();                                     // the weights are in LDS

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  // the step loop is unrolled by the ring size so every ring slot is a
  // compile-time index
  static_for<0, E_AHEAD>([&](auto sc) {
    if (decltype(sc)::value < n_steps) issue(decltype(sc)::value, sc);
  });
  for (int s0 = 0; s0 < n_steps; s0 += E_AHEAD + 1) {
    static_for<0, E_AHEAD + 1>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int s = s0 + u;
      if (s >= n_steps) return;
      if (s + E_AHEAD < n_steps) issue(s + E_AHEAD, std::integral_constant<int, (u + E_AHEAD) % (E_AHEAD + 1)>{});
      const int tile = s / E_NCH, ch = s % E_NCH;
      i16x8 bf[2][4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if constexpr (FP8) {
          dequant16(u32x4{c8[u][tb][0], c8[u][tb][1], c8[u][tb][2], c8[u][tb][3]}, csc[u][tb], bf[tb][0], bf[tb][1]);
          dequant16(u32x4{c8[u][tb][4], c8[u][tb][5], c8[u][tb][6], c8[u][tb][7]}, csc[u][tb], bf[tb][2], bf[tb][3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) bf[tb][j] = cf[u][tb][j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        i16x8 af[2];
        const uint32_t a = wo[j] + ch * 128;
        lds_read_b128<0>(af[0], a);
        lds_read_b128<32 * 1024>(af[1], a);
        wait_lgkm<0>(af[0], af[1]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            acc[nb][tb] = mfma32(__builtin_bit_cast(bf16x8, af[nb]), __builtin_bit_cast(bf16x8, bf[tb][j]), acc[nb][tb]);
      }
      if (ch == E_NCH - 1) {
        // lane holds D[n = 64 nq + 32 nb + 8 g + 4 half + e][t = 64 tq + 32 tb + l32]
        const int b = tile / n_tt, t0 = (tile % n_tt) * ET;
        const int T = p.seqlens[b];
        uint16_t* dst = (part ? p.v : p.k_nope) + ((int64_t)b * p.T_pad + t0) * p.kv_ld + h * D_NOPE;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int t = 64 * tq + 32 * tb + l32;
          const bool live = t0 + t < T;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint64_t v = 0;
              if (live) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v |= (uint64_t)bf16_bits(to_bf16(acc[nb][tb][4 * g + e])) << (16 * e);
              }
              *(uint64_t*)(dst + (int64_t)t * p.kv_ld + 64 * nq + 32 * nb + 8 * g + 4 * half) = v;
            }
            acc[nb][tb] = f32x16{};
          }
        }
      }
    });
  }
}

// the rope keys of every row: [B, T_pad, 64] bf16 (zeros past a sequence's end)
__global__ __launch_bounds__(256) void copy_rope_kernel(PrefillParams p) {
  const int tt = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int T = p.seqlens[b];
  const int t0 = tt * ET;
  uint16_t* rdst = p.rope + ((int64_t)b * p.T_pad + t0) * D_ROPE;
  if (p.fp8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;            // row idx / 4, codes 16 (idx % 4) .. + 15
      const int t = idx >> 2, qd = idx & 3;
      i16x8 lo = {0, 0, 0, 0, 0, 0, 0, 0}, hi = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t0 + t < T) {
        const int64_t r = cache_row(p, b, t0 + t);
        dequant16(*(const u32x4*)((const uint8_t*)p.rows + r * ROWW + D_C + 16 * qd), p.row_scale[r], lo, hi);
      }
      *(i16x8*)(rdst + (int64_t)t * D_ROPE + 16 * qd) = lo;
      *(i16x8*)(rdst + (int64_t)t * D_ROPE + 16 * qd + 8) = hi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;            // row idx / 8, values 8 (idx % 8) .. + 7
      const int t = idx >> 3, c = idx & 7;
      i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t0 + t < T) v = ld16((const uint16_t*)p.rows + cache_row(p, b, t0 + t) * ROWW + D_C + 8 * c);
      *(i16x8*)(rdst + (int64_t)t * D_ROPE + 8 * c) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillParams p, int n_qt, int n_items,
                                                                int per_xcd) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * BUF_BYTES];
  const uint32_t smem_a = lds_addr(smem);
  // XCD-aware order: launch slot L runs on XCD L % 8; the query tiles of one
  // (sequence, head) take consecutive items on one XCD, so its K and V tiles
  // are fetched into that XCD's L2 once; within a head, longest causal rows first
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= n_items) return;
  const int qt = n_qt - 1 - item % n_qt;
  const int h = (item / n_qt) % p.H;
  const int b = item / (n_qt * p.H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int T = p.seqlens[b];
  const int H = p.H, s_q = p.s_q;

  // own query row j (rows past s_q compute on row s_q - 1 and are not stored)
  const int j_own = qt * QT + 32 * wave + l32;
  const bool own_ok = j_own < s_q;
  const int j_eff = min(j_own, s_q - 1);
  const int lim = p.causal ? T - s_q + j_eff + 1 : T;              // visible rows 0 .. lim - 1
  const int j_last = min(qt * QT + QT - 1, s_q - 1);
  const int lim_wg = p.causal ? T - s_q + j_last + 1 : T;
  const int n_tiles = (lim_wg + KT - 1) / KT;

  bf16x8 qf[D_QK / 16];
  {
    const uint16_t* qrow = p.q + (((int64_t)b * s_q + j_eff) * H + h) * D_QK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D_QK / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qrow + 16 * ks));
  }

  // ---- direct-to-LDS tile loads.  Region rows hold R chunks of 16 B (R = 16
  // for K_nope and V, 8 for the rope key) with the chunk index XORed by a
  // per-row pattern; a 1 KB load k fills slots 64 k + lane, so lane l fetches
  // the chunk that lands there.  A 128-bit LDS read is served 16 lanes per
  // pass from 64 banks (256 B) and a 64-bit transposed read 32 lanes per pass,
  // so the patterns make those lane groups hit distinct bank slots:
  //   K_nope (256 B rows; score reads, 16 rows x 1 chunk): chunk ^ (t & 15)
  //   rope   (128 B rows; score reads):                   chunk ^ ((t >> 1) & 7)
  //   V      (256 B rows; transposed reads, 4 rows x 4 chunks): chunk ^ 4 (t & 3)
  // All three are unchanged by t + 32 (and V's by t + 8), which the reads
  // reach through immediate offsets.
  // K_nope and V are token-major [B, T_pad, kv_ld]: the 256-byte rows of
  // head h are RS = 2 kv_ld bytes apart
  const int64_t RS = (int64_t)p.kv_ld * 2;
  const char* kn_base = (const char*)(p.k_nope + (int64_t)b * p.T_pad * p.kv_ld + h * D_NOPE);
  const char* v_base = (const char*)(p.v + (int64_t)b * p.T_pad * p.kv_ld + h * D_V);
  const char* r_base = (const char*)(p.rope + (int64_t)b * p.T_pad * D_ROPE);
  // K_nope load 4 w + i covers rows 16 w + 4 i + (lane >> 4); V the same rows;
  // rope load 2 w + i rows 16 w + 8 i + (lane >> 3)
  // The K_nope and V windows of a tile end at the sequence's last row, so
  // rows past it load as zeros whatever the workspace holds there; the whole
  // offset of a load sits in its lane offset, which the window bounds.
  const int T_u = __builtin_amdgcn_readfirstlane(T);   // the windows must be uniform
  uint32_t offk[4], offv[4], offr[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t base = (uint32_t)(4 * (4 * wave + i) + (lane >> 4)) * (uint32_t)RS;
    offk[i] = base + 16 * ((lane & 15) ^ ((4 * i + (lane >> 4)) & 15));
    offv[i] = base + 16 * ((lane & 15) ^ (4 * (lane >> 4)));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) offr[i] = (uint32_t)((lane >> 3) * 128 + 16 * ((lane & 7) ^ (4 * i + (lane >> 4))));
  auto issue_tile = [&](int tile, int buf) {
    const int64_t r0 = (int64_t)tile * KT;
    const int valid = max(0, min(KT, T_u - (int)r0));
    const int kv_bytes = valid * (int)RS;
    const auto kn = __builtin_amdgcn_make_buffer_rsrc((void*)(kn_base + r0 * RS), (short)0, kv_bytes, 0x00020000);
    const auto vv = __builtin_amdgcn_make_buffer_rsrc((void*)(v_base + r0 * RS), (short)0, kv_bytes, 0x00020000);
    const auto kr = __builtin_amdgcn_make_buffer_rsrc((void*)(r_base + r0 * 128), (short)0, KR_BYTES, 0x00020000);
    char* dst = smem + buf * BUF_BYTES;
    // wave w: K_nope and V loads 4 w .. 4 w + 3, rope loads 2 w, 2 w + 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kn, (lds_void_t*)(dst + k * 1024), 16, offk[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vv, (lds_void_t*)(dst + KN_BYTES + KR_BYTES + k * 1024), 16, offv[i],
                                               0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = 2 * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(dst + KN_BYTES + k * 1024), 16, offr[i], k * 1024, 0,
                                               0);
    }
  };

  // score-phase reads: row l32 (+32), chunk 2 ks + half (k-steps 0..7 in
  // K_nope, 8..11 in the rope key), XOR-swizzled
  uint32_t qo_n[8], qo_r[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qo_n[ks] = l32 * 256 + 16 * ((2 * ks + half) ^ (l32 & 15));
#pragma unroll
  for (int i = 0; i < 4; ++i) qo_r[i] = KN_BYTES + l32 * 128 + 16 * ((2 * i + half) ^ ((l32 >> 1) & 7));
  // value-phase transposed reads (V^T fragments): lane reads row 16 kap + 4
  // half + rsel (+ 8), columns 32 cb + 16 grp + csel
  uint32_t pvo[4];
  {
    const int grp = (lane >> 4) & 1;
    const int rsel = (lane & 15) >> 2;
    const int csel = 4 * (lane & 3);
    const int trow = 4 * half + rsel;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int chunk = 4 * cb + 2 * grp + (csel >> 3);
      pvo[cb] = KN_BYTES + KR_BYTES + trow * 256 + 16 * (chunk ^ (4 * rsel)) + (csel & 7) * 2;
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float m_ref = -INFINITY, l_sum = 0.f;

  if (n_tiles > 0) issue_tile(0, 0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    // tile in LDS (every wave's loads done); every wave is past the previous
    // value phase, so the other buffer is free for the next tile
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tile + 1 < n_tiles) issue_tile(tile + 1, (tile + 1) & 1);
    const uint32_t tb = smem_a + (tile & 1) * BUF_BYTES;
    const int ts = tile * KT;

    // ---- S^T = K Q^T: rows t = 32 sb + ..., columns = own query row.  LDS
    // reads run QK_AHEAD k-steps ahead of the products (inline asm: the
    // compiler would otherwise wait for the next tile's loads before them)
    f32x16 s0 = {}, s1 = {};
    {
      uint32_t an[8], ar[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) an[i] = tb + qo_n[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = tb + qo_r[i];
      constexpr int QK_AHEAD = 3;
      i16x8 ra[QK_AHEAD + 1][2];
      auto issue_qk = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int slot = ks % (QK_AHEAD + 1);
        if constexpr (ks < 8) {
          lds_read_b128<0>(ra[slot][0], an[ks]);
          lds_read_b128<32 * 256>(ra[slot][1], an[ks]);
        } else {
          lds_read_b128<0>(ra[slot][0], ar[ks & 3]);
          lds_read_b128<32 * 128>(ra[slot][1], ar[ks & 3]);
        }
      };
      static_for<0, QK_AHEAD>(issue_qk);
      static_for<0, D_QK / 16>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int NS = D_QK / 16;
        constexpr int ahead = (NS - 1 - ks) < QK_AHEAD ? (NS - 1 - ks) : QK_AHEAD;
        if constexpr (ks + QK_AHEAD < NS) issue_qk(std::integral_constant<int, ks + QK_AHEAD>{});
        constexpr int slot = ks % (QK_AHEAD + 1);
        wait_lgkm<2 * ahead>(ra[slot][0], ra[slot][1]);
        s0 = mfma32(__builtin_bit_cast(bf16x8, ra[slot][0]), qf[ks], s0);
        s1 = mfma32(__builtin_bit_cast(bf16x8, ra[slot][1]), qf[ks], s1);
      });
    }
    // the first two V^T fragments only need the tile: start them now
    uint32_t pv[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) pv[cb] = tb + pvo[cb];
    i16x4 tr[3][2];
    auto issue_a = [&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int kap = u >> 2, cb = u & 3;
      constexpr int off = 16 * kap * 256;
      const uint32_t a = pv[cb];
      lds_read_tr16<off>(tr[u % 3][0], a);
      lds_read_tr16<off + 8 * 256>(tr[u % 3][1], a);
    };
    issue_a(std::integral_constant<int, 0>{});
    issue_a(std::integral_constant<int, 1>{});

    // rows at or past the own limit do not count
    if (__builtin_amdgcn_ballot_w64(ts + KT > lim) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = ts + 8 * (r >> 2) + 4 * half + (r & 3);
        s0[r] = (t < lim) ? s0[r] : -INFINITY;
        s1[r] = (t + 32 < lim) ? s1[r] : -INFINITY;
      }
    }
    float mq[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 4 * c;
      mq[c] = fmaxf(fmaxf(fmaxf(s0[r], s0[r + 1]), fmaxf(s0[r + 2], s0[r + 3])),
                    fmaxf(fmaxf(s1[r], s1[r + 1]), fmaxf(s1[r + 2], s1[r + 3])));
    }
    const float mraw = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    float ma = mraw, mb = mraw;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(ma), "+v"(mb));
    const float mx = fmaxf(ma, mb) * p.scale_log2;
    // lazy reference: moves only when the maximum passes it by more than 2^8
    // (the first tile always holds a visible row of every live query row)
    const bool move = m_ref == -INFINITY || mx > m_ref + REF_STEP;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float m_new = move ? mx : m_ref;
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_sum *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] *= alpha;
      m_ref = m_new;
    }
    bf16x8 pk[2][2];
    float lq[4] = {0.f, 0.f, 0.f, 0.f};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pk[0][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, -m_ref)));
      pk[1][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, -m_ref)));
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pk[sb][jj][e], pk[sb][jj][e + 1]};
          lq[2 * jj + sb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lq[2 * jj + sb], false);
        }
    {
      const float lsum = (lq[0] + lq[1]) + (lq[2] + lq[3]);
      float a2 = lsum, b2 = lsum;
      asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a2), "+v"(b2));
      l_sum += a2 + b2;
    }

    // ---- O^T += V^T P^T: 16 units u = 4 kap + cb (k-step kap of 16 rows,
    // column block cb); the transposed V fragment of a unit is read two units
    // ahead, every wait names the exact number of younger reads
    static_for<0, 16>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int kap = u >> 2, cb = u & 3;
      constexpr int younger = u == 15 ? 0 : 2;
      wait_lgkm<younger>(tr[u % 3][0], tr[u % 3][1]);
      if constexpr (u + 2 < 16) issue_a(std::integral_constant<int, u + 2>{});
      acc[cb] = mfma32(join_tr(tr[u % 3][0], tr[u % 3][1]), pk[kap >> 1][kap & 1], acc[cb]);
    });
  }

  // ---- epilogue: out[b, j, h, dv] = O / l; lane holds dv = 32 cb + 8 g + 4 half + e
  if (!own_ok) return;
  const float inv = l_sum > 0.f ? 1.0f / l_sum : 0.f;
  uint16_t* orow = p.out + (((int64_t)b * s_q + j_own) * H + h) * D_V;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint64_t v = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) v |= (uint64_t)bf16_bits(to_bf16(acc[cb][4 * g + e] * inv)) << (16 * e);
      *(uint64_t*)(orow + 32 * cb + 8 * g + 4 * half) = v;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  hipError_t e = launch_transpose_wuv(p.w_uv, p.w_uvt, p.H, stream);
  if (e != hipSuccess) return e;
  if (p.fp8)
    hipLaunchKernelGGL(expand_kv_kernel<true>, dim3(2 * p.H), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(expand_kv_kernel<false>, dim3(2 * p.H), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(copy_rope_kernel, dim3(p.T_pad / ET, p.B), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (p.s_q + QT - 1) / QT;
  const int n_items = n_qt * p.H * p.B;
  const int per_xcd = (n_items + 7) / 8;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(8 * per_xcd), dim3(256), 0, stream, p, n_qt, n_items, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
