// Prefill by expansion: the other bracketing of the same attention
// ("Why MLA and MTP Fight Each Other", sections 5.5 and 5.6: with many query
// tokens per cached row the per-row expansion is shared by all of them and the
// narrower per-pair contraction wins; "MLA, dim by dim", "MLA Prefill": form
// K = C W_UK and V = C W_UV once, then run ordinary attention over them).
//
// The expansion writes K_nope and V token-major, [B, T_pad, H * 128 + 64]
// bf16 (head h at h * 128 of a row; the pad keeps one head's rows from being
// a power of two apart): expand_kv_kernel, one work-group per (head, K or V)
// that holds that half of the head's weights in registers and streams every
// cached row (contiguous or paged, bf16 or dequantised E4M3) through LDS into
// MFMA, rows past a sequence's end written as 0.
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
constexpr int ET = 128;                       // cached rows per rope-copy work-group
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
// (two values per conversion instruction)
__device__ __forceinline__ void dequant16(u32x4 w, float s, i16x8& lo, i16x8& hi) {
  uint64_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
    o[d] = pack_bf16x4(f32x4{a[0] * s, a[1] * s, c[0] * s, c[1] * s});
  }
  lo = __builtin_bit_cast(i16x8, u32x4{(uint32_t)o[0], (uint32_t)(o[0] >> 32), (uint32_t)o[1], (uint32_t)(o[1] >> 32)});
  hi = __builtin_bit_cast(i16x8, u32x4{(uint32_t)o[2], (uint32_t)(o[2] >> 32), (uint32_t)o[3], (uint32_t)(o[3] >> 32)});
}

// ---------------------------------------------------------------------------
// expansion: one work-group per (head, K or V), one per compute unit.  Its
// weight half -- W_UK[h] or W_UV[h]^T, 128 outputs x 512 -- stays in registers
// as MFMA A fragments (wave w: outputs 32 w .. 32 w + 31, 128 VGPRs a lane).
// The cached rows stream through LDS in 64-row tiles, double-buffered, each
// direct-to-LDS load filling one whole 1 KB row (16-byte chunk c of row t at
// slot c ^ (t & 15), so the fragment reads of 16 consecutive rows hit
// distinct banks): D[n][t] = sum_c W[n][c] C[t][c] in 32 k-steps of 16, every
// C fragment read from LDS once.  A tile's 128 x 64 result is staged in LDS
// and stored one tile later as whole 256-byte row pieces.  E4M3 rows: the
// codes land in LDS and are converted (code x row scale -> bf16) into a
// single bf16 tile buffer at the top of the tile.
// ---------------------------------------------------------------------------
constexpr int X_T = 64;                         // cached rows per tile
constexpr int X_TILE = X_T * D_C * 2;           // 64 KB: bf16 tile, 1 KB rows
constexpr int X_CODES = X_T * D_C;              // 32 KB: e4m3 codes of a tile
constexpr int X_STAGE = X_T * D_NOPE * 2;       // 16 KB: a tile's outputs, 256-byte rows
constexpr int X_RING = 4;                       // k-steps of C fragments in flight
static_assert(2 * X_TILE + 2 * X_STAGE <= 160 * 1024, "LDS budget");
static_assert(X_TILE + 2 * X_CODES == 2 * X_TILE, "E4M3 layout fits the bf16 one");

template <int OFF>
__device__ __forceinline__ void lds_write_b64(uint32_t addr, uint64_t v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void expand_kv_kernel(PrefillParams p) {
  // bf16 rows: tile buffers 0 and 1; E4M3 rows: the bf16 tile, then two code
  // buffers; then two output staging buffers
  __shared__ __attribute__((aligned(1024))) char smem[2 * X_TILE + 2 * X_STAGE];
  const uint32_t smem_a = lds_addr(smem);
  const uint32_t stage_a = smem_a + 2 * X_TILE;
  const int h = blockIdx.x >> 1, part = blockIdx.x & 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int n_tt = p.T_pad / X_T;
  const int n_tiles = p.B * n_tt;
  if (n_tiles == 0) return;

  constexpr int ELEM = FP8 ? 1 : 2;
  constexpr int ROW_BYTES = ROWW * ELEM;
  // tile `it` = (sequence b, rows t0 .. t0 + 63).  Its sequence length and
  // block-table entry are loaded one tile before the tile's loads are issued
  // and only then moved to scalar registers, so that no load waits on them
  // right after they were fetched.
  int meta_len = 0, meta_blk = 0;
  auto load_meta = [&](int it) {
    const int b = it / n_tt, t0 = (it % n_tt) * X_T;
    meta_len = p.seqlens[b];
    if (p.block_table != nullptr)   // an in-range entry; unused for a tile past the sequence's end
      meta_blk = p.block_table[(int64_t)b * p.max_blocks + min(t0 >> 6, p.max_blocks - 1)];
  };
  // wave w loads rows 16 w .. 16 w + 15 of the tile, through a buffer window
  // over its valid rows (rows past the sequence's end read as zero)
  float sc_next = 0.f;                 // E4M3: row scale of row tid / 4 of the next tile
  auto issue_tile = [&](int it) {
    const int b = it / n_tt, t0 = (it % n_tt) * X_T;
    const int valid = __builtin_amdgcn_readfirstlane(min(max(meta_len - t0, 0), X_T));
    int64_t r0 = 0;
    if (valid > 0) {
      if (p.block_table != nullptr) r0 = (int64_t)__builtin_amdgcn_readfirstlane(meta_blk) * X_T;
      else r0 = (int64_t)b * p.T_stride + t0;
    }
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.rows + r0 * ROW_BYTES), (short)0,
                                                        valid * ROW_BYTES, 0x00020000);
    if constexpr (FP8) {
      // two 512-code rows per load, plain order, into code buffer it & 1
      char* dst = smem + X_TILE + (it & 1) * X_CODES + wave * 16 * D_C;
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + q * 1024), 16, half * ROW_BYTES + 16 * l32,
                                                 (16 * wave + 2 * q) * ROW_BYTES, 0, 0);
      });
      const int t = tid >> 2;
      sc_next = t < valid ? p.row_scale[r0 + t] : 0.f;
    } else {
      // one 1 KB row per load: slot `lane` takes chunk lane ^ (row & 15)
      char* dst = smem + (it & 1) * X_TILE + wave * 16 * 1024;
      static_for<0, 16>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + r * 1024), 16, 16 * (lane ^ r),
                                                 (16 * wave + r) * ROW_BYTES, 0, 0);
      });
    }
    if (it + 1 < n_tiles) load_meta(it + 1);
  };
  // E4M3: thread tid converts row tid / 4, codes 128 (tid % 4) .. + 127
  auto convert_tile = [&](int it, float sc) {
    const int t = tid >> 2, qd = tid & 3;
    const char* src = smem + X_TILE + (it & 1) * X_CODES + t * D_C;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = 8 * qd + i;                   // 16-code chunk of the row
      i16x8 lo, hi;
      dequant16(*(const u32x4*)(src + 16 * m), sc, lo, hi);
      *(i16x8*)(smem + t * 1024 + 16 * ((2 * m) ^ (t & 15))) = lo;
      *(i16x8*)(smem + t * 1024 + 16 * ((2 * m + 1) ^ (t & 15))) = hi;
    }
  };
  // staged outputs of tile `it` -> K_nope or V: thread tid stores rows
  // 16 i + tid / 16, 16-byte chunk tid % 16
  // (the LDS reads are inline asm: the compiler would otherwise wait for the
  // tile loads just issued before reading LDS)
  auto store_tile = [&](int it) {
    const int b = it / n_tt, t0 = (it % n_tt) * X_T;
    uint16_t* dst = (part ? p.v : p.k_nope) + ((int64_t)b * p.T_pad + t0) * p.kv_ld + h * D_NOPE;
    const int cc = tid & 15, tr = tid >> 4;
    const uint32_t st = stage_a + (it & 1) * X_STAGE + tr * 256 + 16 * (cc ^ tr);
    i16x8 v[4];
    static_for<0, 4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      lds_read_b128<16 * i * 256>(v[i], st);     // row 16 i + tr: (t & 15) = tr
    });
    wait_lgkm<0>(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) *(i16x8*)(dst + (int64_t)(16 * i + tr) * p.kv_ld + 8 * cc) = v[i];
  };
  // fragment read offsets: row l32 (+ 32 tb), logical chunk 2 ks + half at
  // slot (2 ks + half) ^ (l32 & 15); for ks = 8 m + j that is 16 m + ((2 j +
  // half) ^ (l32 & 15)), so 8 lane offsets and an immediate cover all reads
  uint32_t boff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) boff[j] = l32 * 1024 + 16 * ((2 * j + half) ^ (l32 & 15));

  load_meta(0);
  issue_tile(0);
  // A fragments: weight row 32 wave + l32, columns 16 ks + 8 half .. + 7,
  // fetched while the first tile loads; both are complete before the loop
  // (so the compiler's own waits inside it have nothing left to wait for)
  i16x8 aw[D_C / 16];
  {
    const uint16_t* W = (part ? p.w_uvt : p.w_uk) + ((int64_t)h * D_NOPE + 32 * wave + l32) * D_C + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D_C / 16; ++ks) aw[ks] = ld16(W + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < D_C / 16; ++ks) touch_reg(aw[ks]);
  }
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int it = 0; it < n_tiles; ++it) {
    barrier_tile_ready();       // tile it landed; every wave is past tile it - 1's products
    uint32_t tb_a;
    if constexpr (FP8) {
      convert_tile(it, sc_next);
      barrier_lds();
      tb_a = smem_a;
    } else {
      tb_a = smem_a + (it & 1) * X_TILE;
    }
    if (it + 1 < n_tiles) issue_tile(it + 1);
    if (it > 0) store_tile(it - 1);

    i16x8 rb[X_RING][2];
    uint32_t ba[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ba[j] = tb_a + boff[j];
    auto issue_b = [&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      lds_read_b128<256 * (ks >> 3)>(rb[ks % X_RING][0], ba[ks & 7]);
      lds_read_b128<256 * (ks >> 3) + 32 * 1024>(rb[ks % X_RING][1], ba[ks & 7]);
    };
    static_for<0, X_RING - 1>(issue_b);
    static_for<0, D_C / 16>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      constexpr int last = D_C / 16 - 1;
      constexpr int ahead = (last - ks) < (X_RING - 1) ? (last - ks) : (X_RING - 1);
      if constexpr (ks + X_RING - 1 <= last) issue_b(std::integral_constant<int, ks + X_RING - 1>{});
      constexpr int slot = ks % X_RING;
      wait_lgkm<2 * ahead>(rb[slot][0], rb[slot][1]);
      const bf16x8 a = __builtin_bit_cast(bf16x8, aw[ks]);
      acc[0] = mfma32(a, __builtin_bit_cast(bf16x8, rb[slot][0]), acc[0]);
      acc[1] = mfma32(a, __builtin_bit_cast(bf16x8, rb[slot][1]), acc[1]);
    });

    // lane holds D[n = 32 wave + 8 g + 4 half + e][t = 32 tb + l32]: staged as
    // row t, logical chunk 4 wave + g (bytes 8 half ..) at slot chunk ^ (t & 15)
    const uint32_t st_a = stage_a + (it & 1) * X_STAGE;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = 32 * tb + l32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {acc[tb][4 * g], acc[tb][4 * g + 1], acc[tb][4 * g + 2], acc[tb][4 * g + 3]};
        lds_write_b64<0>(st_a + t * 256 + 16 * ((4 * wave + g) ^ (t & 15)) + 8 * half, pack_bf16x4(v4));
      }
      acc[tb] = f32x16{};
    }
  }
  barrier_tile_ready();
  store_tile(n_tiles - 1);
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
    // (in a scalar register: a buffer resource must be uniform)
    const int valid = __builtin_amdgcn_readfirstlane(max(0, min(KT, T_u - (int)r0)));
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
      // row t = ts + 4 half + o (o = 8 (r / 4) + r % 4, + 32 in s1) is
      // visible when o < lim - ts - 4 half: one distance, constant offsets
      const int d = lim - ts - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 8 * (r >> 2) + (r & 3);
        s0[r] = (o < d) ? s0[r] : -INFINITY;
        s1[r] = (o + 32 < d) ? s1[r] : -INFINITY;
      }
    }
    // (max3 only: no NaN-quieting moves; scores are finite or -inf)
    float mq[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 4 * c;
      mq[c] = max3f(max3f(s0[r], s0[r + 1], s0[r + 2]), max3f(s0[r + 3], s1[r], s1[r + 1]),
                    max3f(s1[r + 2], s1[r + 3], s1[r + 3]));
    }
    const float mraw = max3f(max3f(mq[0], mq[1], mq[2]), mq[3], mq[3]);
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
