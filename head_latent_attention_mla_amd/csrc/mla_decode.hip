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
// Work is balanced over ragged lengths: the 64-row tiles of all sequences are
// cut into equal ranges; each (range, row group) is one work-group, which
// writes, per sequence segment it covers, a normalised partial output row per
// query row and its log2-domain log-sum-exp.  The merge kernels combine the
// parts of each sequence.
#include "mla_common.h"
#include "mla_internal.h"
#include "mla_split_store.h"

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
static_assert(SPLIT_STAGE_BYTES <= 2 * TILE_BYTES, "partial staging fits the tile buffers");

__device__ __forceinline__ int lds_off(int t, int elem) {
  const int c = elem >> 3;
  return (t * CHUNKS + (c ^ tile_swz(t))) * 16 + (elem & 7) * 2;
}

// floor(a / b) for 0 <= a < 2^62, 0 < b: a double estimate corrected with
// exact integer products (cheaper than the 64-bit division routine).
__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = (int64_t)((double)a / (double)b);
  while (q > 0 && q * b > a) --q;
  while ((q + 1) * b <= a) ++q;
  return q;
}

// A value every lane holds alike, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// keep a value opaque to the optimiser (stops loop-invariant hoisting of
// per-lane address arithmetic that would otherwise pin registers)
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// LDS layout.  bf16 cache: two tile buffers (double-buffered loads) + P.
// FP8 cache: one bf16 tile buffer, two staging buffers for the e4m3 codes
// (double-buffered loads) + P; each tile's codes are decoded exactly to bf16
// into the tile buffer, and each row's scale is applied outside the products:
// to the row's scores, and to its probabilities in the value product.
constexpr int STAGE_BYTES = KT * ROWW;        // 36,864: e4m3 codes of one tile
static_assert(TILE_BYTES + 2 * STAGE_BYTES == 2 * TILE_BYTES, "layouts share the P offset");

// SPARSE (contiguous bf16 caches): the tile rows are the selected positions
// sel_idx[b, ts ..] of sequence b instead of rows ts.. -- the gather of sparse
// top-k decode fused into the tile loader; p.seqlens holds the selection
// counts (clamped here to [0, k_max]) and p.src_len the cache lengths.
template <bool PAGED, bool FP8, bool SPARSE = false>
__global__ __launch_bounds__(NTHREADS, 1) void decode_split_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * TILE_BYTES + P_BYTES];
  char* const pbuf = smem + 2 * TILE_BYTES;
  const uint32_t smem_a = lds_addr(smem);
  const uint32_t pbuf_a = smem_a + 2 * TILE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- the work plan (the same derivation as plan_work() in mla_plan.h, kept
  // inline here: as a call it changed this kernel's register allocation and
  // added spills inside the tile loop).  Sequence b (n_t tiles of 64 rows, N tiles in all)
  // is scanned in parts(b) = clamp(n_t * n_ranges / N, 1, n_t) nearly equal parts,
  // so the work per part is about the same for every sequence (and exactly
  // n_ranges / B parts each when all lengths are equal).  Its parts take the
  // partial slots Qp[b] .. Qp[b] + parts(b) - 1 (Qp: prefix sum of parts),
  // fewer than n_ranges + B in all.  Every work-group derives the same plan
  // from the sequence lengths (chunked sums and two inclusive scans over the
  // 256 chunks), then takes one (slot, row group) pair; the blockIdx -> pair
  // map puts consecutive slots on one XCD (shared L2) and the surplus
  // work-groups of the launch at its end.
  int b, j, parts;
  int sl;
  int g;
  int T;                                   // rows of sequence b (selected rows when SPARSE)
  auto seq_len = [&](int bb) -> int {
    if constexpr (SPARSE) return min(max(p.seqlens[bb], 0), p.k_max);
    return p.seqlens[bb];
  };
  {
    int64_t* scan = (int64_t*)pbuf;        // 2 x 256 entries; the probability buffer is idle here
    int64_t* found = scan + 2 * NTHREADS;  // the slot's sequence and its first slot
    const int chunk = (p.B + NTHREADS - 1) / NTHREADS;
    const int c0 = min(p.B, tid * chunk), c1 = min(p.B, c0 + chunk);
    // inclusive prefix over the 256 threads: shuffle scan within each wave,
    // then the wave totals through LDS; found[2] receives the grand total
    auto inclusive_scan = [&](int64_t mine) -> int64_t {
      int64_t v = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
      }
      if (lane == 63) scan[wave] = v;
      __syncthreads();
      int64_t before = 0;
      for (int w2 = 0; w2 < wave; ++w2) before += scan[w2];
      const int64_t all = scan[0] + scan[1] + scan[2] + scan[3];
      __syncthreads();
      found[2] = all;
      return v + before;
    };
    // the first length of the chunk (the whole chunk while B <= 256) is
    // fetched once and kept
    const int len_c0 = c0 < c1 ? seq_len(c0) : 0;
    auto len_at = [&](int bb) -> int { return bb == c0 ? len_c0 : seq_len(bb); };
    int64_t tiles_mine = 0;
    for (int bb = c0; bb < c1; ++bb) tiles_mine += (len_at(bb) + KT - 1) / KT;
    (void)inclusive_scan(tiles_mine);
    const int64_t total = uniform64(found[2]);
    // in [1, max(n_t, 1)]: every part holds a tile, and a sequence without
    // rows still gets one (empty) part, whose partial merges to zero
    auto parts_from_len = [&](int len) -> int {
      const int64_t nt = (len + KT - 1) / KT;
      if (total == 0 || nt == 0) return 1;
      const int64_t q = floor_div(nt * p.n_ranges, total);
      return (int)(q < 1 ? 1 : (q > nt ? nt : q));
    };
    const int parts_c0 = parts_from_len(len_c0);
    auto parts_of = [&](int bb) -> int { return bb == c0 ? parts_c0 : parts_from_len(seq_len(bb)); };
    int64_t parts_mine = 0;
    for (int bb = c0; bb < c1; ++bb) parts_mine += parts_of(bb);
    const int64_t pincl = inclusive_scan(parts_mine);
    const int n_slots = (int)uniform64(found[2]);
    const int n_real = n_slots * p.n_groups;
    const int per_xcd = (n_real + 7) / 8;
    const int w_item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (w_item >= n_real || blockIdx.x / 8 >= per_xcd) return;   // surplus (uniform per work-group)
    g = w_item % p.n_groups;
    sl = w_item / p.n_groups;
    if (pincl - parts_mine <= sl && sl < pincl) {
      int bb = c0;
      int64_t q = pincl - parts_mine;
      while (q + parts_of(bb) <= sl) {
        q += parts_of(bb);
        ++bb;
      }
      found[0] = bb;
      found[1] = q;
      found[3] = parts_of(bb);
      found[4] = len_at(bb);
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane((int)found[0]);
    const int q0 = __builtin_amdgcn_readfirstlane((int)found[1]);
    parts = __builtin_amdgcn_readfirstlane((int)found[3]);
    T = __builtin_amdgcn_readfirstlane((int)found[4]);
    __syncthreads();                       // the buffer is reused below
    j = sl - q0;
    if (g == 0 && tid == 0 && j == 0) {    // where sequence b's partials are
      p.seg_first[b] = q0;
      p.seg_count[b] = parts;
    }
  }
  if (p.fixup) {
    // fix-up after the FP8-arithmetic scan (same plan): with E4M3 queries and
    // weights a row stays within the FP8 bar while its largest probability is
    // at most 1/32 of its total; recompute this (sequence, row group) only if
    // one of its rows passes that, i.e. max over parts of the part maxima
    // against the merged log-sum-exp (log2 domain) exceeds -5
    bool peaked = false;
    if (tid < 128 && g * 128 + tid < p.R) {
      const int64_t row = g * 128 + tid;
      const int s0 = p.seg_first[b], ns = p.seg_count[b];
      float m = -INFINITY, lmax = -INFINITY;
      for (int s = 0; s < ns; ++s) {
        m = fmaxf(m, p.part_mrun[(s0 + s) * (int64_t)p.R + row]);
        lmax = fmaxf(lmax, p.part_lse[(s0 + s) * (int64_t)p.R + row]);
      }
      float sum = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float l = p.part_lse[(s0 + s) * (int64_t)p.R + row];
        sum += l == -INFINITY ? 0.f : exp2f(l - lmax);
      }
      peaked = sum > 0.f && m - (lmax + log2f(sum)) > -5.0f;
    }
    // any row of the work-group: one word per wave in the idle probability buffer
    int* const any = (int*)pbuf;
    const bool wave_any = __builtin_amdgcn_ballot_w64(peaked) != 0;
    if (lane == 0) any[wave] = wave_any ? 1 : 0;
    __syncthreads();
    const int flagged = any[0] | any[1] | any[2] | any[3];
    __syncthreads();                         // the buffer is reused below
    if (flagged == 0) return;                // uniform per work-group
  }
  const int nt_b = (T + KT - 1) / KT;
  const int t_begin = (int)floor_div((int64_t)j * nt_b, parts) * KT;
  const int t_end = min(T, (int)floor_div((int64_t)(j + 1) * nt_b, parts) * KT);
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + KT - 1) / KT : 0;

  // ---- rows owned by this wave for the score phase
  const int own_r = g * 128 + wave * 32 + l32;
  const bool own_ok = own_r < p.R;
  const bool wave_on = g * 128 + wave * 32 < p.R;
  const int jq = own_ok ? own_r / p.H : 0;
  const int visible = p.causal ? (T - p.s_q + jq + 1) : T;
  const int lim = min(visible, t_end);

  // the latent queries of the owned rows, B fragments of the 36 k-steps
  // (nothing waits for them before the first tile's barrier, so they load
  // together with the first tile).  Rows past the last query row take row
  // 0's query: their scores are computed but never stored.
  bf16x8 qf[ROWW / 16];
  {
    const uint16_t* qrow = p.q_lat + ((int64_t)b * p.R + (own_ok ? own_r : 0)) * ROWW + half * 8;
#pragma unroll
    for (int ks = 0; ks < ROWW / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const i16x8*)(qrow + ks * 16));
  }

  // ---- tile loader.  Wave w copies rows 16w..16w+15 of the tile: 18 loads
  // of 64 lanes x 16 B, each filling 1 KB of LDS in order.  The chunk that
  // lane l fetches for LDS slot 64 k + l follows the XOR swizzle.  Loads k
  // and k + 9 cover the same slots of rows 8 apart (9 loads fill 8 rows), whose
  // XORs differ by 2, so 18 per-lane byte offsets within an 8-row group (<
  // 2^14, packed two per register) cover all loads; the second group's 8-row
  // displacement is an immediate.  The buffer window of a tile ends at the
  // sequence's last row, so rows past it read as zero.
  uint32_t loff[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 18; ++k) {
    const int s = 64 * (k % 9) + lane;
    const int tl = s / CHUNKS;
    const int c = (s - tl * CHUNKS) ^ tile_swz(tl + (k >= 9 ? 8 : 0));
    loff[k >> 1] |= (uint32_t)(tl * ROWW * 2 + c * 16) << (16 * (k & 1));
  }
  const char* rows = (const char*)p.rows;
  constexpr int ELEM = FP8 ? 1 : 2;            // bytes per cached element
  // per-tile load state: buffer window over the tile's rows
  auto tile_base = [&](int tile) -> int64_t {  // element index of the tile's first row
    const int ts = t_begin + tile * KT;
    // (the table entry moved to a scalar register: a buffer resource must be uniform)
    if (PAGED) return (int64_t)__builtin_amdgcn_readfirstlane(p.block_table[(int64_t)b * p.max_blocks + (ts >> 6)]) * KT;
    return (int64_t)b * p.T_stride + ts;
  };
  // live = false gives an empty window: its loads fetch nothing and write zeros
  auto tile_rsrc = [&](int tile, bool live) {
    if constexpr (SPARSE) {
      // the whole sequence: a selected position outside it reads as a zero row
      const int src_rows = __builtin_amdgcn_readfirstlane(live ? p.src_len[b] : 0);   // uniform
      return __builtin_amdgcn_make_buffer_rsrc((void*)(rows + (int64_t)b * p.T_stride * ROWW * ELEM), (short)0,
                                               src_rows * ROWW * ELEM, 0x00020000);
    }
    const int ts = t_begin + tile * KT;
    const int valid = __builtin_amdgcn_readfirstlane(live ? min(KT, T - ts) : 0);   // uniform
    return __builtin_amdgcn_make_buffer_rsrc((void*)(rows + tile_base(tile) * ROWW * ELEM), (short)0,
                                             valid * ROWW * ELEM, 0x00020000);
  };
  // SPARSE: row offsets of this wave's 16 tile rows, relative to the loader's
  // 8-row pattern (adj[r] + the pattern offset = position * 1152 + chunk);
  // rows past the selection or outside the sequence point past the window.
  // The selected positions are fetched one tile ahead of their use, with a
  // vector load (lane l < 16 -> row 16 wave + l), so the wait for them is
  // the tile loads' own.
  constexpr uint32_t OOB = 0x40000000u;
  uint32_t adj[16];
  int sel_v = -1;
  auto fetch_rows = [&](int tile) {
    if constexpr (SPARSE) {
      const int t = t_begin + tile * KT + 16 * wave + (lane & 15);
      sel_v = t < T ? p.sel_idx[(int64_t)b * p.k_max + t] : -1;
    }
  };
  const int src_b = SPARSE ? p.src_len[b] : 0;
  auto set_rows = [&]() {
    if constexpr (SPARSE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = __builtin_amdgcn_readlane(sel_v, r);
        const uint32_t a = (pos >= 0 && pos < src_b) ? (uint32_t)(pos - (r & 7)) * (ROWW * 2) : OOB;
        adj[r] = __builtin_amdgcn_readfirstlane(a);   // keep the offsets in scalar registers
      }
    }
  };
  const int soff = wave * (16 * ROWW * ELEM);
  auto issue_load = [&](__amdgpu_buffer_rsrc_t rsrc, int buf, auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (FP8) {
      // 16 rows of codes are 9 KB contiguous: plain lane order into staging
      char* dst = smem + TILE_BYTES + buf * STAGE_BYTES + wave * (16 * ROWW) + k * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, lane * 16, soff + k * 1024, 0, 0);
    } else {
      constexpr int k9 = k % 9;
      const uint32_t vo = (loff[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
      char* dst = smem + buf * TILE_BYTES + wave * (16 * ROWW * 2) + k * 1024;
      if constexpr (SPARSE) {
        // load k covers pattern rows a and a + 1 (lanes from `split` on)
        constexpr int a = (64 * k9) / CHUNKS;
        constexpr int split = CHUNKS * (a + 1) - 64 * k9;
        constexpr int r = a + (k >= 9 ? 8 : 0);
        uint32_t row_adj = adj[r];
        if constexpr (split < 64) row_adj = lane < split ? adj[r] : adj[r + 1];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, vo + row_adj, 0, 0, CPOL_STREAM);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 16, vo,
                                                 soff + (k >= 9 ? 8 * ROWW * 2 : 0), 0, CPOL_STREAM);
      }
    }
  };
  constexpr int NLOADS = FP8 ? 9 : 18;         // 1 KB loads per wave per tile
  auto issue_tile = [&](int tile, int buf) {
    const auto rsrc = tile_rsrc(tile, true);
    static_for<0, NLOADS>([&](auto kc) { issue_load(rsrc, buf, kc); });
  };
  // FP8: thread tid converts row tid / 4 of a tile, quarter tid % 4 (144 codes);
  // its row scale is fetched one tile ahead
  const int cv_row = tid >> 2, cv_q = tid & 3;
  auto load_scale = [&](int tile) -> float {
    const int ts = t_begin + tile * KT;
    return (ts + cv_row < T) ? p.row_scale[tile_base(tile) + cv_row] : 0.f;
  };
  // every E4M3 value is a bf16 value: the codes are decoded exactly (gfx950's
  // scaled conversion with scale 1, two codes per instruction).  The nine
  // 16-code chunks are read first (one LDS round trip, not nine).  The row's
  // scale goes to each wave's copy of the tile's 64 scales, at the head of
  // that wave's probability fragments (idle until the wave writes them).
  auto convert_tile = [&](int buf, float scale) {
    const char* src = smem + TILE_BYTES + buf * STAGE_BYTES + cv_row * ROWW + cv_q * 9 * 16;
    u32x4 w[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = *(const u32x4*)(src + i * 16);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int m = cv_q * 9 + i;                 // 16-code chunk of the row
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        o[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][d], 1.0f, false));
        o[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][d], 1.0f, true));
      }
      *(u32x4*)(smem + lds_off(cv_row, 16 * m)) = u32x4{o[0], o[1], o[2], o[3]};
      *(u32x4*)(smem + lds_off(cv_row, 16 * m + 8)) = u32x4{o[4], o[5], o[6], o[7]};
    }
    if (cv_q == 0) {
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) *(float*)(pbuf + w2 * 4096 + cv_row * 4) = scale;
    }
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
    const int sw = tile_swz(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i) qoff[i] = l32 * (CHUNKS * 16) + 16 * ((2 * i + half) ^ sw);
  }
  // value-phase transposed-read geometry: lane reads row 16 kap + 4 half +
  // rsel (+8), columns 128 wave + 32 cb + 16 grp + csel; the XOR pattern of
  // that row is lane-constant (the +8 row's differs by 2) and only the parity
  // of cb changes the swizzled chunk, so four lane offsets cover every read
  uint32_t pvoff[2][2];   // [row + 8][cb parity]
  {
    const int grp = (lane >> 4) & 1;
    const int rsel = (lane & 15) >> 2;
    const int csel = 4 * (lane & 3);
    const int trow = 4 * half + rsel;
#pragma unroll
    for (int r8 = 0; r8 < 2; ++r8) {
      const int sw = tile_swz(trow + 8 * r8);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int chunk = 16 * wave + 4 * i + 2 * grp + (csel >> 3);
        pvoff[r8][i] = trow * (CHUNKS * 16) + 16 * (chunk ^ sw) + (csel & 7) * 2;
      }
    }
  }
  const uint32_t pb_lane = pbuf_a + lane * 16;

  // No clearing of the tile buffers is needed: every tile row the loop reads
  // was written by the loads (rows outside a tile's window load as zeros) or,
  // for FP8 caches, by the conversion of all 64 staged rows.

  float sc_cur = 0.f, sc_next = 0.f;            // FP8 row scales (this tile, next)
  if (n_tiles > 0) {
    fetch_rows(0);
    set_rows();
    issue_tile(0, 0);
    fetch_rows(1);
    if constexpr (FP8) sc_next = load_scale(0);
  }

  for (int tile = 0; tile < n_tiles; ++tile) {
    barrier_tile_ready();   // tile ready; every wave is past the previous value phase
    const bool has_next = tile + 1 < n_tiles;
    // past the last tile the loads still run (no branch in the loop) but
    // read an empty window into the idle buffer
    const auto next = tile_rsrc(has_next ? tile + 1 : tile, has_next);
    if constexpr (SPARSE) {
      // positions of tile + 1 (landed with the tile); past the last tile the
      // window is empty and the offsets do not matter
      set_rows();
      fetch_rows(tile + 2);
    }
    const int next_buf = (tile + 1) & 1;
    uint32_t tb_a;
    if constexpr (FP8) {
      // decode the staged codes into the bf16 tile buffer (rows past the
      // sequence end load as zero codes and have scale 0)
      sc_cur = sc_next;
      if (has_next) sc_next = load_scale(tile + 1);
      convert_tile(tile & 1, sc_cur);
      barrier_lds();
      tb_a = smem_a;
    } else {
      tb_a = smem_a + (tile & 1) * TILE_BYTES;
    }
    const int ts = t_begin + tile * KT;

    // ================= score phase (owned rows) =================
    bf16x8 pk[2][2];
    if (wave_on) {
      f32x16 s0, s1;
      uint32_t qa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qa[i] = tb_a + qoff[i];
      // k-steps of A fragments in flight (the sparse variant gives one up for
      // the prefetched positions)
      constexpr int QK_AHEAD = (SPARSE || FP8) ? 2 : 3;
      i16x8 ra[QK_AHEAD + 1][2];
      auto issue_qk = [&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        lds_read_b128<128 * (ks >> 2)>(ra[ks % (QK_AHEAD + 1)][0], qa[ks & 3]);
        lds_read_b128<128 * (ks >> 2) + 32 * CHUNKS * 16>(ra[ks % (QK_AHEAD + 1)][1], qa[ks & 3]);
      };
      static_for<0, QK_AHEAD>(issue_qk);
      static_for<0, ROWW / 16>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int ahead = (ROWW / 16 - 1 - ks) < QK_AHEAD ? (ROWW / 16 - 1 - ks) : QK_AHEAD;
        if constexpr (ks + QK_AHEAD < ROWW / 16) issue_qk(std::integral_constant<int, ks + QK_AHEAD>{});
        // the next tile's loads ride along, one per two k-steps
        constexpr int every = FP8 ? 4 : 2;
        if constexpr (ks % every == 0 && ks / every < NLOADS) {
          issue_load(next, next_buf, std::integral_constant<int, ks / every>{});
        }
        constexpr int slot = ks % (QK_AHEAD + 1);
        wait_lgkm<2 * ahead>(ra[slot][0], ra[slot][1]);
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra[slot][0]);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra[slot][1]);
        if constexpr (ks == 0) {
          mfma32_v0(s0, a0, qf[ks]);
          mfma32_v0(s1, a1, qf[ks]);
        } else {
          mfma32_v(s0, a0, qf[ks]);
          mfma32_v(s1, a1, qf[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the k-step's waits, reads and MFMAs in order
      });
      mfma_v_drain(s0, s1);
      // FP8: the scales of the lane's 32 tile rows, 8 (r / 4) + 4 half + r % 4
      // (group g = r / 4) and 32 more (group 4 + g), read from this wave's
      // copy four groups at a time
      const uint32_t scl_a = pbuf_a + wave * 4096 + 16 * half;
      auto read_scales = [&](f32x4 (&sg)[4], auto g0c) {
        constexpr int g0 = decltype(g0c)::value;
        static_for<0, 4>([&](auto gc) {
          constexpr int g8 = g0 + decltype(gc)::value;
          i16x8 t;
          lds_read_b128<32 * g8>(t, scl_a);
          sg[g8 - g0] = __builtin_bit_cast(f32x4, t);
        });
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < 4; ++i) touch_reg(sg[i]);
      };
      if constexpr (FP8) {
        f32x4 sg[4];
        read_scales(sg, std::integral_constant<int, 0>{});
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[r] *= sg[r >> 2][r & 3];
        read_scales(sg, std::integral_constant<int, 4>{});
#pragma unroll
        for (int r = 0; r < 16; ++r) s1[r] *= sg[r >> 2][r & 3];
      }

      // mask only where the tile reaches past a row's last visible row
      if (__builtin_amdgcn_ballot_w64(ts + KT > lim) != 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = ts + 8 * (r >> 2) + 4 * half + (r & 3);
          s0[r] = (t < lim) ? s0[r] : -INFINITY;
          s1[r] = (t + 32 < lim) ? s1[r] : -INFINITY;
        }
      }
      // running maximum on raw scores (the scale is positive): four
      // independent chains, then their maximum
      float mq[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * c;
        mq[c] = max3f(max3f(s0[r], s0[r + 1], s0[r + 2]), max3f(s0[r + 3], s1[r], s1[r + 1]),
                      max3f(s1[r + 2], s1[r + 3], s1[r + 3]));
      }
      const float mraw = max3f(max3f(mq[0], mq[1], mq[2]), mq[3], mq[3]);
      const float mx = max_halves(mraw) * p.scale_log2;
      // reference update, branch-free: the first visible scores set it; later
      // it moves up in steps of REF_STEP only when the maximum passes it by more
      const bool first = m_ref == -INFINITY;
      const float over = (mx - m_ref - REF_STEP) * (1.0f / REF_STEP);
      const int kraw = (!first && over > 0.f) ? (int)ceilf(over) : 0;
      const int kstep = kraw > 7 ? 7 : kraw;
      l_sum = kstep == 7 ? 0.f : l_sum * __builtin_amdgcn_exp2f(-REF_STEP * kstep);
      m_ref = (first || kstep == 7) ? mx : m_ref + REF_STEP * kstep;
      const float nbase = (m_ref == -INFINITY) ? 0.f : -m_ref;
      float lq[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
        // value-product weights p * (row scale), rounded to bf16; the
        // normaliser is the sum of the probabilities themselves
        f32x4 sg[4];
        read_scales(sg, std::integral_constant<int, 0>{});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, nbase));
          lq[r & 3] += e0;
          pk[0][r >> 3][r & 7] = to_bf16(e0 * sg[r >> 2][r & 3]);
        }
        read_scales(sg, std::integral_constant<int, 4>{});
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, nbase));
          lq[r & 3] += e1;
          pk[1][r >> 3][r & 7] = to_bf16(e1 * sg[r >> 2][r & 3]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pk[0][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.scale_log2, nbase)));
          pk[1][r >> 3][r & 7] = to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.scale_log2, nbase)));
        }
        // row sum of the rounded probabilities, two at a time in four chains
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const bf16x2 pr = {pk[sb][j][e], pk[sb][j][e + 1]};
              lq[2 * j + sb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lq[2 * j + sb], false);
            }
      }
      l_sum += sum_halves((lq[0] + lq[1]) + (lq[2] + lq[3]));
      if (kstep != 0) {
        // sign bits of the fragment's first three probabilities carry the
        // reference step (both lane halves, so every reader lane sees it)
#pragma unroll
        for (int e = 0; e < 3; ++e)
          if (kstep & (1 << e)) pk[0][0][e] = -pk[0][0][e];
      }
    } else {
      if (has_next) static_for<0, NLOADS>([&](auto kc) { issue_load(next, next_buf, kc); });
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

    // ================= value phase (128 columns x all rows) =================
    // 16 units u = 4 kap + cb, each 4 MFMAs (one per row block rb) sharing one
    // transposed tile fragment A[u]; the probability fragments B[kap] of the
    // 4 row blocks serve the 4 units of a kap.  A runs in a ring of three
    // (issued two units ahead), B in two buffers (issued at unit cb = 2 of the
    // previous kap); every wait names the exact number of younger LDS reads.
    {
      const uint32_t pa0 = tb_a + pvoff[0][0];
      const uint32_t pa1 = tb_a + pvoff[0][1];
      const uint32_t pa0_8 = tb_a + pvoff[1][0];
      const uint32_t pa1_8 = tb_a + pvoff[1][1];
      i16x8 bq[2][4];
      i16x4 tr[3][2];
      auto issue_a = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int kap = u >> 2, cb = u & 3;
        constexpr int off = 16 * kap * (CHUNKS * 16) + 128 * (cb >> 1);
        lds_read_tr16<off>(tr[u % 3][0], (cb & 1) ? pa1 : pa0);
        lds_read_tr16<off + 8 * CHUNKS * 16>(tr[u % 3][1], (cb & 1) ? pa1_8 : pa0_8);
      };
      auto issue_b = [&](auto kc) {
        constexpr int kap = decltype(kc)::value;
        static_for<0, 4>([&](auto rbc) {
          constexpr int rb = decltype(rbc)::value;
          lds_read_b128<(rb * 4 + kap) * 1024>(bq[kap & 1][rb], pb_lane);
        });
      };
      // the first transposed tile reads only need the tile: issue them before
      // the barrier that publishes the probabilities
      issue_a(std::integral_constant<int, 0>{});
      issue_a(std::integral_constant<int, 1>{});
      barrier_lds();   // probabilities of all 128 rows visible
      issue_b(std::integral_constant<int, 0>{});
      static_for<0, 16>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int kap = u >> 2, cb = u & 3;
        // reads issued after A[u] (and after B[kap] when cb == 0): A[u + 1]
        // (2) unless it is the last unit, plus B[kap + 1] (4) when cb == 3
        constexpr int younger = (u == 15 ? 0 : 2) + ((cb == 3 && kap < 3) ? 4 : 0) - (u == 0 ? 2 : 0);
        if constexpr (cb == 0) {
          wait_lgkm<younger>(tr[u % 3][0], tr[u % 3][1], bq[kap & 1][0], bq[kap & 1][1], bq[kap & 1][2],
                             bq[kap & 1][3]);
        } else {
          wait_lgkm<younger>(tr[u % 3][0], tr[u % 3][1]);
        }
        if constexpr (u + 2 < 16) issue_a(std::integral_constant<int, u + 2>{});
        if constexpr (cb == 2 && kap < 3) issue_b(std::integral_constant<int, kap + 1>{});
        if constexpr (u == 0) {
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
            for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
              for (int rb = 0; rb < 4; ++rb) scale_acc(acc[c2][rb], alpha[rb]);
          }
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) {
            u32x4 v = __builtin_bit_cast(u32x4, bq[0][rb]);
            v[0] &= 0x7FFF7FFFu;
            v[1] &= 0x7FFF7FFFu;
            bq[0][rb] = __builtin_bit_cast(i16x8, v);
          }
        }
        const bf16x8 a = join_tr(tr[u % 3][0], tr[u % 3][1]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[cb][rb] = mfma32(a, __builtin_bit_cast(bf16x8, bq[kap & 1][rb]), acc[cb][rb]);
        __builtin_amdgcn_sched_barrier(0);   // a unit's MFMAs stay ahead of the next unit's wait
      });
    }
  }

  // ---- epilogue: share each row's normaliser, write the normalised partials.
  // The partials are staged over the tile buffers: the loads issued past the
  // last tile must have landed first.
  barrier_tile_ready();
  float* const lsh = (float*)pbuf;          // [128] l_sum
  if (half == 0) lsh[wave * 32 + l32] = l_sum;
  barrier_lds();

  // the tile buffers are idle: the partial rows are staged there
  const int64_t pbase = (int64_t)sl * p.R;
  store_split_partials(p, acc, lsh, smem, pbase, g, wave, lane);
  if (half == 0 && own_ok) p.part_lse[pbase + own_r] = l_sum > 0.f ? m_ref + log2f(l_sum) : -INFINITY;
}

// Merge the partials of each query row: the parts of sequence b sit in
// slots seg_first[b] .. seg_first[b] + seg_count[b] - 1; weights
// 2^(lse_s - max_s), then the weighted mean of the normalised partial rows.
// One thread per (row, 4 latent columns); partial and output rows are
// contiguous, so every load and store is coalesced.
template <bool PB16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      const int32_t* __restrict__ seg_first,
                                                      const int32_t* __restrict__ seg_count, int B, int R,
                                                      void* o_lat, int o_bf16, float* lse_out) {
  const int64_t row_g = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);   // b * R + row
  if (row_g >= (int64_t)B * R) return;
  const int b = (int)(row_g / R);
  const int row = (int)(row_g - (int64_t)b * R);
  const int c4 = (threadIdx.x & 127) * 4;
  const int64_t s0 = seg_first[b];
  const int ns = seg_count[b];
  // splits four at a time, all loads of a group in flight together (the
  // first group's with the log-sum-exps); added in split order (the same
  // order and arithmetic as combine_out_kernel's merge)
  constexpr int SG = 4;
  float l[SG];
  PartRaw<PB16> d[SG];
  auto load_group = [&](int g0) {
#pragma unroll
    for (int u = 0; u < SG; ++u) {
      const int s = max(min(g0 + u, ns - 1), 0);
      l[u] = part_lse[(s0 + s) * R + row];
      d[u] = part_load<PB16>(part_o, ((s0 + s) * R + row) * D_C + c4);
    }
  };
  load_group(0);
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < SG; ++u) mx = fmaxf(mx, l[u]);
  for (int g0 = SG; g0 < ns; g0 += SG) {
#pragma unroll
    for (int u = 0; u < SG; ++u) mx = fmaxf(mx, part_lse[(s0 + min(g0 + u, ns - 1)) * R + row]);
  }
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < ns; g0 += SG) {
    if (g0 > 0) load_group(g0);
    float w[SG];
#pragma unroll
    for (int u = 0; u < SG; ++u) w[u] = (g0 + u < ns && l[u] != -INFINITY) ? exp2f(l[u] - mx) : 0.f;
#pragma unroll
    for (int u = 0; u < SG; ++u) {
      if (w[u] == 0.f) continue;
      wsum += w[u];
      acc += w[u] * part_vals<PB16>(d[u]);
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  acc *= inv;
  part_store(o_lat, row_g * D_C + c4, acc, o_bf16 != 0);
  if (lse_out != nullptr && (threadIdx.x & 127) == 0)
    lse_out[row_g] = wsum > 0.f ? (mx + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_decode_split(const DecodeParams& p, hipStream_t stream) {
  const int grid = 8 * p.work_per_xcd;
  if (p.sel_idx != nullptr) {
    hipLaunchKernelGGL((decode_split_kernel<false, false, true>), dim3(grid), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
  }
  if (p.paged) {
    if (p.fp8)
      hipLaunchKernelGGL((decode_split_kernel<true, true>), dim3(grid), dim3(NTHREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_split_kernel<true, false>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  } else {
    if (p.fp8)
      hipLaunchKernelGGL((decode_split_kernel<false, true>), dim3(grid), dim3(NTHREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_split_kernel<false, false>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* part_o, int part_bf16, const float* part_lse, const int32_t* seg_first,
                          const int32_t* seg_count, int B, int R, void* o_lat, int o_bf16, float* lse,
                          hipStream_t stream) {
  const int64_t rows = (int64_t)B * R;
  const dim3 grid((unsigned)((rows + 1) / 2));
  if (part_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, part_o, part_lse, seg_first, seg_count, B,
                       R, o_lat, o_bf16, lse);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, part_o, part_lse, seg_first, seg_count, B,
                       R, o_lat, o_bf16, lse);
  return hipGetLastError();
}

}  // namespace mla
