// The balanced work plan of the split-T scan kernels, derived alike by every
// work-group from the device-resident sequence lengths.
#pragma once

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

constexpr int PLAN_THREADS = 256;             // work-group size the plan is written for
constexpr int PLAN_TILE = 64;                 // cached rows per tile
constexpr int PLAN_SCRATCH_BYTES = (2 * PLAN_THREADS + 4) * 8;   // LDS the plan borrows

// (decode_split_kernel carries its own inline copy of the same plan.)

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

// Pick this work-group's (sequence b, part j of parts, partial slot sl, row
// group g).  Returns false for a surplus work-group (uniform per work-group),
// which must exit.  NT: threads of the work-group (a multiple of 64, at most
// 1024); lds_scratch: (2 NT + 4) * 8 bytes of LDS, free on entry and on
// return.  The first work-group of a sequence records where its partials are
// (seg_first / seg_count).
template <int NT>
__device__ __forceinline__ bool plan_work_t(const DecodeParams& p, int64_t* lds_scratch, int& b, int& j,
                                            int& parts, int& sl, int& g) {
  constexpr int NTHREADS = NT;
  constexpr int NWAVES = NT / 64;
  constexpr int KT = PLAN_TILE;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // ---- the work plan.  Sequence b (n_t tiles of 64 rows, N tiles in all)
  // is scanned in parts(b) = clamp(n_t * n_ranges / N, 1, n_t) nearly equal parts,
  // so the work per part is about the same for every sequence (and exactly
  // n_ranges / B parts each when all lengths are equal).  Its parts take the
  // partial slots Qp[b] .. Qp[b] + parts(b) - 1 (Qp: prefix sum of parts),
  // fewer than n_ranges + B in all.  Every work-group derives the same plan
  // from the sequence lengths (chunked sums and two inclusive scans over the
  // NT chunks), then takes one (slot, row group) pair; the blockIdx -> pair
  // map puts consecutive slots (and the row groups of a slot) on one XCD
  // (shared L2) and the surplus work-groups of the launch at its end.
  {
    int64_t* scan = lds_scratch;           // 2 x NT entries
    int64_t* found = scan + 2 * NTHREADS;  // the slot's sequence and its first slot
    const int chunk = (p.B + NTHREADS - 1) / NTHREADS;
    const int c0 = min(p.B, tid * chunk), c1 = min(p.B, c0 + chunk);
    // inclusive prefix over the NT threads: shuffle scan within each wave,
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
      int64_t before = 0, all = 0;
#pragma unroll
      for (int w2 = 0; w2 < NWAVES; ++w2) {
        before += w2 < wave ? scan[w2] : 0;
        all += scan[w2];
      }
      __syncthreads();
      found[2] = all;
      return v + before;
    };
    int64_t tiles_mine = 0;
    for (int bb = c0; bb < c1; ++bb) tiles_mine += (p.seqlens[bb] + KT - 1) / KT;
    (void)inclusive_scan(tiles_mine);
    const int64_t total = uniform64(found[2]);
    // in [1, max(n_t, 1)]: every part holds a tile, and a sequence without
    // rows still gets one (empty) part, whose partial merges to zero
    auto parts_of = [&](int bb) -> int {
      const int64_t nt = (p.seqlens[bb] + KT - 1) / KT;
      if (total == 0 || nt == 0) return 1;
      const int64_t q = floor_div(nt * p.n_ranges, total);
      return (int)(q < 1 ? 1 : (q > nt ? nt : q));
    };
    int64_t parts_mine = 0;
    for (int bb = c0; bb < c1; ++bb) parts_mine += parts_of(bb);
    const int64_t pincl = inclusive_scan(parts_mine);
    const int n_slots = (int)uniform64(found[2]);
    const int n_real = n_slots * p.n_groups;
    const int per_xcd = (n_real + 7) / 8;
    const int w_item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (w_item >= n_real || blockIdx.x / 8 >= per_xcd) return false;   // surplus (uniform per work-group)
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
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane((int)found[0]);
    const int q0 = __builtin_amdgcn_readfirstlane((int)found[1]);
    __syncthreads();                       // the buffer is reused below
    parts = parts_of(b);
    j = sl - q0;
    if (g == 0 && tid == 0 && j == 0) {    // where sequence b's partials are
      p.seg_first[b] = q0;
      p.seg_count[b] = parts;
    }
  }
  return true;
}

__device__ __forceinline__ bool plan_work(const DecodeParams& p, int64_t* lds_scratch, int& b, int& j, int& parts,
                                          int& sl, int& g) {
  return plan_work_t<PLAN_THREADS>(p, lds_scratch, b, j, parts, sl, g);
}

}  // namespace mla
