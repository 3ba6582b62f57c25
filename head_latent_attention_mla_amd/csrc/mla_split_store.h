// Partial-output store shared by the split-T scan kernels.
//
// At the end of its part, a work-group holds the unnormalised output of its
// 128 query rows over all 512 latent columns: wave w, accumulator
// acc[cb][rb], lane (l32, half) and register r hold latent column
// 128 w + 32 cb + 8 (r / 4) + 4 half + r % 4 of query row 32 rb + l32 (the
// MFMA 32x32 output layout of O^T).  Written straight from registers, every
// store instruction would touch 32 partial rows, 16 bytes each.  bf16
// partials are therefore first transposed through LDS, which is idle by then,
// and then written one whole 1 KB row per wave instruction.
#pragma once

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

constexpr int SPLIT_STAGE_PITCH = D_C * 2 + 16;                 // bytes per staged row (16 B pad)
constexpr int SPLIT_STAGE_BYTES = 128 * SPLIT_STAGE_PITCH;      // 133,120

// Normalise (row normalisers in lsh[128], accumulators in units of unscale)
// and store the partial rows of row group g into slot rows pbase + g * 128 +
// ...  stage: SPLIT_STAGE_BYTES of
// LDS, unused by anything else from here on; lsh must not overlap it.  All
// 256 threads of the work-group call this together.
__device__ __forceinline__ void store_split_partials(const DecodeParams& p, const f32x16 (&acc)[4][4],
                                                     const float* lsh, char* stage, int64_t pbase, int g,
                                                     int wave, int lane, float unscale = 1.0f) {
  const int half = lane >> 5, l32 = lane & 31;
  if (p.part_bf16) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = rb * 32 + l32;
      const float l = lsh[r];
      const float inv = l > 0.f ? unscale / l : 0.f;
      char* const srow = stage + r * SPLIT_STAGE_PITCH + (wave * 128 + 4 * half) * 2;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = {acc[cb][rb][4 * q4] * inv, acc[cb][rb][4 * q4 + 1] * inv, acc[cb][rb][4 * q4 + 2] * inv,
                           acc[cb][rb][4 * q4 + 3] * inv};
          *(uint64_t*)(srow + (cb * 32 + 8 * q4) * 2) = pack_bf16x4(v);
        }
    }
    barrier_lds();
    // wave w writes rows w, w + 4, ...; lane l covers bytes 16 l .. 16 l + 15
    const int n_rows = min(128, p.R - g * 128);
    uint16_t* const dst = (uint16_t*)p.part_o + (pbase + g * 128) * D_C + lane * 8;
    for (int r = wave; r < n_rows; r += 4) {
      const u32x4 v = *(const u32x4*)(stage + r * SPLIT_STAGE_PITCH + lane * 16);
      *(u32x4*)(dst + (int64_t)r * D_C) = v;
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = g * 128 + rb * 32 + l32;
      if (row >= p.R) continue;
      const float l = lsh[rb * 32 + l32];
      const float inv = l > 0.f ? unscale / l : 0.f;
      float* const prow = (float*)p.part_o + (pbase + row) * D_C + wave * 128 + 4 * half;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(f32x4*)(prow + cb * 32 + 8 * q4) = f32x4{acc[cb][rb][4 * q4] * inv, acc[cb][rb][4 * q4 + 1] * inv,
                                                     acc[cb][rb][4 * q4 + 2] * inv, acc[cb][rb][4 * q4 + 3] * inv};
    }
  }
}

}  // namespace mla
