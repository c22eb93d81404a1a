// Tile-level helpers shared by the MFMA kernels: key-tile ranges from the
// row-block interval envelopes, whole-tile visibility tests and per-row
// column bitmasks for tiles some rows see only partly.
#pragma once

#include "common.h"

namespace hstu {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t low_bits(int n) {  // n in [0, 32]
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// Visibility bits of 32 consecutive columns [cb, cb+32) for one row.
__device__ __forceinline__ uint32_t col_mask32(const int* lo, const int* hi, int ni, int cb) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    if (j < ni) {
      const int a = min(max(lo[j] - cb, 0), 32);
      const int e = min(max(hi[j] - cb, 0), 32);
      m |= low_bits(e) & ~low_bits(a);
    }
  }
  return m;
}

struct TileRanges {
  int a[kMaxNI], e[kMaxNI];      // live key tiles per interval, inclusive (empty: a > e)
  int ilo[kMaxNI], ihi[kMaxNI];  // intersection envelope (columns)
  int tmax;
};

__device__ __forceinline__ bool tile_live(const TileRanges& R, int ni, int t) {
  bool r = false;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j)
    if (j < ni) r = r || (t >= R.a[j] && t <= R.e[j]);
  return r;
}

__device__ __forceinline__ bool tile_full(const TileRanges& R, int ni, int c0, int c1) {
  bool r = false;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j)
    if (j < ni) r = r || (R.ilo[j] <= c0 && c1 <= R.ihi[j]);
  return r;
}

__device__ __forceinline__ int next_live(const TileRanges& R, int ni, int t) {
  for (; t <= R.tmax; ++t)
    if (tile_live(R, ni, t)) return t;
  return -1;
}

// Envelope of the query rows [r0, r0 + rows) (whole row blocks) -> key tiles.
__device__ __forceinline__ void tile_ranges(const Prep& P, int b, int r0, int rows, int L, int ni,
                                            int bn, TileRanges& R) {
  const int rb0 = r0 / kRB;
  const int nrb = min((rows + kRB - 1) / kRB, (L - r0 + kRB - 1) / kRB);
  const int4* env = P.env + (int64_t)(P.rb_off[b] + rb0) * ni;
  R.tmax = -1;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    int ulo = L, uhi = 0, ilo = INT32_MIN, ihi = INT32_MAX;
    if (j < ni) {
      for (int r = 0; r < nrb; ++r) {
        const int4 v = env[r * ni + j];
        ulo = min(ulo, v.x);
        uhi = max(uhi, v.y);
        ilo = max(ilo, v.z);
        ihi = min(ihi, v.w);
      }
    }
    if (ulo < uhi) {
      R.a[j] = ulo / bn;
      R.e[j] = (uhi - 1) / bn;
      R.tmax = max(R.tmax, R.e[j]);
    } else {
      R.a[j] = 1;
      R.e[j] = 0;
    }
    R.ilo[j] = ilo;
    R.ihi[j] = ihi;
  }
}


// Whether row block `rb` (envelope row `env`) reaches key columns [c0, c1),
// and whether every valid row of it sees all of them.
__device__ __forceinline__ void block_vs_cols(const int4* env, int ni, int c0, int c1, bool& live,
                                              bool& full) {
  live = false;
  full = false;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    if (j < ni) {
      const int4 e = env[j];
      live = live || (e.x < e.y && e.x < c1 && e.y > c0);
      full = full || (e.z <= c0 && c1 <= e.w);
    }
  }
}

}  // namespace hstu
