// Tile-level helpers shared by the MFMA kernels:
//   * the interval envelope of a block of query rows (from the per-row-block
//     envelopes the decoder wrote), and the key tiles it reaches;
//   * a per-workgroup list of those key tiles in LDS, built 64 tiles at a time
//     by one wave with a ballot, each entry flagged "full" when every valid
//     row of the block sees the whole tile (no per-element mask needed);
//   * per-row column bitmasks for tiles some rows see only partly;
//   * buffer resources whose hardware range check returns zeros for rows past
//     the end of a sequence (no predication on the loads).
#pragma once

#include "common.h"

namespace hstu {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kListWin = 64;        // key tiles per list window

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

// Union [ulo, uhi) and intersection [ilo, ihi) envelopes of every interval
// over the query rows [r0, r0 + rows) (a whole number of row blocks).
struct Envelope {
  int ulo[kMaxNI], uhi[kMaxNI], ilo[kMaxNI], ihi[kMaxNI];
};

__device__ __forceinline__ void rows_envelope(const Prep& P, int rb_seq, int r0, int rows, int L,
                                              int ni, Envelope& E) {
  const int rb0 = r0 / kRB;
  const int nrb = min((rows + kRB - 1) / kRB, (L - r0 + kRB - 1) / kRB);
  const int4* env = P.env + (int64_t)(rb_seq + rb0) * ni;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    E.ulo[j] = L;
    E.uhi[j] = 0;
    E.ilo[j] = INT32_MIN;
    E.ihi[j] = INT32_MAX;
    if (j < ni) {
      for (int r = 0; r < nrb; ++r) {
        const int4 v = env[r * ni + j];
        E.ulo[j] = min(E.ulo[j], v.x);
        E.uhi[j] = max(E.uhi[j], v.y);
        E.ilo[j] = max(E.ilo[j], v.z);
        E.ihi[j] = min(E.ihi[j], v.w);
      }
    }
  }
}

// Key tiles [t_begin, t_end) that may hold visible columns.
__device__ __forceinline__ void envelope_tile_span(const Envelope& E, int ni, int bn, int& t_begin,
                                                   int& t_end) {
  t_begin = INT32_MAX;
  t_end = 0;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    if (j < ni && E.ulo[j] < E.uhi[j]) {
      t_begin = min(t_begin, E.ulo[j] / bn);
      t_end = max(t_end, (E.uhi[j] - 1) / bn + 1);
    }
  }
  if (t_end <= t_begin) t_begin = t_end = 0;
}

// Wave-level: lists the live tiles of [w0, min(w0 + 64, w1)) in two arrays,
// those some valid row sees only partly (part[0..*n_part)) and those every
// valid row sees whole (full[0..*n_full)), in increasing order.  Must be
// called by a whole wave; the counts are returned in every lane.
__device__ __forceinline__ void tile_window(const Envelope& E, int ni, int bn, int L, int w0,
                                            int w1, int* part, int* full_list, int& n_part,
                                            int& n_full) {
  const int lane = threadIdx.x & 63;
  const int t = w0 + lane;
  const int c0 = t * bn, c1 = min(c0 + bn, L);
  bool live = false, full = false;
  if (t < w1) {
#pragma unroll
    for (int j = 0; j < kMaxNI; ++j) {
      if (j < ni) {
        live = live || (E.ulo[j] < E.uhi[j] && E.ulo[j] < c1 && E.uhi[j] > c0);
        full = full || (E.ilo[j] <= c0 && c1 <= E.ihi[j]);
      }
    }
  }
  full = full && live;
  const bool partial = live && !full;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t mp = __ballot(partial), mf = __ballot(full);
  if (partial) part[__popcll(mp & below)] = t;
  if (full) full_list[__popcll(mf & below)] = t;
  n_part = __popcll(mp);
  n_full = __popcll(mf);
}

// Whether row block `rb` (its envelope row `env`) reaches key columns [c0, c1),
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

// Buffer resource over `rows` rows of `row_bytes` bytes starting at `base`,
// exposing only the first `width_bytes` of the last row: reads at
// row*row_bytes + col (col < width_bytes) return data for row < rows and zeros
// past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows,
                                                             int row_bytes, int width_bytes) {
  const int n = rows > 0 ? (rows - 1) * row_bytes + width_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Asynchronous 16-byte-per-lane copy from a buffer resource into LDS: lane l's
// 16 bytes land at lds + 16*l (lds must be the same in every lane), whatever
// global offset the lane reads; out-of-range lanes write zeros.  Completion is
// tracked by vmcnt (a workgroup barrier waits for it).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// Waits until every DMA this wave issued has landed in LDS, then joins the
// workgroup barrier: afterwards every wave sees every wave's copied tiles.
// The wait is explicit because the barrier's own lowering waits for LDS DMA
// only when the compiler cannot prove that the next LDS reads miss it, which
// says nothing about the reads of the other waves.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Workgroup barrier ordering LDS accesses only: it waits for this wave's own
// LDS operations but not for its vector-memory loads, so loads of later
// tiles stay in flight across it (a plain __syncthreads() may wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// lds_dma16 issued from inline assembly: the same copy, but invisible to the
// compiler's memory model, which then adds no waits of its own for it (it
// treats copies into LDS and loads into registers as completing out of order
// and would wait for every outstanding load before reading any LDS).  The
// caller orders it explicitly: s_waitcnt vmcnt plus a barrier before the
// copied data is read, and a barrier before its destination is overwritten.
// `lds` must be wave-uniform.  M0 is set here; no other code in these kernels
// keeps a value in M0.  A copy into LDS that reads M0 needs one wait state
// after the write to M0 (the compiler cannot see inside the assembly to add it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_raw(__amdgpu_buffer_rsrc_t r, const void* lds,
                                              int voffset) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0),
               "v"(voffset), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A voffset no buffer in this library reaches: its DMA lane writes zeros.
constexpr int kDmaSkip = 0x7ff00000;

// Per-lane global offset of DMA slot s for rows of `chunks` 16-byte slots of
// which the first 16 hold a 256-byte row (the rest is LDS padding).
__device__ __forceinline__ int dma_slot_offset(int s, int chunks, int row_bytes) {
  const int r = s / chunks, c = s - r * chunks;
  return c < 16 ? r * row_bytes + c * 16 : kDmaSkip;
}

// Swizzled LDS tiles: 256-byte rows (one D = 128 bf16 row) of 16 16-byte
// chunks, chunk c of row r stored at position c ^ swz(r).  Every 16
// consecutive rows read at one chunk (the 16 lanes a b128 row read serves per
// LDS cycle) and every 4 aligned consecutive rows read across an aligned quad
// of chunks (the 32 lanes of a pair of transpose-read groups) land on 16
// distinct positions, i.e. on all 64 banks once.  swz depends on r mod 16
// only, and swz(r + 8) = swz(r) ^ 2.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// bf16 element index of (row r, column col) in a swizzled tile.
__device__ __forceinline__ int swz_index(int r, int col) {
  return r * 128 + ((((col >> 3) ^ swz(r))) << 3) + (col & 7);
}

// 16-byte row read and 8-byte transpose read (lds_read_tr) at a byte offset
// into an LDS tile.
__device__ __forceinline__ bf16x8 lds_row16(const uint16_t* tile, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + byte_off);
}
__device__ __forceinline__ bf16x4 lds_tr8(const uint16_t* tile, int byte_off) {
  return lds_read_tr(reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const char*>(tile) + byte_off));
}

// The value of x, hidden from the optimiser: offsets derived from it inside a
// loop are recomputed there instead of being hoisted into live registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Global byte offset that DMA slot s (LDS bytes [16 s, 16 s + 16)) of a
// swizzled tile copies, for rows row_bytes apart.
__device__ __forceinline__ int swz_dma_offset(int s, int row_bytes) {
  const int r = s >> 4;
  return r * row_bytes + (((s & 15) ^ swz(r)) << 4);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voffset) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
  return __builtin_bit_cast(uint4, v);
}

}  // namespace hstu
