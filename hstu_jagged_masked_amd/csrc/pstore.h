// Layout of the stored-P buffer of the stored-P backward, shared by the host
// (buffer size), the preparation kernel (per-sequence block prefix), the
// key-owner pass that writes P and the dQ pass that reads it back.
//
// Per (sequence b, head h) the buffer holds a grid of 8 KiB blocks, one per
// (128-key tile kt, 32-row step t) of the sequence's L x L square:
//   kt < ceil(L/128), t < ceil(L/32),
//   block index = pblk[b] * H + h * nkt * nsteps + kt * nsteps + t,
// with pblk[b] the number of blocks (per head) of the sequences before b.
// A block holds, for the 32 query rows of step t and the 128 keys of tile kt,
// the four key-owner waves' bf16 P registers as they are (2 KiB per wave).
//
// Every access goes through a buffer resource that spans one key tile's
// blocks (all steps t of one (b, h, kt)), clipped to the caller's buffer:
// the hardware range check turns a read past it into zeros and drops a write
// past it, so no index computed here can reach outside the caller's buffer,
// whatever the offsets or the buffer size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

constexpr int kPKeys = 128;            // keys per stored-P tile
constexpr int kPRows = 32;             // query rows per stored-P step
constexpr int kPBlockBytes = 8192;     // kPKeys * kPRows * 2 bytes
constexpr int kCacheNT = 2;            // buffer load / store cache policy: non-temporal

__host__ __device__ inline int64_t pstore_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Blocks of one head of a sequence of length L.
__host__ __device__ inline int64_t pstore_seq_blocks(int64_t L) {
  return pstore_cdiv(L, kPKeys) * pstore_cdiv(L, kPRows);
}

// The blocks of key tile kt of (sequence with block prefix pblk_seq, head h,
// length L) as a byte range [base, base + bytes) of a buffer of cap bytes:
// `bytes` covers the tile's ceil(L/32) steps, clipped to the end of the
// buffer and to the 32-bit range of a buffer resource.
struct PRegion {
  uint64_t base;
  uint32_t bytes;
};

__host__ __device__ inline PRegion pstore_tile_region(int64_t pblk_seq, int H, int h, int L,
                                                      int kt, uint64_t cap) {
  const int64_t nkt = pstore_cdiv(L, kPKeys), nsteps = pstore_cdiv(L, kPRows);
  const uint64_t blk = (uint64_t)(pblk_seq * H + (int64_t)h * nkt * nsteps + (int64_t)kt * nsteps);
  const uint64_t base = blk * kPBlockBytes;
  uint64_t want = (uint64_t)nsteps * kPBlockBytes;
  const uint64_t avail = base < cap ? cap - base : 0;
  if (want > avail) want = avail;
  if (want > 0xffffffffull) want = 0xffffffffull;
  PRegion r;
  r.base = base < cap ? base : 0;
  r.bytes = (uint32_t)want;
  return r;
}

// Byte offset, inside a tile's region, of the 16 bytes that lane `lane` of
// wave `wave` stores or loads for step t, part `part` (the key-owner wave's
// two 1 KiB halves, or the dQ wave's 8 key steps of 1 KiB: part = 2*wave' +
// half or part = ks -- both address [t][part][lane]).  Steps t >= ceil(L/32)
// lie past the region: their loads read zeros.
__host__ __device__ inline uint32_t pstore_offset(int t, int part, int lane) {
  return (uint32_t)t * kPBlockBytes + (uint32_t)part * 1024u + (uint32_t)lane * 16u;
}

}  // namespace hstu
