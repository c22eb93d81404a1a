// Index arithmetic of the atomic-dQ key-owner pass (k_bwd_kv<false, true> in
// bwd.hip), shared by the kernel and the host-side replay of its accesses
// (tests/atomic_bounds.cpp).
//
// Per 32-row half, the workgroup's four waves publish their bf16 P registers
// (the B operand of the dK product: lane (n, g) holds key 32 wave + n at row
// positions hh*16 + g*8 + 0..7 in register hh) in an exchange buffer of 8 KiB,
// 2 KiB per wave: key rows of 64 bytes, the 16-byte chunk c = 2 hh + g of key
// row n at position c ^ ((n/4) mod 4).  Every wave then reads all 128 keys
// back with 8-byte transpose reads, so that lane l holds keys 16 ks + 8 (l/32)
// + 0..7 of row position l % 32: the A operand of dQ[row position][dim] += P K.
// Row position hh*16 + g'*8 + e is query row (2 hh + e/4)*8 + g'*4 + e%4 of
// the half (the order of the P registers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

constexpr int kXchgWaveBytes = 2048;                // one wave's P registers
constexpr int kXchgHalfBytes = 4 * kXchgWaveBytes;  // one half's exchange buffer
constexpr int kXchgBytes = 2 * kXchgHalfBytes;      // both halves

// Byte offset, in a half's exchange buffer, of the 16-byte write of P
// register hh by lane (n, g) of wave `wave`.
__host__ __device__ inline int xchg_write_offset(int wave, int n, int g, int hh) {
  return wave * kXchgWaveBytes + ((n * 64 + ((g ^ ((n >> 2) & 3)) << 4)) ^ (hh * 32));
}

// Byte offset, in a half's exchange buffer, of lane `lane`'s 8-byte transpose
// read `second` (0 or 1) for key step ks (keys 16 ks .. 16 ks + 15).
__host__ __device__ inline int xchg_read_offset(int lane, int ks, int second) {
  const int grp = lane >> 4, gl = lane & 15;
  const int pr = (8 * (grp >> 1) + (gl >> 2)) * 64 +
                 ((((grp & 1) * 2 + ((gl & 3) >> 1)) ^ (2 * (grp >> 1))) << 4) + (gl & 1) * 8;
  return (ks >> 1) * kXchgWaveBytes + (ks & 1) * 1024 + (second ? (pr ^ 16) + 256 : pr);
}

// Query row (0..31, within the half) of element i (0..15) of lane half g of
// the dQ[row position][dim] accumulator: row position (i/4)*8 + g*4 + i%4.
__host__ __device__ inline int xchg_acc_row(int i, int g) {
  const int m = (i >> 2) * 8 + g * 4 + (i & 3);
  return (2 * (m >> 4) + ((m & 7) >> 2)) * 8 + ((m >> 3) & 1) * 4 + (m & 3);
}

// Key (relative to the tile's first key) of element e of lane half g's K
// operand for key step ks: keys 16 ks + 8 g + 0..7.
__host__ __device__ inline int xchg_k_key(int ks, int g, int e) { return 16 * ks + 8 * g + e; }

}  // namespace hstu
