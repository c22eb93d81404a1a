// Host-side replay of the atomic-dQ key-owner pass's index arithmetic, through
// the functions the kernel itself calls (atomic_dq.h), for the sequence
// lengths given on the command line.  It checks that
//   * in each half's exchange buffer, the four waves' 16-byte writes of their
//     two P registers cover the buffer's bytes exactly once, and every 8-byte
//     transpose read lies inside the buffer;
//   * the accumulator's row map is a permutation: over the 32 (lane half g,
//     element i) pairs, xchg_acc_row(i, g) takes every value 0..31 once;
//   * the K gather (keys < L) and the atomics (rows < L) address only the
//     sequence's own rows of the [total, H, D] tensors, and over a key tile's
//     walk of every row block each (row, dim) of the sequence receives one
//     atomic per key tile: no element twice, none missed;
//   * the exchange buffers fit the kernel's LDS array (kXchgBytes).
// Usage: atomic_bounds H L0 L1 ...   Prints the first violation of each kind,
// then "elements=<n> ok" (or FAILED, exit status 1).  Built with
// PLANT_DROP_HALF_OFFSET, the replay forgets the second half's 32-row offset
// (a planted mistake the coverage check must catch).
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "atomic_dq.h"

using namespace hstu;

namespace {

long g_violations = 0;
std::vector<const char*> g_seen;
void bad(const char* what, long a, long b) {
  ++g_violations;
  if (std::find(g_seen.begin(), g_seen.end(), what) != g_seen.end()) return;
  g_seen.push_back(what);
  printf("violation: %s (%ld, %ld)\n", what, a, b);
}

void check_exchange() {
  std::vector<int> cover(kXchgHalfBytes, 0);
  for (int w = 0; w < 4; ++w)
    for (int lane = 0; lane < 64; ++lane)
      for (int hh = 0; hh < 2; ++hh) {
        const int off = xchg_write_offset(w, lane & 31, lane >> 5, hh);
        if (off < 0 || off + 16 > kXchgHalfBytes || (off & 15)) {
          bad("exchange write outside the half's buffer", w, lane);
          continue;
        }
        for (int b = 0; b < 16; ++b) ++cover[off + b];
      }
  for (int b = 0; b < kXchgHalfBytes; ++b)
    if (cover[b] != 1) bad("exchange byte not written exactly once", b, cover[b]);
  for (int lane = 0; lane < 64; ++lane)
    for (int ks = 0; ks < 8; ++ks)
      for (int s = 0; s < 2; ++s) {
        const int off = xchg_read_offset(lane, ks, s);
        if (off < 0 || off + 8 > kXchgHalfBytes || (off & 7)) bad("exchange read outside", lane, ks);
        // the kernel adds the per-ks part to the ks = 0 offset
        if (off != xchg_read_offset(lane, 0, s) + (ks >> 1) * kXchgWaveBytes + (ks & 1) * 1024)
          bad("exchange read offset not additive in ks", lane, ks);
      }
  if (2 * kXchgHalfBytes != kXchgBytes) bad("exchange buffers do not fit the LDS array", 0, 0);
}

void check_rows() {
  std::vector<int> seen(32, 0);
  for (int g = 0; g < 2; ++g)
    for (int i = 0; i < 16; ++i) {
      const int r = xchg_acc_row(i, g);
      if (r < 0 || r >= 32) bad("accumulator row out of the half", g, i);
      else ++seen[r];
    }
  for (int r = 0; r < 32; ++r)
    if (seen[r] != 1) bad("accumulator row map is not a permutation", r, seen[r]);
  for (int ks = 0; ks < 8; ++ks)
    for (int g = 0; g < 2; ++g)
      for (int e = 0; e < 8; ++e) {
        const int key = xchg_k_key(ks, g, e);
        if (key < 0 || key >= 128) bad("K operand key outside the tile", ks, g * 8 + e);
      }
}

long check_sequences(const std::vector<int64_t>& L, int H) {
  const int D = 128;
  int64_t total = 0;
  for (int64_t len : L) total += len;
  const int64_t rs = (int64_t)H * D, limit = total * rs;
  long elements = 0;
  int64_t s = 0;
  for (size_t b = 0; b < L.size(); s += L[b], ++b) {
    const int len = (int)L[b];
    const int nkt = (len + 127) / 128;
    for (int h = 0; h < H; ++h) {
      std::vector<int> hits((size_t)len * D, 0);
      for (int kt = 0; kt < nkt; ++kt) {
        const int c0 = kt * 128;
        for (int w = 0; w < 4; ++w)
          for (int lane = 0; lane < 64; ++lane) {
            const int n = lane & 31, g = lane >> 5;
            // the K gather: rows c0 + key < L only
            for (int ks = 0; ks < 8; ++ks)
              for (int e = 0; e < 8; ++e) {
                const int key = c0 + xchg_k_key(ks, g, e);
                if (key >= len) continue;
                const int64_t idx = (s + key) * rs + (int64_t)h * D + w * 32 + n;
                if (idx < s * rs || idx >= (s + len) * rs || idx >= limit)
                  bad("K gather outside the sequence", (long)b, key);
              }
            // the atomics of every half of every row block
            for (int q0 = 0; q0 < len; q0 += 64) {
              const int nh = q0 + 32 < len ? 2 : 1;
              for (int hf = 0; hf < nh; ++hf)
                for (int i = 0; i < 16; ++i) {
#ifdef PLANT_DROP_HALF_OFFSET
                  const int row = q0 + xchg_acc_row(i, g);  // planted: second half lands on the first
#else
                  const int row = q0 + 32 * hf + xchg_acc_row(i, g);
#endif
                  if (row >= len) continue;
                  const int64_t idx = (s + row) * rs + (int64_t)h * D + w * 32 + n;
                  if (idx < s * rs || idx >= (s + len) * rs || idx >= limit)
                    bad("atomic outside the sequence", (long)b, row);
                  else
                    ++hits[(size_t)row * D + w * 32 + n];
                }
            }
          }
      }
      for (size_t j = 0; j < hits.size(); ++j)
        if (hits[j] != nkt) bad("dQ element not added once per key tile", (long)b, (long)j);
      elements += (long)hits.size();
    }
  }
  return elements;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s H L0 [L1 ...]\n", argv[0]);
    return 2;
  }
  const int H = atoi(argv[1]);
  std::vector<int64_t> L;
  for (int i = 2; i < argc; ++i) L.push_back(atoll(argv[i]));
  check_exchange();
  check_rows();
  const long elements = check_sequences(L, H);
  printf("elements=%ld %s\n", elements, g_violations ? "FAILED" : "ok");
  return g_violations ? 1 : 0;
}
