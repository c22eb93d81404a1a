// Host-side replay of every stored-P access the two stored-P kernels can
// make, through the same layout functions they call (pstore.h), for a set of
// sequence lengths given on the command line.  It checks that
//   * every access of the key-owner pass (rows r < L of each key tile kt) and
//     of the dQ pass (the 4 waves' steps q0 = 128 qt + 32 w of every query
//     tile qt, whether or not q0 < L) either lies inside its tile's region or
//     past the region's end (then the hardware range check returns zeros /
//     drops the write), and every region lies inside the buffer;
//   * with a buffer of the size the library reports, every access to a real
//     block (t < ceil(L/32)) is served, and regions of different (sequence,
//     head, key tile) are disjoint;
//   * with a buffer one block short, no access leaves the buffer.
// Usage: pstore_bounds H L0 L1 ...   Prints the first violation of each kind,
// then "need=<bytes> past_end=<n> ok" (or FAILED, exit status 1).  With FLAT_ADDRESSING defined, it
// replays plain unchecked global accesses at the same addresses (the form
// these kernels had before their accesses were range-checked), which must be
// caught for lengths whose last query tile has idle waves.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "pstore.h"

using namespace hstu;

namespace {

struct Access {
  uint64_t lo, hi;  // absolute byte range in the buffer
  bool served;      // inside its range check (else it reads zeros / is dropped)
};

// The byte range the hardware serves for an access at `off` into `pr`.
Access resolve(const PRegion& pr, uint32_t off) {
#ifdef FLAT_ADDRESSING
  // plain global accesses from the tile's first block: nothing bounds them
  const uint64_t lo = pr.base + off;
  return Access{lo, lo + 16, true};
#else
  const bool in = (uint64_t)off + 16 <= pr.bytes;
  return Access{pr.base + off, pr.base + off + 16, in};
#endif
}

// Prints the first violation of each kind; counts them all.
long g_violations = 0;
std::vector<const char*> g_seen;
void bad(const char* what, int b, int h, int kt, int t) {
  ++g_violations;
  if (std::find(g_seen.begin(), g_seen.end(), what) != g_seen.end()) return;
  g_seen.push_back(what);
  printf("violation: %s (sequence %d, head %d, key tile %d, step %d)\n", what, b, h, kt, t);
}

void check(const std::vector<int64_t>& L, int H, uint64_t cap, bool full, long* past_end) {
  const int B = (int)L.size();
  std::vector<int64_t> pblk(B + 1, 0);
  for (int b = 0; b < B; ++b) pblk[b + 1] = pblk[b] + pstore_seq_blocks(L[b]);
  std::vector<std::pair<uint64_t, uint64_t>> regions;
  for (int b = 0; b < B; ++b) {
    const int len = (int)L[b];
    const int nkt = (int)pstore_cdiv(len, kPKeys), nsteps = (int)pstore_cdiv(len, kPRows);
    const int nqt = (int)pstore_cdiv(len, 128);
    for (int h = 0; h < H; ++h) {
      for (int kt = 0; kt < nkt; ++kt) {
        const PRegion pr = pstore_tile_region(pblk[b], H, h, len, kt, cap);
        if (pr.base + pr.bytes > cap) bad("region past the buffer", b, h, kt, -1);
        regions.push_back({pr.base, pr.base + pr.bytes});
        // key-owner pass: steps of rows r < L, parts 2 w + half, all lanes
        for (int t = 0; t < nsteps; ++t)
          for (int part = 0; part < 8; ++part)
            for (int lane = 0; lane < 64; lane += 63) {
              const Access a = resolve(pr, pstore_offset(t, part, lane));
              if (a.served && a.hi > cap) bad("store past the buffer", b, h, kt, t);
              if (full && !a.served) bad("store to a real block dropped", b, h, kt, t);
              if (full && a.served && (a.lo < pr.base || a.hi > pr.base + (uint64_t)nsteps *
                                                                              kPBlockBytes))
                bad("store outside its tile", b, h, kt, t);
            }
        // dQ pass: every wave of every query tile loads, rows or not
        for (int qt = 0; qt < nqt; ++qt)
          for (int w = 0; w < 4; ++w) {
            const int t = (qt * 128 + 32 * w) / kPRows;
            for (int ks = 0; ks < 8; ++ks)
              for (int lane = 0; lane < 64; lane += 63) {
                const Access a = resolve(pr, pstore_offset(t, ks, lane));
                if (a.served && a.hi > cap) bad("load past the buffer", b, h, kt, t);
                if (t >= nsteps) {
                  ++*past_end;
                  if (a.served && full && a.hi <= cap &&
                      a.hi > pr.base + (uint64_t)nsteps * kPBlockBytes)
                    bad("idle wave reads another tile's blocks", b, h, kt, t);
                } else if (full && !a.served) {
                  bad("load of a real block returns zeros", b, h, kt, t);
                }
              }
          }
      }
    }
  }
  if (full) {
    std::sort(regions.begin(), regions.end());
    for (size_t i = 1; i < regions.size(); ++i)
      if (regions[i].first < regions[i - 1].second && regions[i].first < regions[i].second)
        bad("overlapping regions", -1, -1, -1, -1);
  }
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
  uint64_t need = 0;
  for (int64_t len : L) need += (uint64_t)pstore_seq_blocks(len) * H * kPBlockBytes;
  long past_end = 0;
  check(L, H, need, true, &past_end);
  if (need >= (uint64_t)kPBlockBytes) check(L, H, need - kPBlockBytes, false, &past_end);
  printf("need=%llu past_end=%ld %s\n", (unsigned long long)need, past_end,
         g_violations ? "FAILED" : "ok");
  return g_violations ? 1 : 0;
}
