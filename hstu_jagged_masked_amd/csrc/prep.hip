// Preparation kernels: sanitized offsets, the jagged tile scheduler (longest
// sequences first, dealt over the XCDs), per-row-block interval envelopes,
// and exact per-row visible-column counts.
//
// The interval semantics follow TorchEasyRec PR #670 ("What changed"):
// interval 0 = [0, f0), interval j = [f(2j-1), f(2j)), empty when end <= start,
// visible set = union, bounds sequence-local and clipped to [0, L).
#include <algorithm>

#include "common.h"
#include "pstore.h"

namespace hstu {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / 64;

struct SumOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct MaxOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a > b ? a : b; }
};

// Inclusive scan of one value per thread across the 1024-thread block.
// `scratch` holds kPrepWaves entries.  Returns the inclusive prefix; *total
// receives the block-wide reduction.
template <typename T, typename Op>
__device__ T block_inclusive_scan(T x, T* scratch, T* total, Op op) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int s = 1; s < 64; s <<= 1) {
    T y = __shfl_up(x, s, 64);
    if (lane >= s) x = op(x, y);
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kPrepWaves; ++w) scratch[w] = op(scratch[w - 1], scratch[w]);
  }
  __syncthreads();
  if (wave > 0) x = op(scratch[wave - 1], x);
  *total = scratch[kPrepWaves - 1];
  __syncthreads();
  return x;
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Position of sorted rank p after snake-dealing B ranks over 8 bins and
// concatenating the bins (bin 0 first).  Within a bin, ranks keep their order.
__device__ int dealt_position(int p, int B) {
  const int R = B / kNumXcd, rem = B % kNumXcd;
  int round = p / kNumXcd, pos = p % kNumXcd;
  int bin = (round & 1) ? (kNumXcd - 1 - pos) : pos;
  int start = 0;
  for (int x = 0; x < bin; ++x) {
    int n = R;
    if (rem) {
      bool extra = (R & 1) ? (x >= kNumXcd - rem) : (x < rem);
      n += extra ? 1 : 0;
    }
    start += n;
  }
  return start + round;
}

__global__ __launch_bounds__(kPrepThreads) void k_prep(Prep P, const int64_t* __restrict__ off,
                                                       const int32_t* __restrict__ target_rows) {
  __shared__ int hist[kHistBins];
  __shared__ int64_t scan64[kPrepWaves];
  __shared__ int scan32[kPrepWaves];
  __shared__ int sflags;
  const int tid = threadIdx.x;
  const int B = P.B;
  if (tid == 0) sflags = 0;
  for (int i = tid; i < kHistBins; i += kPrepThreads) hist[i] = 0;
  __syncthreads();

  // 1. sanitized offsets: clamp into [lo, hi] (0 and total for a whole
  // batch) and take a running maximum.
  const int64_t lo = P.row_lo, hi = P.row_hi;
  int flags = 0;
  int64_t run = lo;
  for (int base = 0; base <= B; base += kPrepThreads) {
    const int b = base + tid;
    int64_t x = lo;
    if (b <= B) {
      int64_t raw = off[b];
      if (b == 0 && raw != lo) flags |= kFlagOffsetsStart;
      if (b == B && raw != hi) flags |= kFlagOffsetsEnd;
      if (raw < lo || raw > hi) flags |= kFlagOffsetsOrder;
      if (b > 0 && raw < off[b - 1]) flags |= kFlagOffsetsOrder;
      x = raw < lo ? lo : (raw > hi ? hi : raw);
    }
    int64_t chunk_max;
    int64_t m = block_inclusive_scan(x, scan64, &chunk_max, MaxOp());
    m = m > run ? m : run;
    if (b == 0) m = lo;
    if (b == B) m = hi;
    if (b <= B) P.so[b] = m;
    run = chunk_max > run ? chunk_max : run;
  }
  __syncthreads();

  // 2. lengths -> histogram keyed by decreasing length; target-row checks.
  for (int b = tid; b < B; b += kPrepThreads) {
    const int L = (int)(P.so[b + 1] - P.so[b]);
    if (target_rows) {
      const int t = target_rows[b];
      if (L > 0 && (t < 0 || t >= L)) flags |= kFlagTargetRange;
    }
    const int bucket = min(L >> 4, kHistBins - 1);
    atomicAdd(&hist[kHistBins - 1 - bucket], 1);
  }
  __syncthreads();

  // 3. exclusive scan of the histogram (4 bins per thread).
  {
    int v[4], s = 0;
    for (int i = 0; i < 4; ++i) { v[i] = hist[tid * 4 + i]; s += v[i]; }
    int tot;
    int incl = block_inclusive_scan(s, scan32, &tot, SumOp());
    int run_bin = incl - s;
    for (int i = 0; i < 4; ++i) { hist[tid * 4 + i] = run_bin; run_bin += v[i]; }
  }
  __syncthreads();

  // 4. scatter: sorted rank from the bucket cursor, then dealt position.
  for (int b = tid; b < B; b += kPrepThreads) {
    const int L = (int)(P.so[b + 1] - P.so[b]);
    const int bucket = min(L >> 4, kHistBins - 1);
    const int rank = atomicAdd(&hist[kHistBins - 1 - bucket], 1);
    P.order[dealt_position(rank, B)] = b;
  }
  __syncthreads();

  // 5. row-block offsets (original order) and tile prefixes (dealt order).
  int carry_rb = 0, carry64 = 0, carry128 = 0;
  int64_t carry_blk = 0;
  for (int base = 0; base < B; base += kPrepThreads) {
    const int b = base + tid;
    int nrb = 0, n64 = 0, n128 = 0;
    if (b < B) {
      const int L = (int)(P.so[b + 1] - P.so[b]);
      nrb = cdiv(L, kRB);
      const int sb = P.order[b];
      const int Ls = (int)(P.so[sb + 1] - P.so[sb]);
      n64 = cdiv(Ls, 64);
      n128 = cdiv(Ls, 128);
    }
    int t_rb, t64, t128;
    int i_rb = block_inclusive_scan(nrb, scan32, &t_rb, SumOp());
    int i64 = block_inclusive_scan(n64, scan32, &t64, SumOp());
    int i128 = block_inclusive_scan(n128, scan32, &t128, SumOp());
    if (b < B) {
      P.rb_off[b] = carry_rb + i_rb - nrb;
      P.tiles64[b] = carry64 + i64 - n64;
      P.tiles128[b] = carry128 + i128 - n128;
    }
    carry_rb += t_rb;
    carry64 += t64;
    carry128 += t128;
    if (P.pblk) {
      // stored-P blocks of one head: (128-key tiles) x (32-row halves)
      int64_t nblk = 0;
      if (b < B) {
        const int L = (int)(P.so[b + 1] - P.so[b]);
        nblk = pstore_seq_blocks(L);
      }
      int64_t t_blk;
      const int64_t i_blk = block_inclusive_scan(nblk, scan64, &t_blk, SumOp());
      if (b < B) P.pblk[b] = carry_blk + i_blk - nblk;
      carry_blk += t_blk;
    }
  }
  if (tid == 0) {
    P.rb_off[B] = carry_rb;
    P.tiles64[B] = carry64;
    P.tiles128[B] = carry128;
    if (P.pblk) P.pblk[B] = carry_blk;
  }
  if (flags) atomicOr(&sflags, flags);
  __syncthreads();
  if (tid == 0) {
    P.flags[0] = sflags;
    P.flags[3] = carry_rb;
  }
}

constexpr int kUnitThreads = 1024;
// Lists of at most this many units run in a few rounds of the GPU's
// workgroup slots: their critical path is the heaviest unit, so they are
// ordered heaviest first instead of sequence by sequence.
constexpr int kSmallUnits = 4096;
constexpr int kUnitsPerThread = kSmallUnits / kUnitThreads;

// Unit lam of the sequence-major order: sequence p of the dealt order owns
// [H*T[p], H*T[p+1]); within it head-major, position tr in the sequence's
// tile order (decreasing tile index when `descending`, else increasing).
struct UnitPos {
  int p, nt, h, tr;
};

__device__ __forceinline__ UnitPos unit_pos(const int* T, int B, int H, int lam) {
  UnitPos u;
  u.p = upper_index(T, B, lam / H);
  u.nt = T[u.p + 1] - T[u.p];
  const int r = lam - H * T[u.p];
  u.h = r / u.nt;
  u.tr = r - u.h * u.nt;
  return u;
}

// The two int4 of a unit's record.
struct UnitRecord {
  int4 a, c;
};

__device__ __forceinline__ UnitRecord unit_record(const Prep& P, const UnitPos& u,
                                                  int descending) {
  const int b = P.order[u.p];
  const int64_t s = P.so[b];
  const int64_t pb = P.pblk ? P.pblk[b] : 0;
  UnitRecord r;
  r.a = make_int4(b, descending ? u.nt - 1 - u.tr : u.tr, u.h, (int)(P.so[b + 1] - s));
  r.c = make_int4((int)s, P.rb_off[b], (int)(uint32_t)(uint64_t)pb,
                  (int)(uint32_t)((uint64_t)pb >> 32));
  return r;
}

__device__ __forceinline__ void put_record(int4* list, int64_t at, int4 a, int4 c) {
  list[2 * at] = a;
  list[2 * at + 1] = c;
}

// Unit list for tiles of `tile` rows, one record per workgroup.
// Long lists (more than kSmallUnits units): unit lam of the sequence-major
// order runs on the workgroup that xcd_slot maps to lam, so each XCD takes a
// contiguous share of the list and a sequence's tiles, which re-read the same
// rows, share an L2; sequences come longest first and, within one, tiles
// heaviest first for prefix-like masks.
// Short lists: workgroup 0 sorts the units by a work estimate, heaviest
// first -- for query tiles (`descending`) the higher tile index, for key tiles
// the more tiles from it to the end of its sequence, which is what a causal
// or prefix mask makes them cost -- and unit i runs on workgroup i, so the
// heavy units start in the first round, spread over the XCDs.  (Units of
// equal estimate take positions in an order the atomics decide; every unit
// computes the same outputs wherever it runs.)
struct UnitShared {
  int hist[kSmallUnits];
  int part[kUnitThreads / 64];
  int smax;
};

// Block `blk` of the list's grid (kUnitThreads threads).
__device__ void units_block(const Prep& P, const UnitJob& J, int H, int blk, UnitShared& sh) {
  const Units& U = J.U;
  const int tile = J.tile, descending = J.descending, count_slot = J.count_slot;
  int* const hist = sh.hist;
  int* const part = sh.part;
  int& smax = sh.smax;
  const int tid = threadIdx.x;
  const int bid = blk * kUnitThreads + tid;
  const int* T = tile == 64 ? P.tiles64 : P.tiles128;
  const int B = P.B;
  const int n = H * T[B];
  if (bid == 0) P.flags[count_slot] = n;
  const int4 idle_a = make_int4(-1, 0, 0, 0), idle_c = make_int4(0, 0, 0, 0);
  if (n > kSmallUnits) {
    if (bid >= U.cap) return;
    const int lam = xcd_slot(bid, n);
    if (lam < 0) {
      put_record(U.list, bid, idle_a, idle_c);
      return;
    }
    const UnitRecord r = unit_record(P, unit_pos(T, B, H, lam), descending);
    put_record(U.list, bid, r.a, r.c);
    return;
  }
  if (bid >= n && bid < U.cap) put_record(U.list, bid, idle_a, idle_c);
  if (blk != 0) return;
  for (int i = tid; i < kSmallUnits; i += kUnitThreads) hist[i] = 0;
  if (tid == 0) smax = 0;
  // each thread's units, decoded once (their loads overlap)
  UnitPos up[kUnitsPerThread];
  UnitRecord rec[kUnitsPerThread];
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const int lam = tid + i * kUnitThreads;
    if (lam < n) {
      up[i] = unit_pos(T, B, H, lam);
      rec[i] = unit_record(P, up[i], descending);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i)
    if (tid + i * kUnitThreads < n) atomicMax(&smax, up[i].nt);
  __syncthreads();
  const int maxnt = smax;
  // estimate rank: 0 = heaviest; < maxnt <= n <= kSmallUnits
  int key[kUnitsPerThread];
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    const int t = descending ? up[i].nt - 1 - up[i].tr : up[i].tr;
    key[i] = descending ? maxnt - 1 - t : maxnt - up[i].nt + t;
    if (tid + i * kUnitThreads < n) atomicAdd(&hist[key[i]], 1);
  }
  __syncthreads();
  // exclusive scan of the histogram: thread tid owns bins [4 tid, 4 tid + 4)
  constexpr int kRun = kSmallUnits / kUnitThreads;
  int v[kRun], sum = 0;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    v[i] = hist[tid * kRun + i];
    sum += v[i];
  }
  const int lane = tid & 63, w = tid >> 6;
  int incl = sum;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  int base = 0;
  for (int j = 0; j < w; ++j) base += part[j];
  int run = base + incl - sum;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    hist[tid * kRun + i] = run;
    run += v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kUnitsPerThread; ++i) {
    if (tid + i * kUnitThreads < n) {
      const int pos = atomicAdd(&hist[key[i]], 1);
      // pos < n <= U.cap by the host's sizing of the list; the check keeps
      // the write inside the list whatever the lengths
      if (pos < U.cap) put_record(U.list, pos, rec[i].a, rec[i].c);
    }
  }
}

// One wave per row block g: envelopes of every interval.
__device__ void envelopes_wave(const Prep& P, const int32_t* __restrict__ func, int nfunc,
                               int g) {
  const int nrb = P.rb_off[P.B];
  if (g >= nrb) return;
  const int b = upper_index(P.rb_off, P.B, g);
  const int rb = g - P.rb_off[b];
  const int64_t s = P.so[b];
  const int L = (int)(P.so[b + 1] - s);
  const int lane = threadIdx.x & 63;
  const int i = rb * kRB + lane;
  const bool valid = i < L;
  const int ni = (nfunc + 1) / 2;
  for (int j = 0; j < ni; ++j) {
    int lo = L, hi = 0;
    if (valid) row_interval(func, P.total, s + i, j, L, lo, hi);
    int ulo = lo, uhi = hi;
    int ilo = valid ? lo : INT32_MIN, ihi = valid ? hi : INT32_MAX;
    for (int m = 1; m < 64; m <<= 1) {
      ulo = min(ulo, __shfl_xor(ulo, m, 64));
      uhi = max(uhi, __shfl_xor(uhi, m, 64));
      ilo = max(ilo, __shfl_xor(ilo, m, 64));
      ihi = min(ihi, __shfl_xor(ihi, m, 64));
    }
    if (lane == 0) P.env[(int64_t)g * ni + j] = make_int4(ulo, uhi, ilo, ihi);
  }
}

// What the kernels of one call need after k_prep, in one launch: blocks
// [0, env_blocks) compute the envelopes (one wave per row block), then each
// unit list takes its own run of blocks.  The parts are independent of each
// other; all read only what k_prep wrote.
constexpr int kEnvPerBlock = kUnitThreads / 64;

__global__ __launch_bounds__(kUnitThreads) void k_lists(Prep P, const int32_t* __restrict__ func,
                                                        int nfunc, int env_blocks, UnitJob J0,
                                                        int blocks0, UnitJob J1, int H) {
  __shared__ UnitShared sh;
  int b = blockIdx.x;
  if (b < env_blocks) {
    envelopes_wave(P, func, nfunc, b * kEnvPerBlock + (threadIdx.x >> 6));
    return;
  }
  b -= env_blocks;
  if (b < blocks0) {
    units_block(P, J0, H, b, sh);
    return;
  }
  units_block(P, J1, H, b - blocks0, sh);
}

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

// |V_i| per row (or per candidate): union of up to kMaxNI clipped intervals.
__global__ void k_visible_counts(const int64_t* __restrict__ off, int B, int64_t total,
                                 const int32_t* __restrict__ func, int nfunc,
                                 const int32_t* __restrict__ target_rows, int32_t* counts,
                                 unsigned long long* total_pairs) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int n = 0;
  bool active;
  if (target_rows) {
    active = t < B;
  } else {
    active = t < total;
  }
  if (active) {
    int b;
    int64_t row;
    if (target_rows) {
      b = (int)t;
    } else {
      b = upper_index(off, B, t);
      if (b >= B) b = B - 1;
    }
    int64_t start = off[b];
    start = start < 0 ? 0 : (start > total ? total : start);
    int64_t end = off[b + 1];
    end = end < start ? start : (end > total ? total : end);
    const int L = (int)(end - start);
    if (target_rows) {
      row = target_rows[b];
    } else {
      row = t - start;
    }
    if (row >= 0 && row < L) {
      int lo[kMaxNI], hi[kMaxNI];
      const int m = merged_intervals(func, total, start + row, nfunc, L, lo, hi);
      for (int k = 0; k < m; ++k) n += hi[k] - lo[k];
    }
    if (counts) counts[t] = n;
  }
  if (total_pairs) {
    unsigned long long s = (unsigned long long)n;
    for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
    if ((threadIdx.x & 63) == 0 && s) atomicAdd(total_pairs, s);
  }
}

}  // namespace

hipError_t launch_prep(const Prep& P, const int64_t* seq_offsets, const int32_t* target_rows,
                       hipStream_t stream) {
  ProfScope ps(stream, "k_prep");
  hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, stream, P, seq_offsets,
                     target_rows);
  return hipGetLastError();
}

hipError_t launch_lists(const Prep& P, const int32_t* func, int nfunc, const UnitJob* jobs,
                        int njobs, int H, hipStream_t stream) {
  const int env_blocks = func && P.nrb_cap > 0 ? (P.nrb_cap + kEnvPerBlock - 1) / kEnvPerBlock : 0;
  UnitJob J[2] = {};
  int blocks[2] = {0, 0};
  for (int i = 0; i < njobs && i < 2; ++i) {
    J[i] = jobs[i];
    blocks[i] = std::max(1, (J[i].U.cap + kUnitThreads - 1) / kUnitThreads);
  }
  const int grid = env_blocks + blocks[0] + blocks[1];
  if (grid == 0) return hipSuccess;
  ProfScope ps(stream, "k_lists");
  hipLaunchKernelGGL(k_lists, dim3(grid), dim3(kUnitThreads), 0, stream, P, func, nfunc,
                     env_blocks, J[0], blocks[0], J[1], H);
  return hipGetLastError();
}

hipError_t launch_visible_counts(const int64_t* seq_offsets, int B, int64_t total,
                                 const int32_t* func, int nfunc, const int32_t* target_rows,
                                 int32_t* counts, int64_t* total_pairs, hipStream_t stream) {
  if (total_pairs) {
    hipLaunchKernelGGL(k_zero_i64, dim3(1), dim3(1), 0, stream, total_pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = target_rows ? (int64_t)B : total;
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  ProfScope ps(stream, "k_visible_counts");
  hipLaunchKernelGGL(k_visible_counts, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     seq_offsets, B, total, func, nfunc, target_rows, counts,
                     reinterpret_cast<unsigned long long*>(total_pairs));
  return hipGetLastError();
}

}  // namespace hstu
