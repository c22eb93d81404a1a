// Internal declarations shared by the HIP sources of libhstu_attn.so (gfx950).
//
// Terms used throughout:
//   so[B+1]    sanitized sequence offsets (int64): so[0] = 0, nondecreasing,
//              so[B] = total; equal to seq_offsets for well-formed input.
//   row block  RB = 64 consecutive query rows of one sequence; the interval
//              decoder summarizes the func bounds of each row block.
//   envelope   per row block and interval j: union bounds [ulo, uhi) (smallest
//              start / largest end over rows whose clipped interval j is not
//              empty) and intersection bounds [ilo, ihi) (largest start /
//              smallest end over all valid rows; empty unless every row has a
//              non-empty interval j).  A key tile that meets no union envelope is
//              skipped; one inside an intersection envelope needs no mask.
//   unit       one workgroup's work item {b, tile, h}; unit lists are built on
//              the device, sequences ordered longest first and dealt across the
//              8 XCDs so each XCD gets a balanced share and keeps a sequence's
//              tiles (which re-read the same K/V) in its own L2.  The list is
//              indexed by workgroup and each record also carries the
//              sequence's start, length, first row block and stored-P base, so
//              a workgroup's first load is its whole unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

constexpr int kRB = 64;          // rows per row block (decoder granularity)
constexpr int kMaxNfunc = 9;     // largest nfunc accepted
constexpr int kMaxNI = (kMaxNfunc + 1) / 2;  // largest number of intervals
constexpr int kHistBins = 4096;  // length buckets of the scheduler's counting sort
constexpr int kNumXcd = 8;       // MI355X: 8 XCDs, workgroups dealt round-robin

// error flags written by the preparation kernel (bit set = problem seen)
enum : int {
  kFlagOffsetsStart = 1,   // seq_offsets[0] != 0
  kFlagOffsetsEnd = 2,     // seq_offsets[B] != total
  kFlagOffsetsOrder = 4,   // decreasing or out of [0, total]
  kFlagTargetRange = 8,    // a target row outside [0, L_b)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Slots of Prep::flags holding unit counts written by the unit-list kernel.
constexpr int kSlotFwdUnits = 4, kSlotKvUnits = 5, kSlotQUnits = 6;

// Device pointers into the caller's workspace (laid out by plan_workspace).
struct Prep {
  int* flags;          // [16]: [0] error bits, [1] units of tile 64, [2] units of tile 128
  int64_t* so;         // [B+1] sanitized offsets
  int* order;          // [B] sequences: longest first, dealt over the XCDs
  int* rb_off;         // [B+1] first row block of each sequence (original order)
  int* tiles64;        // [B+1] prefix over `order` of ceil(L/64)
  int* tiles128;       // [B+1] prefix over `order` of ceil(L/128)
  int4* env;           // [nrb_cap * ni] envelopes {ulo, uhi, ilo, ihi}
  int64_t* pblk;       // [B+1] prefix of ceil(L/128)*ceil(L/32) (stored-P blocks per
                       // head of each sequence, original order); null when not planned
  int B;
  int64_t total;       // rows of q, k, v and func (the func row stride)
  int64_t row_lo;      // the offsets are clamped into [row_lo, row_hi], the first
  int64_t row_hi;      // set to row_lo and the last to row_hi (0 and total for a
                       // whole batch, a run's rows for a run of its sequences)
  int nrb_cap;         // capacity of row blocks: ceil((row_hi - row_lo)/64) + B
};

struct Units {
  int4* list;  // 2 int4 per workgroup: {b, tile, h, L}, {s, rb_off[b], pblk[b] lo, hi};
               // b < 0 marks an idle workgroup
  int cap;     // workgroups (multiple of 8)
};

// One workgroup's unit, decoded from its record (all fields wave-uniform).
struct UnitRec {
  int b, tile, h, L;
  int64_t s;     // first row of the sequence
  int rb;        // first row block of the sequence
  int64_t pblk;  // stored-P blocks before the sequence (per head), 0 if not planned
};

// ---------------------------------------------------------------------------
// host-side planning
// ---------------------------------------------------------------------------
struct Plan {
  size_t bytes = 0;
  size_t off_flags, off_so, off_order, off_rb, off_t64, off_t128, off_env;
  size_t off_units_a, off_units_b, off_units_c;  // unit lists (kernel specific)
  size_t off_partial;                             // targets-only partial sums
  size_t off_pblk = 0;                            // stored-P block prefix (backward)
  int cap_a = 0, cap_b = 0, cap_c = 0;
  int nrb_cap = 0;
  int ni = 0;
  size_t partial_bytes = 0;
};

// Fills `plan` for a call; returns false if sizes are out of range.
bool plan_workspace(Plan& plan, int is_bwd, int64_t B, int64_t total, int H, int D, int nfunc,
                    int targets_only);
Prep prep_view(const Plan& plan, void* ws, int B, int64_t total);

// ---------------------------------------------------------------------------
// per-kernel timing: while profiling is on (hstu_profile_enable), a ProfScope
// records a HIP event before and after the kernel it wraps, on its stream.
// ---------------------------------------------------------------------------
class ProfScope {
 public:
  ProfScope(hipStream_t stream, const char* name);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  hipStream_t stream_;
  const char* name_;
  hipEvent_t start_ = nullptr;
};

// ---------------------------------------------------------------------------
// launchers (each returns a hipError_t from the launch)
// ---------------------------------------------------------------------------
hipError_t launch_prep(const Prep& P, const int64_t* seq_offsets, const int32_t* target_rows,
                       hipStream_t stream);
// One unit list to build: `U` for tiles of `tile` rows (descending: query
// tiles, heaviest = highest index), its unit count stored in P.flags[count_slot].
struct UnitJob {
  Units U;
  int tile, descending, count_slot;
};
// After launch_prep: the envelopes (when func is given; the MFMA kernels read
// them) and up to two unit lists, in one launch.
hipError_t launch_lists(const Prep& P, const int32_t* func, int nfunc, const UnitJob* jobs,
                        int njobs, int H, hipStream_t stream);
hipError_t launch_visible_counts(const int64_t* seq_offsets, int B, int64_t total,
                                 const int32_t* func, int nfunc, const int32_t* target_rows,
                                 int32_t* counts, int64_t* total_pairs, hipStream_t stream);

// generic fp32-FMA kernels (any supported dtype and D)
hipError_t launch_generic_fwd(int dtype, int D, const void* q, const void* k, const void* v,
                              void* o, const Prep& P, int H, const int32_t* func, int nfunc,
                              float alpha, float inv_max_len, const int32_t* target_rows,
                              hipStream_t stream);
hipError_t launch_generic_bwd(int dtype, int D, const void* q, const void* k, const void* v,
                              const void* dout, void* dq, void* dk, void* dv, const Prep& P,
                              int H, const int32_t* func, int nfunc, float alpha,
                              float inv_max_len, const int32_t* target_rows, hipStream_t stream);

// bf16, D = 128 MFMA kernels (full-length mode)
hipError_t launch_mfma_fwd(const void* q, const void* k, const void* v, void* o, const Prep& P,
                           const Units& U, int H, const int32_t* func, int nfunc, float alpha,
                           float inv_max_len, hipStream_t stream);
// pstore == nullptr: dQ by the query-owner kernel (recomputes S and dS);
// otherwise the key-owner kernel also stores P (bf16) there and dQ = P K is
// formed from it by k_bwd_dq.
hipError_t launch_mfma_bwd(const void* q, const void* k, const void* v, const void* dout,
                           void* dq, void* dk, void* dv, const Prep& P, const Units& Ukv,
                           const Units& Uq, int H, const int32_t* func, int nfunc, float alpha,
                           float inv_max_len, uint16_t* pstore, uint64_t pstore_cap,
                           hipStream_t stream);
hipError_t launch_mfma_bwd_atomic(const void* q, const void* k, const void* v, const void* dout,
                                  void* dq, void* dk, void* dv, const Prep& P, const Units& Ukv,
                                  int H, const int32_t* func, int nfunc, float alpha,
                                  float inv_max_len, float* dq_acc, int64_t total,
                                  hipStream_t stream);
hipError_t launch_dq_from_p(const void* k, void* dq, const Prep& P, const Units& Uq, int H,
                            int nfunc, const uint16_t* pstore, uint64_t pstore_cap,
                            float out_scale, hipStream_t stream);

// targets-only streaming kernels (any dtype, D); U lists 128-row key tiles
int targets_chunk_rows();
hipError_t launch_targets_fwd(int dtype, int D, const void* q, const void* k, const void* v,
                              void* o, const Prep& P, const Units& U, int H, const int32_t* func,
                              int nfunc, float alpha, float inv_max_len,
                              const int32_t* target_rows, float* partial, hipStream_t stream);
hipError_t launch_targets_bwd(int dtype, int D, const void* q, const void* k, const void* v,
                              const void* dout, void* dq, void* dk, void* dv, const Prep& P,
                              const Units& U, int H, const int32_t* func, int nfunc, float alpha,
                              float inv_max_len, const int32_t* target_rows, float* partial,
                              hipStream_t stream);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Workgroup index -> position in a unit list whose XCD shares are contiguous.
// Workgroup i runs on XCD i % 8; with n valid units, XCD x takes positions
// [x*per, (x+1)*per), per = ceil(n / 8).  Returns -1 for idle workgroups.
__device__ __forceinline__ int xcd_slot(int bid, int n) {
  int per = (n + kNumXcd - 1) / kNumXcd;
  int k = bid / kNumXcd;
  int slot = (bid % kNumXcd) * per + k;
  return (k < per && slot < n) ? slot : -1;
}

// Values every lane of the wave holds in common, moved to scalar registers.

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The unit of workgroup blockIdx.x; false for an idle workgroup.
__device__ __forceinline__ bool unit_of_block(const int4* __restrict__ list, UnitRec& u) {
  const int4 a = list[2 * (int64_t)blockIdx.x];
  const int4 c = list[2 * (int64_t)blockIdx.x + 1];
  u.b = uniform(a.x);
  u.tile = uniform(a.y);
  u.h = uniform(a.z);
  u.L = uniform(a.w);
  u.s = (int64_t)uniform(c.x);
  u.rb = uniform(c.y);
  u.pblk = (int64_t)(((uint64_t)(uint32_t)uniform(c.w) << 32) | (uint32_t)uniform(c.z));
  return u.b >= 0;
}

// Largest index i in [0, n] with a[i] <= x (a nondecreasing, a[0] <= x).
template <typename T>
__device__ __forceinline__ int upper_index(const T* a, int n, T x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer in [lo, hi]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Clipped interval j of the row whose func column is `col`: [lo, hi) within
// [0, L); an empty interval is returned as lo = L, hi = 0 (so that min/max
// reductions of starts and ends ignore it).
__device__ __forceinline__ void row_interval(const int32_t* func, int64_t total, int64_t col,
                                             int j, int L, int& lo, int& hi) {
  int a, b;
  if (j == 0) {
    a = 0;
    b = func[col];
  } else {
    a = func[(int64_t)(2 * j - 1) * total + col];
    b = func[(int64_t)(2 * j) * total + col];
  }
  a = max(a, 0);
  b = min(b, L);
  if (b <= a) { a = L; b = 0; }
  lo = a;
  hi = b;
}

// Visible columns of one row as sorted, disjoint intervals (union of the
// clipped func intervals).  Returns the number of intervals written.
__device__ __forceinline__ int merged_intervals(const int32_t* func, int64_t total, int64_t col,
                                                int nfunc, int L, int* lo, int* hi) {
  const int ni = (nfunc + 1) / 2;
  int m = 0;
  for (int j = 0; j < ni; ++j) {
    int a, c;
    row_interval(func, total, col, j, L, a, c);
    if (c > a) {
      int k = m++;
      while (k > 0 && lo[k - 1] > a) {
        lo[k] = lo[k - 1];
        hi[k] = hi[k - 1];
        --k;
      }
      lo[k] = a;
      hi[k] = c;
    }
  }
  int w = 0;
  for (int k = 0; k < m; ++k) {
    if (w > 0 && lo[k] <= hi[w - 1]) {
      hi[w - 1] = max(hi[w - 1], hi[k]);
    } else {
      lo[w] = lo[k];
      hi[w] = hi[k];
      ++w;
    }
  }
  return w;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive 16-bit values M[j][0..3]; lane i
// receives M[i/4 + 4t][i%4] for t = 0..3.  If the 16 lanes address a 4 x 16
// block of a row-major matrix A -- lane j at &A[r0 + j/4][c0 + 4*(j%4)] -- lane i
// receives A[r0 + t][c0 + i], t = 0..3: four consecutive rows of one column,
// which is the K-contiguous operand layout the MFMA wants.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}

// SiLU pieces on the fast transcendental units: logistic(a*x) with
// c = -a*log2(e) precomputed.  v_exp_f32 / v_rcp_f32 are accurate to ~1 ulp;
// overflow of the exponent gives rcp(inf) = 0, the correct limit.
__device__ __forceinline__ float logistic_scaled(float x, float c) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(c * x));
}

// x where bit b of m is set, +0 where it is clear.  The signed one-bit field
// extract is all ones or all zeros, and it is and-ed with the float's bits: two
// instructions per element, with no compare, select or separate conversion.
// bit_keep takes a per-lane b; bit_keep_imm a b that is a constant after
// unrolling (inline assembly: the compiler turns a field extract at a known
// offset back into a compare and a select).
__device__ __forceinline__ uint32_t bit_keep(uint32_t m, int b) {
  return (uint32_t)__builtin_amdgcn_sbfe((int)m, b, 1);
}
__device__ __forceinline__ uint32_t bit_keep_imm(uint32_t m, int b) {
  uint32_t k;
  asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(k) : "v"(m), "I"(b));
  return k;
}
__device__ __forceinline__ float keep_bits(float x, uint32_t keep) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & keep);
}

}  // namespace hstu
