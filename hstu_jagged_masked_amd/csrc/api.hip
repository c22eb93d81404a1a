// C ABI of libhstu_attn.so: argument validation, workspace planning and the
// launch sequence of each entry point.  Declarations and the full contract are
// in include/hstu_attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.h"
#include "hstu_attn.h"
#include "pstore.h"

namespace hstu {

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int device_fail(hipError_t e, const char* what) {
  return fail(HSTU_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int round8(int64_t x) { return (int)((x + kNumXcd - 1) / kNumXcd * kNumXcd); }

bool mfma_path(int dtype, int D) { return dtype == HSTU_BF16 && D == 128; }

}  // namespace

bool plan_workspace(Plan& p, int is_bwd, int64_t B, int64_t total, int H, int D, int nfunc,
                    int targets_only) {
  p = Plan();
  if (B < 1 || B > (1 << 24) || total < 0 || total > (int64_t)INT32_MAX || H < 1 || H > 255 ||
      nfunc < 1 || nfunc > kMaxNfunc)
    return false;
  p.ni = (nfunc + 1) / 2;
  const int64_t nrb = cdiv64(total, kRB) + B;
  if (nrb > INT32_MAX / 8) return false;
  p.nrb_cap = (int)nrb;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  p.off_flags = take(64 * sizeof(int));
  p.off_so = take((size_t)(B + 1) * sizeof(int64_t));
  p.off_order = take((size_t)B * sizeof(int));
  p.off_rb = take((size_t)(B + 1) * sizeof(int));
  p.off_t64 = take((size_t)(B + 1) * sizeof(int));
  p.off_t128 = take((size_t)(B + 1) * sizeof(int));
  p.off_env = take((size_t)nrb * p.ni * sizeof(int4));
  // unit lists: tiles of 128 rows, H per tile (one workgroup each: the
  // count must fit a grid dimension)
  const int64_t cap128 = (int64_t)H * (cdiv64(total, 128) + B);
  if (cap128 > INT32_MAX - kNumXcd) return false;
  p.cap_a = round8(cap128);
  p.cap_b = is_bwd ? round8(cap128) : 0;
  p.cap_c = is_bwd ? round8(cap128) : 0;
  p.off_units_a = take((size_t)p.cap_a * 2 * sizeof(int4));
  p.off_units_b = take((size_t)p.cap_b * 2 * sizeof(int4));
  p.off_units_c = take((size_t)p.cap_c * 2 * sizeof(int4));
  p.partial_bytes = 0;
  if (targets_only) {
    const int64_t nchunk = cdiv64(total, targets_chunk_rows()) + B;
    p.partial_bytes = (size_t)nchunk * H * D * sizeof(float);
  }
  p.off_partial = take(p.partial_bytes);
  if (is_bwd && !targets_only) p.off_pblk = take((size_t)(B + 1) * sizeof(int64_t));
  p.bytes = off;
  return true;
}

Prep prep_view(const Plan& p, void* ws, int B, int64_t total) {
  char* base = static_cast<char*>(ws);
  Prep P;
  P.flags = reinterpret_cast<int*>(base + p.off_flags);
  P.so = reinterpret_cast<int64_t*>(base + p.off_so);
  P.order = reinterpret_cast<int*>(base + p.off_order);
  P.rb_off = reinterpret_cast<int*>(base + p.off_rb);
  P.tiles64 = reinterpret_cast<int*>(base + p.off_t64);
  P.tiles128 = reinterpret_cast<int*>(base + p.off_t128);
  P.env = reinterpret_cast<int4*>(base + p.off_env);
  P.pblk = p.off_pblk ? reinterpret_cast<int64_t*>(base + p.off_pblk) : nullptr;
  P.B = B;
  P.total = total;
  P.row_lo = 0;
  P.row_hi = total;
  P.nrb_cap = p.nrb_cap;
  return P;
}

namespace {

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

// Common validation; on success fills the plan.
int validate(Plan& plan, int is_bwd, int dtype, int64_t B, int64_t total, int H, int D, int nfunc,
             float alpha, int64_t max_len, const int64_t* seq_offsets, const int32_t* func,
             const int32_t* target_rows, void* workspace, size_t workspace_bytes) {
  if (dtype != HSTU_BF16 && dtype != HSTU_FP32)
    return fail(HSTU_ERR_INVALID, "dtype must be HSTU_BF16 (0) or HSTU_FP32 (1), got %d", dtype);
  if (B < 1) return fail(HSTU_ERR_INVALID, "B must be >= 1, got %lld", (long long)B);
  if (B > (1 << 24)) return fail(HSTU_ERR_UNSUPPORTED, "B must be <= 2^24");
  if (total < 0) return fail(HSTU_ERR_INVALID, "total must be >= 0");
  if (total > (int64_t)INT32_MAX) return fail(HSTU_ERR_UNSUPPORTED, "total must be < 2^31");
  if (H < 1) return fail(HSTU_ERR_INVALID, "H must be >= 1, got %d", H);
  if (H > 255) return fail(HSTU_ERR_UNSUPPORTED, "H must be <= 255, got %d", H);
  if (D != 32 && D != 64 && D != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "D must be 32, 64 or 128, got %d", D);
  if (nfunc < 1 || (nfunc % 2) == 0)
    return fail(HSTU_ERR_INVALID, "nfunc must be odd and >= 1, got %d", nfunc);
  if (nfunc > kMaxNfunc)
    return fail(HSTU_ERR_UNSUPPORTED, "nfunc must be <= %d, got %d", kMaxNfunc, nfunc);
  if (!isfinite(alpha)) return fail(HSTU_ERR_INVALID, "alpha must be finite");
  if (max_len < 1) return fail(HSTU_ERR_INVALID, "max_len must be >= 1");
  if (!seq_offsets) return fail(HSTU_ERR_INVALID, "seq_offsets is NULL");
  if (!func && total > 0) return fail(HSTU_ERR_INVALID, "func is NULL");
  if (misaligned(seq_offsets) || misaligned(func) || misaligned(target_rows))
    return fail(HSTU_ERR_INVALID, "seq_offsets, func and target_rows must be 16-byte aligned");
  if (!plan_workspace(plan, is_bwd, B, total, H, D, nfunc, target_rows != nullptr))
    return fail(HSTU_ERR_UNSUPPORTED, "sizes out of range");
  if (workspace_bytes < plan.bytes || (!workspace && plan.bytes))
    return fail(HSTU_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                plan.bytes);
  if (misaligned(workspace)) return fail(HSTU_ERR_INVALID, "workspace must be 16-byte aligned");
  return HSTU_OK;
}

int check_tensor(const void* p, int64_t rows, const char* name) {
  if (rows > 0 && !p) return fail(HSTU_ERR_INVALID, "%s is NULL", name);
  if (misaligned(p)) return fail(HSTU_ERR_INVALID, "%s must be 16-byte aligned", name);
  return HSTU_OK;
}

Units units_view(void* ws, size_t off, int cap) {
  Units U;
  U.list = reinterpret_cast<int4*>(static_cast<char*>(ws) + off);
  U.cap = cap;
  return U;
}

}  // namespace

}  // namespace hstu

using namespace hstu;

extern "C" int hstu_max_nfunc(void) { return kMaxNfunc; }

extern "C" const char* hstu_last_error(void) { return g_last_error.c_str(); }

extern "C" size_t hstu_attn_workspace_size(int is_bwd, int64_t B, int64_t total, int H, int D,
                                           int nfunc, int targets_only) {
  Plan plan;
  if (!plan_workspace(plan, is_bwd, B, total, H, D, nfunc, targets_only)) return 0;
  return plan.bytes;
}

extern "C" int hstu_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o,
                             const int64_t* seq_offsets, int64_t B, int64_t total, int H, int D,
                             const int32_t* func, int nfunc, float alpha, int64_t max_len,
                             const int32_t* target_rows, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Plan plan;
  int st = validate(plan, 0, dtype, B, total, H, D, nfunc, alpha, max_len, seq_offsets, func,
                    target_rows, workspace, workspace_bytes);
  if (st) return st;
  const int64_t qrows = target_rows ? B : total;
  if ((st = check_tensor(q, qrows, "q")) || (st = check_tensor(k, total, "k")) ||
      (st = check_tensor(v, total, "v")) || (st = check_tensor(o, qrows, "o")))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float inv_max_len = (float)(1.0 / (double)max_len);
  Prep P = prep_view(plan, workspace, (int)B, total);
  hipError_t e = launch_prep(P, seq_offsets, target_rows, s);
  if (e != hipSuccess) return device_fail(e, "prep");
  if (target_rows) {
    float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.off_partial);
    const UnitJob job{units_view(workspace, plan.off_units_a, plan.cap_a), 128, 0, kSlotFwdUnits};
    e = launch_lists(P, nullptr, nfunc, &job, 1, H, s);
    if (e != hipSuccess) return device_fail(e, "unit list");
    const Units& U = job.U;
    e = launch_targets_fwd(dtype, D, q, k, v, o, P, U, H, func, nfunc, alpha, inv_max_len,
                           target_rows, partial, s);
    if (e != hipSuccess) return device_fail(e, "targets-only forward");
    return HSTU_OK;
  }
  if (mfma_path(dtype, D)) {
    const UnitJob job{units_view(workspace, plan.off_units_a, plan.cap_a), 128, 1, kSlotFwdUnits};
    e = launch_lists(P, func, nfunc, &job, 1, H, s);
    if (e != hipSuccess) return device_fail(e, "envelopes and unit list");
    e = launch_mfma_fwd(q, k, v, o, P, job.U, H, func, nfunc, alpha, inv_max_len, s);
  } else {
    e = launch_generic_fwd(dtype, D, q, k, v, o, P, H, func, nfunc, alpha, inv_max_len, nullptr,
                           s);
  }
  if (e != hipSuccess) return device_fail(e, "forward");
  return HSTU_OK;
}

// ---------------------------------------------------------------------------
// The forward without a caller workspace, for callers that cannot allocate
// device memory.  Its workspace is `scratch`, a fixed array in device memory
// that every GPU the library runs on holds (one copy per device) until the
// process ends.  Host code never passes the array's name to a kernel or a
// copy: the name is a host-side stand-in.  It uses the device address that
// hipGetSymbolAddress returns, fetched once per device with that device
// current and kept in g_scratch_ptr.  Every kernel of the forward writes the
// workspace bytes it later reads (the previous call's contents are never
// used), so nothing is cleared between calls.  Calls that overlap on one
// device share the array and race.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the device of `stream` (the current
// device for the null stream).
int scratch_address(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return device_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HSTU_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return device_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HSTU_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSTU_OK;
}

}  // namespace

extern "C" int hstu_attn_fwd_noalloc(int dtype, const void* q, const void* k, const void* v,
                                     void* o, const int64_t* seq_offsets, int64_t B,
                                     int64_t total, int H, int D, const int32_t* func, int nfunc,
                                     float alpha, int64_t max_len, const int32_t* target_rows,
                                     void* stream) {
  Plan plan;
  if (plan_workspace(plan, 0, B, total, H, D, nfunc, target_rows != nullptr) &&
      plan.bytes > kScratchBytes)
    return fail(HSTU_ERR_UNSUPPORTED,
                "these sizes need %zu bytes of workspace; the no-allocation forward holds %zu "
                "(use hstu_attn_fwd with a workspace)",
                plan.bytes, kScratchBytes);
  void* ws = nullptr;
  int st = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (st) return st;
  return hstu_attn_fwd(dtype, q, k, v, o, seq_offsets, B, total, H, D, func, nfunc, alpha,
                       max_len, target_rows, ws, kScratchBytes, stream);
}

extern "C" int hstu_attn_bwd(int dtype, const void* q, const void* k, const void* v,
                             const void* dout, void* dq, void* dk, void* dv,
                             const int64_t* seq_offsets, int64_t B, int64_t total, int H, int D,
                             const int32_t* func, int nfunc, float alpha, int64_t max_len,
                             const int32_t* target_rows, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Plan plan;
  int st = validate(plan, 1, dtype, B, total, H, D, nfunc, alpha, max_len, seq_offsets, func,
                    target_rows, workspace, workspace_bytes);
  if (st) return st;
  const int64_t qrows = target_rows ? B : total;
  if ((st = check_tensor(q, qrows, "q")) || (st = check_tensor(k, total, "k")) ||
      (st = check_tensor(v, total, "v")) || (st = check_tensor(dout, qrows, "dout")) ||
      (st = check_tensor(dq, qrows, "dq")) || (st = check_tensor(dk, total, "dk")) ||
      (st = check_tensor(dv, total, "dv")))
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float inv_max_len = (float)(1.0 / (double)max_len);
  Prep P = prep_view(plan, workspace, (int)B, total);
  hipError_t e = launch_prep(P, seq_offsets, target_rows, s);
  if (e != hipSuccess) return device_fail(e, "prep");
  if (target_rows) {
    float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.off_partial);
    const UnitJob job{units_view(workspace, plan.off_units_a, plan.cap_a), 128, 0, kSlotFwdUnits};
    e = launch_lists(P, nullptr, nfunc, &job, 1, H, s);
    if (e != hipSuccess) return device_fail(e, "unit list");
    const Units& U = job.U;
    e = launch_targets_bwd(dtype, D, q, k, v, dout, dq, dk, dv, P, U, H, func, nfunc, alpha,
                           inv_max_len, target_rows, partial, s);
    if (e != hipSuccess) return device_fail(e, "targets-only backward");
    return HSTU_OK;
  }
  if (mfma_path(dtype, D)) {
    const UnitJob jobs[2] = {
        {units_view(workspace, plan.off_units_b, plan.cap_b), 128, 0, kSlotKvUnits},
        {units_view(workspace, plan.off_units_c, plan.cap_c), 128, 1, kSlotQUnits}};
    e = launch_lists(P, func, nfunc, jobs, 2, H, s);
    if (e != hipSuccess) return device_fail(e, "envelopes and unit lists");
    e = launch_mfma_bwd(q, k, v, dout, dq, dk, dv, P, jobs[0].U, jobs[1].U, H, func, nfunc,
                        alpha, inv_max_len, nullptr, 0, s);
  } else {
    e = launch_generic_bwd(dtype, D, q, k, v, dout, dq, dk, dv, P, H, func, nfunc, alpha,
                           inv_max_len, nullptr, s);
  }
  if (e != hipSuccess) return device_fail(e, "backward");
  return HSTU_OK;
}

extern "C" size_t hstu_attn_pstore_bytes(const int64_t* seq_offsets, int64_t B, int64_t total,
                                         int H) {
  if (!seq_offsets || B < 1 || B > (1 << 24) || total < 0 || total > (int64_t)INT32_MAX || H < 1 ||
      H > 255)
    return 0;
  // the lengths the device sees: offsets clamped into [0, total], running
  // maximum, first 0 and last `total`
  int64_t blocks = 0, prev = 0, run = 0;
  for (int64_t b = 1; b <= B; ++b) {
    int64_t x = seq_offsets[b] < 0 ? 0 : (seq_offsets[b] > total ? total : seq_offsets[b]);
    run = x > run ? x : run;
    const int64_t cur = b == B ? total : run;
    blocks += pstore_seq_blocks(cur - prev);
    prev = cur;
  }
  return (size_t)blocks * H * kPBlockBytes;
}

namespace {

// Checks shared by the stored-P entry points (after validate()).
int check_pstore_args(int64_t total, int D, const void* q, const void* k, const void* v,
                      const void* dout, const void* dq, const void* dk, const void* dv,
                      const void* pstore) {
  int st;
  if (D != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "the stored-P backward needs D = 128, got %d", D);
  if ((st = check_tensor(q, total, "q")) || (st = check_tensor(k, total, "k")) ||
      (st = check_tensor(v, total, "v")) || (st = check_tensor(dout, total, "dout")) ||
      (st = check_tensor(dq, total, "dq")) || (st = check_tensor(dk, total, "dk")) ||
      (st = check_tensor(dv, total, "dv")))
    return st;
  if (total > 0 && !pstore) return fail(HSTU_ERR_INVALID, "pstore is NULL");
  if (reinterpret_cast<uintptr_t>(pstore) & 255u)
    return fail(HSTU_ERR_INVALID, "pstore must be 256-byte aligned");
  return HSTU_OK;
}

// The stored-P backward of the `nb` sequences whose offsets start at
// `seq_offsets`, their rows clamped into [row_lo, row_hi]: prep, both unit
// lists and the two passes, with grids sized for those rows.
int bwd_pstore_run(const Plan& plan, void* workspace, const void* q, const void* k,
                   const void* v, const void* dout, void* dq, void* dk, void* dv,
                   const int64_t* seq_offsets, int64_t nb, int64_t total, int64_t row_lo,
                   int64_t row_hi, int H, const int32_t* func, int nfunc, float alpha,
                   float inv_max_len, void* pstore, size_t pstore_bytes, hipStream_t s) {
  Prep P = prep_view(plan, workspace, (int)nb, total);
  P.row_lo = row_lo;
  P.row_hi = row_hi;
  const int64_t rows = row_hi - row_lo;
  P.nrb_cap = (int)std::min<int64_t>(plan.nrb_cap, cdiv64(rows, kRB) + nb);
  hipError_t e = launch_prep(P, seq_offsets, nullptr, s);
  if (e != hipSuccess) return device_fail(e, "prep");
  // The size the lengths need is known on the device only; the kernels
  // compare it with pstore_bytes themselves (every P access is range-checked
  // against the buffer, and dq is written as NaN when the buffer is too
  // small), so nothing here waits for the device.  Whatever the offsets
  // hold, the sanitized lengths sum to `rows`, so the grids below hold
  // every unit.
  const int cap = std::min(plan.cap_b, round8((int64_t)H * (cdiv64(rows, 128) + nb)));
  const UnitJob jobs[2] = {{units_view(workspace, plan.off_units_b, cap), 128, 0, kSlotKvUnits},
                           {units_view(workspace, plan.off_units_c, cap), 128, 1, kSlotQUnits}};
  e = launch_lists(P, func, nfunc, jobs, 2, H, s);
  if (e != hipSuccess) return device_fail(e, "envelopes and unit lists");
  e = launch_mfma_bwd(q, k, v, dout, dq, dk, dv, P, jobs[0].U, jobs[1].U, H, func, nfunc, alpha,
                      inv_max_len, static_cast<uint16_t*>(pstore), (uint64_t)pstore_bytes, s);
  if (e != hipSuccess) return device_fail(e, "backward");
  return HSTU_OK;
}

}  // namespace

extern "C" int hstu_attn_bwd_pstore(const void* q, const void* k, const void* v, const void* dout,
                                    void* dq, void* dk, void* dv, const int64_t* seq_offsets,
                                    int64_t B, int64_t total, int H, int D, const int32_t* func,
                                    int nfunc, float alpha, int64_t max_len, void* workspace,
                                    size_t workspace_bytes, void* pstore, size_t pstore_bytes,
                                    void* stream) {
  Plan plan;
  int st = validate(plan, 1, HSTU_BF16, B, total, H, D, nfunc, alpha, max_len, seq_offsets, func,
                    nullptr, workspace, workspace_bytes);
  if (st) return st;
  if ((st = check_pstore_args(total, D, q, k, v, dout, dq, dk, dv, pstore))) return st;
  return bwd_pstore_run(plan, workspace, q, k, v, dout, dq, dk, dv, seq_offsets, B, total, 0,
                        total, H, func, nfunc, alpha, (float)(1.0 / (double)max_len), pstore,
                        pstore_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int hstu_attn_bwd_pstore_chunked(const void* q, const void* k, const void* v,
                                         const void* dout, void* dq, void* dk, void* dv,
                                         const int64_t* seq_offsets, const int64_t* host_offsets,
                                         int64_t B, int64_t total, int H, int D,
                                         const int32_t* func, int nfunc, float alpha,
                                         int64_t max_len, void* workspace, size_t workspace_bytes,
                                         void* pstore, size_t pstore_bytes, void* stream) {
  Plan plan;
  int st = validate(plan, 1, HSTU_BF16, B, total, H, D, nfunc, alpha, max_len, seq_offsets, func,
                    nullptr, workspace, workspace_bytes);
  if (st) return st;
  if ((st = check_pstore_args(total, D, q, k, v, dout, dq, dk, dv, pstore))) return st;
  if (!host_offsets) return fail(HSTU_ERR_INVALID, "host_offsets is NULL");
  if (host_offsets[0] != 0 || host_offsets[B] != total)
    return fail(HSTU_ERR_INVALID, "host_offsets must run from 0 to total = %lld",
                (long long)total);
  for (int64_t b = 0; b < B; ++b)
    if (host_offsets[b + 1] < host_offsets[b])
      return fail(HSTU_ERR_INVALID, "host_offsets decrease at sequence %lld", (long long)b);
  // runs of consecutive sequences whose stored P fits the buffer, each cut
  // as long as it can be; every run is checked before the first launch, so
  // an error leaves the outputs untouched
  auto seq_bytes = [&](int64_t b) {
    return (uint64_t)pstore_seq_blocks(host_offsets[b + 1] - host_offsets[b]) * (uint64_t)H *
           kPBlockBytes;
  };
  auto run_end = [&](int64_t b0) {
    uint64_t need = 0;
    int64_t b1 = b0;
    while (b1 < B && need + seq_bytes(b1) <= (uint64_t)pstore_bytes) need += seq_bytes(b1++);
    return b1;
  };
  for (int64_t b0 = 0, b1; b0 < B; b0 = b1) {
    b1 = run_end(b0);
    if (b1 == b0)
      return fail(HSTU_ERR_INVALID,
                  "sequence %lld needs %llu bytes of stored P; the buffer holds %zu", (long long)b0,
                  (unsigned long long)seq_bytes(b0), pstore_bytes);
  }
  const float inv_max_len = (float)(1.0 / (double)max_len);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t b0 = 0, b1; b0 < B; b0 = b1) {
    b1 = run_end(b0);
    st = bwd_pstore_run(plan, workspace, q, k, v, dout, dq, dk, dv, seq_offsets + b0, b1 - b0,
                        total, host_offsets[b0], host_offsets[b1], H, func, nfunc, alpha,
                        inv_max_len, pstore, pstore_bytes, s);
    if (st) return st;
  }
  return HSTU_OK;
}

extern "C" int hstu_attn_bwd_atomic(const void* q, const void* k, const void* v, const void* dout,
                                    void* dq, void* dk, void* dv, const int64_t* seq_offsets,
                                    int64_t B, int64_t total, int H, int D, const int32_t* func,
                                    int nfunc, float alpha, int64_t max_len, void* workspace,
                                    size_t workspace_bytes, void* dq_accum, size_t dq_accum_bytes,
                                    void* stream) {
  Plan plan;
  int st = validate(plan, 1, HSTU_BF16, B, total, H, D, nfunc, alpha, max_len, seq_offsets, func,
                    nullptr, workspace, workspace_bytes);
  if (st) return st;
  if (D != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "the atomic-dQ backward needs D = 128, got %d", D);
  if ((st = check_tensor(q, total, "q")) || (st = check_tensor(k, total, "k")) ||
      (st = check_tensor(v, total, "v")) || (st = check_tensor(dout, total, "dout")) ||
      (st = check_tensor(dq, total, "dq")) || (st = check_tensor(dk, total, "dk")) ||
      (st = check_tensor(dv, total, "dv")))
    return st;
  const uint64_t need = (uint64_t)total * (uint64_t)H * (uint64_t)D * 4u;
  if (total > 0 && !dq_accum) return fail(HSTU_ERR_INVALID, "dq_accum is NULL");
  if (reinterpret_cast<uintptr_t>(dq_accum) & 255u)
    return fail(HSTU_ERR_INVALID, "dq_accum must be 256-byte aligned");
  if ((uint64_t)dq_accum_bytes < need)
    return fail(HSTU_ERR_INVALID, "dq_accum holds %zu bytes; [total, H, D] fp32 needs %llu",
                dq_accum_bytes, (unsigned long long)need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Prep P = prep_view(plan, workspace, (int)B, total);
  hipError_t e = launch_prep(P, seq_offsets, nullptr, s);
  if (e != hipSuccess) return device_fail(e, "prep");
  const UnitJob job{units_view(workspace, plan.off_units_b, plan.cap_b), 128, 0, kSlotKvUnits};
  e = launch_lists(P, func, nfunc, &job, 1, H, s);
  if (e != hipSuccess) return device_fail(e, "envelopes and unit list");
  e = launch_mfma_bwd_atomic(q, k, v, dout, dq, dk, dv, P, job.U, H, func, nfunc, alpha,
                             (float)(1.0 / (double)max_len), static_cast<float*>(dq_accum), total,
                             s);
  if (e != hipSuccess) return device_fail(e, "atomic-dQ backward");
  return HSTU_OK;
}

extern "C" int hstu_attn_visible_counts(const int64_t* seq_offsets, int64_t B, int64_t total,
                                        const int32_t* func, int nfunc,
                                        const int32_t* target_rows, int32_t* counts,
                                        int64_t* total_pairs, void* stream) {
  if (B < 1) return fail(HSTU_ERR_INVALID, "B must be >= 1");
  if (B > (1 << 24) || total > (int64_t)INT32_MAX)
    return fail(HSTU_ERR_UNSUPPORTED, "sizes out of range");
  if (total < 0) return fail(HSTU_ERR_INVALID, "total must be >= 0");
  if (nfunc < 1 || (nfunc % 2) == 0)
    return fail(HSTU_ERR_INVALID, "nfunc must be odd and >= 1, got %d", nfunc);
  if (nfunc > kMaxNfunc)
    return fail(HSTU_ERR_UNSUPPORTED, "nfunc must be <= %d, got %d", kMaxNfunc, nfunc);
  if (!seq_offsets) return fail(HSTU_ERR_INVALID, "seq_offsets is NULL");
  if (!func && total > 0) return fail(HSTU_ERR_INVALID, "func is NULL");
  hipError_t e = launch_visible_counts(seq_offsets, (int)B, total, func, nfunc, target_rows,
                                       counts, total_pairs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "visible counts");
  return HSTU_OK;
}

extern "C" int hstu_attn_check_inputs(const int64_t* seq_offsets, int64_t B, int64_t total,
                                      const int32_t* target_rows, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (B < 1) return fail(HSTU_ERR_INVALID, "B must be >= 1");
  if (total < 0) return fail(HSTU_ERR_INVALID, "total must be >= 0");
  if (!seq_offsets) return fail(HSTU_ERR_INVALID, "seq_offsets is NULL");
  if (misaligned(seq_offsets) || misaligned(target_rows))
    return fail(HSTU_ERR_INVALID, "seq_offsets and target_rows must be 16-byte aligned");
  Plan plan;
  if (!plan_workspace(plan, 0, B, total, 1, 128, 1, 0))
    return fail(HSTU_ERR_UNSUPPORTED, "sizes out of range");
  if (workspace_bytes < plan.bytes || !workspace)
    return fail(HSTU_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                plan.bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Prep P = prep_view(plan, workspace, (int)B, total);
  hipError_t e = launch_prep(P, seq_offsets, target_rows, s);
  if (e != hipSuccess) return device_fail(e, "prep");
  int flags = 0;
  e = hipMemcpyAsync(&flags, P.flags, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_fail(e, "reading validation flags");
  if (flags) {
    return fail(HSTU_ERR_INPUT, "malformed device input:%s%s%s%s",
                (flags & kFlagOffsetsStart) ? " seq_offsets[0] != 0;" : "",
                (flags & kFlagOffsetsEnd) ? " seq_offsets[B] != total;" : "",
                (flags & kFlagOffsetsOrder) ? " seq_offsets decreasing or out of range;" : "",
                (flags & kFlagTargetRange) ? " target row outside its sequence;" : "");
  }
  return HSTU_OK;
}
