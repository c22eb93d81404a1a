// Generic kernels: plain fp32 FMA loops over visible columns, for every
// supported element type and head dimension.  They serve the fp32 path (exact
// fp32 arithmetic with the accurate expf, no bf16 rounding of intermediates)
// and D in {32, 64} for bf16.  One thread owns one (query row, head) for the
// forward and dQ, and one (key row, head, 32-wide slice of D) for dK/dV.
//
// Operator (HSTU attention with the PR #670 interval mask):
//   S_ij = silu(alpha <q_i,k_j>) / max_len over visible j,  O_i = sum S_ij v_j,
//   dP_ij = <dO_i,v_j> silu'(alpha <q_i,k_j>) / max_len,
//   dQ_i = alpha sum_j dP_ij k_j,  dK_j = alpha sum_i dP_ij q_i,  dV_j = sum_i S_ij dO_i.
#include "common.h"

namespace hstu {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st(T* p, float x);
template <>
__device__ __forceinline__ void st<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

__device__ __forceinline__ float silu_exact(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float silu_grad_exact(float x) {
  const float s = 1.0f / (1.0f + expf(-x));
  return s * (1.0f + x * (1.0f - s));
}

// Locate query row `t` (a global row, or sequence `t` in targets-only mode).
// Returns false when the row has no sequence (cannot happen for sane input).
__device__ __forceinline__ bool locate(const Prep& P, int64_t t, const int32_t* target_rows,
                                       int& b, int64_t& start, int& L, int& i) {
  if (target_rows) {
    b = (int)t;
  } else {
    b = upper_index(P.so, P.B, t);
    if (b >= P.B) return false;
  }
  start = P.so[b];
  L = (int)(P.so[b + 1] - start);
  if (target_rows) {
    i = target_rows[b];
    if (L == 0) return false;
    i = min(max(i, 0), L - 1);
  } else {
    i = (int)(t - start);
  }
  return i >= 0 && i < L;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_fwd_rows(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, T* __restrict__ o,
                                                 Prep P, int H, const int32_t* __restrict__ func,
                                                 int nfunc, float alpha, float inv_max_len,
                                                 const int32_t* __restrict__ target_rows) {
  const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y;
  const int64_t rows = target_rows ? P.B : P.total;
  if (t >= rows) return;
  T* orow = o + (t * H + h) * D;
  int b, L, i;
  int64_t s;
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  if (locate(P, t, target_rows, b, s, L, i)) {
    const T* qrow = q + (t * H + h) * D;
    float qv[D];
    for (int d = 0; d < D; ++d) qv[d] = ld(qrow + d);
    int lo[kMaxNI], hi[kMaxNI];
    const int m = merged_intervals(func, P.total, s + i, nfunc, L, lo, hi);
    for (int r = 0; r < m; ++r) {
      for (int c = lo[r]; c < hi[r]; ++c) {
        const T* kr = k + ((s + c) * H + h) * D;
        const T* vr = v + ((s + c) * H + h) * D;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot += qv[d] * ld(kr + d);
        const float sc = silu_exact(alpha * dot) * inv_max_len;
        for (int d = 0; d < D; ++d) acc[d] += sc * ld(vr + d);
      }
    }
  }
  for (int d = 0; d < D; ++d) st(orow + d, acc[d]);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_bwd_rows(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v,
                                                 const T* __restrict__ dout, T* __restrict__ dq,
                                                 Prep P, int H, const int32_t* __restrict__ func,
                                                 int nfunc, float alpha, float inv_max_len,
                                                 const int32_t* __restrict__ target_rows) {
  const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y;
  const int64_t rows = target_rows ? P.B : P.total;
  if (t >= rows) return;
  T* dqrow = dq + (t * H + h) * D;
  int b, L, i;
  int64_t s;
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  if (locate(P, t, target_rows, b, s, L, i)) {
    const T* qrow = q + (t * H + h) * D;
    const T* grow = dout + (t * H + h) * D;
    int lo[kMaxNI], hi[kMaxNI];
    const int m = merged_intervals(func, P.total, s + i, nfunc, L, lo, hi);
    for (int r = 0; r < m; ++r) {
      for (int c = lo[r]; c < hi[r]; ++c) {
        const T* kr = k + ((s + c) * H + h) * D;
        const T* vr = v + ((s + c) * H + h) * D;
        float dot = 0.f, ds = 0.f;
        for (int d = 0; d < D; ++d) {
          dot += ld(qrow + d) * ld(kr + d);
          ds += ld(grow + d) * ld(vr + d);
        }
        const float dp = ds * silu_grad_exact(alpha * dot) * inv_max_len;
        for (int d = 0; d < D; ++d) acc[d] += alpha * dp * ld(kr + d);
      }
    }
  }
  for (int d = 0; d < D; ++d) st(dqrow + d, acc[d]);
}

// dK/dV for key row t, head h, dims [32*blockIdx.z, +32).  Scans the query rows
// of the sequence (only the candidate in targets-only mode) and tests whether
// each sees column j.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_bwd_cols(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v,
                                                 const T* __restrict__ dout, T* __restrict__ dk,
                                                 T* __restrict__ dv, Prep P, int H,
                                                 const int32_t* __restrict__ func, int nfunc,
                                                 float alpha, float inv_max_len,
                                                 const int32_t* __restrict__ target_rows) {
  const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y;
  const int d0 = blockIdx.z * 32;
  if (t >= P.total) return;
  float ak[32], av[32];
  for (int d = 0; d < 32; ++d) ak[d] = av[d] = 0.f;
  const int b = upper_index(P.so, P.B, t);
  if (b < P.B) {
    const int64_t s = P.so[b];
    const int L = (int)(P.so[b + 1] - s);
    const int j = (int)(t - s);
    const T* kr = k + (t * H + h) * D;
    const T* vr = v + (t * H + h) * D;
    int r0 = 0, r1 = L;
    if (target_rows) {
      r0 = min(max((int)target_rows[b], 0), L - 1);
      r1 = r0 + 1;
    }
    for (int i = r0; i < r1; ++i) {
      const int ni = (nfunc + 1) / 2;
      bool vis = false;
      for (int jj = 0; jj < ni; ++jj) {
        int lo, hi;
        row_interval(func, P.total, s + i, jj, L, lo, hi);
        vis = vis || (j >= lo && j < hi);
      }
      if (!vis) continue;
      const int64_t qr = target_rows ? (int64_t)b : s + i;
      const T* qrow = q + (qr * H + h) * D;
      const T* grow = dout + (qr * H + h) * D;
      float dot = 0.f, ds = 0.f;
      for (int d = 0; d < D; ++d) {
        dot += ld(qrow + d) * ld(kr + d);
        ds += ld(grow + d) * ld(vr + d);
      }
      const float x = alpha * dot;
      const float sc = silu_exact(x) * inv_max_len;
      const float dp = ds * silu_grad_exact(x) * inv_max_len;
      for (int d = 0; d < 32; ++d) {
        ak[d] += alpha * dp * ld(qrow + d0 + d);
        av[d] += sc * ld(grow + d0 + d);
      }
    }
  }
  T* dkr = dk + (t * H + h) * D + d0;
  T* dvr = dv + (t * H + h) * D + d0;
  for (int d = 0; d < 32; ++d) {
    st(dkr + d, ak[d]);
    st(dvr + d, av[d]);
  }
}

template <typename T, int D>
hipError_t fwd_impl(const void* q, const void* k, const void* v, void* o, const Prep& P, int H,
                    const int32_t* func, int nfunc, float alpha, float inv_max_len,
                    const int32_t* target_rows, hipStream_t stream) {
  const int64_t rows = target_rows ? P.B : P.total;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 63) / 64), H);
  ProfScope ps(stream, "k_generic_fwd");
  hipLaunchKernelGGL((k_fwd_rows<T, D>), grid, dim3(64), 0, stream, (const T*)q, (const T*)k,
                     (const T*)v, (T*)o, P, H, func, nfunc, alpha, inv_max_len, target_rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_impl(const void* q, const void* k, const void* v, const void* dout, void* dq,
                    void* dk, void* dv, const Prep& P, int H, const int32_t* func, int nfunc,
                    float alpha, float inv_max_len, const int32_t* target_rows,
                    hipStream_t stream) {
  const int64_t rows = target_rows ? P.B : P.total;
  if (rows > 0) {
    dim3 grid((unsigned)((rows + 63) / 64), H);
    ProfScope ps(stream, "k_generic_bwd_rows");
    hipLaunchKernelGGL((k_bwd_rows<T, D>), grid, dim3(64), 0, stream, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)dout, (T*)dq, P, H, func, nfunc, alpha,
                       inv_max_len, target_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (P.total > 0) {
    dim3 grid((unsigned)((P.total + 63) / 64), H, D / 32);
    ProfScope ps(stream, "k_generic_bwd_cols");
    hipLaunchKernelGGL((k_bwd_cols<T, D>), grid, dim3(64), 0, stream, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)dout, (T*)dk, (T*)dv, P, H, func, nfunc, alpha,
                       inv_max_len, target_rows);
  }
  return hipGetLastError();
}

}  // namespace

#define HSTU_DISPATCH_D(T, FN, ...)                     \
  switch (D) {                                          \
    case 32: return FN<T, 32>(__VA_ARGS__);             \
    case 64: return FN<T, 64>(__VA_ARGS__);             \
    case 128: return FN<T, 128>(__VA_ARGS__);           \
    default: return hipErrorInvalidValue;               \
  }

hipError_t launch_generic_fwd(int dtype, int D, const void* q, const void* k, const void* v,
                              void* o, const Prep& P, int H, const int32_t* func, int nfunc,
                              float alpha, float inv_max_len, const int32_t* target_rows,
                              hipStream_t stream) {
  if (dtype == 1) {
    HSTU_DISPATCH_D(float, fwd_impl, q, k, v, o, P, H, func, nfunc, alpha, inv_max_len,
                    target_rows, stream)
  }
  HSTU_DISPATCH_D(uint16_t, fwd_impl, q, k, v, o, P, H, func, nfunc, alpha, inv_max_len,
                  target_rows, stream)
}

hipError_t launch_generic_bwd(int dtype, int D, const void* q, const void* k, const void* v,
                              const void* dout, void* dq, void* dk, void* dv, const Prep& P,
                              int H, const int32_t* func, int nfunc, float alpha,
                              float inv_max_len, const int32_t* target_rows, hipStream_t stream) {
  if (dtype == 1) {
    HSTU_DISPATCH_D(float, bwd_impl, q, k, v, dout, dq, dk, dv, P, H, func, nfunc, alpha,
                    inv_max_len, target_rows, stream)
  }
  HSTU_DISPATCH_D(uint16_t, bwd_impl, q, k, v, dout, dq, dk, dv, P, H, func, nfunc, alpha,
                  inv_max_len, target_rows, stream)
}

}  // namespace hstu
