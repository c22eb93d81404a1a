// Targets-only mode (MLCommons training PR #903, "Summary"): one candidate row
// i_b per sequence forms Q against the full-length K and V.  The work per
// sequence is a pair of matrix-vector products over L_b key rows, so the path
// is bound by streaming K and V (and writing dK, dV) through HBM.
//
// Each wave owns one 64-row chunk of one (sequence, head); lanes are split into
// row groups of D/VEC lanes that each hold VEC consecutive elements of a key
// row (16-byte loads), so one wave instruction covers 64/(D/VEC) rows.  Dot
// products reduce across a row group with xor shuffles.  Rows the candidate
// does not see are never loaded (their dK, dV rows are written as zeros).
//
// Forward: O_b = (alpha/max_len) sum_j y_j v_j with y_j = x_j logistic(alpha x_j),
// x_j = <q_b, k_j>; each chunk writes a partial sum, and a second kernel adds the
// partials of a sequence in chunk order (fixed order: bitwise repeatable).
// Backward: dV_j = (alpha/max_len) y_j dO_b, dK_j = (alpha/max_len) p_j q_b with
// p_j = <dO_b, v_j> silu'(alpha x_j); dQ_b = (alpha/max_len) sum_j p_j k_j via the
// same chunk partials.
#include "common.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kChunk = kRB;  // rows per wave (partials indexed like row blocks)
constexpr int kWaves = 2;    // waves per workgroup: one unit = 128 rows

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  // K and V rows are streamed once and dK / dV written once: non-temporal
  // accesses (measured 3.6% faster than cached ones for the 2663-row shape)
  __device__ static void load(const uint16_t* p, float* out) {
    const u32x4 rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const uint4 r = make_uint4(rv[0], rv[1], rv[2], rv[3]);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(x[2 * i]) | ((uint32_t)f32_to_bf16(x[2 * i + 1]) << 16);
    const u32x4 wv = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(wv, reinterpret_cast<u32x4*>(p));
  }
  __device__ static uint16_t cvt(float x) { return f32_to_bf16(x); }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* out) {
    const float4 r = *reinterpret_cast<const float4*>(p);
    out[0] = r.x;
    out[1] = r.y;
    out[2] = r.z;
    out[3] = r.w;
  }
  __device__ static void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  __device__ static float cvt(float x) { return x; }
};

struct Candidate {
  int lo[kMaxNI], hi[kMaxNI];
  __device__ bool sees(int c, int ni) const {
    bool r = false;
#pragma unroll
    for (int j = 0; j < kMaxNI; ++j)
      if (j < ni) r = r || (c >= lo[j] && c < hi[j]);
    return r;
  }
};

// Common unit decoding.  Returns false if this wave has no chunk.
struct ChunkCtx {
  int b, h, chunk, L, cand, rb;
  int64_t s;
};

__device__ __forceinline__ bool chunk_ctx(const int4* units, const int32_t* target_rows,
                                          ChunkCtx& C) {
  UnitRec u;
  if (!unit_of_block(units, u)) return false;
  C.b = u.b;
  C.h = u.h;
  C.s = u.s;
  C.L = u.L;
  C.rb = u.rb;
  C.chunk = u.tile * kWaves + (int)(threadIdx.x >> 6);
  if (C.chunk * kChunk >= C.L) return false;
  C.cand = min(max((int)target_rows[C.b], 0), C.L - 1);
  return true;
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kWaves) void k_targets_fwd(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    float* __restrict__ partial, Prep P, const int4* __restrict__ units,
    int H, const int32_t* __restrict__ func, int nfunc,
    float alpha, const int32_t* __restrict__ target_rows) {
  using V = Vec16<T>;
  constexpr int VEC = V::N, LPR = D / VEC, RPW = 64 / LPR;
  ChunkCtx C;
  if (!chunk_ctx(units, target_rows, C)) return;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, rg = lane / LPR;
  const int ni = (nfunc + 1) / 2;
  Candidate cd;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    cd.lo[j] = C.L;
    cd.hi[j] = 0;
    if (j < ni) row_interval(func, P.total, C.s + C.cand, j, C.L, cd.lo[j], cd.hi[j]);
  }
  const int64_t rs = (int64_t)H * D;
  float qv[VEC], acc[VEC];
  V::load(q + ((int64_t)C.b * H + C.h) * D + sub * VEC, qv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const float c_exp = -alpha * kLog2e;
  const T* kbase = k + C.s * rs + (int64_t)C.h * D + sub * VEC;
  const T* vbase = v + C.s * rs + (int64_t)C.h * D + sub * VEC;
  for (int it = 0; it < kChunk / RPW; ++it) {
    const int c = C.chunk * kChunk + it * RPW + rg;
    const bool vis = c < C.L && cd.sees(c, ni);
    float kv[VEC], vv[VEC];
    if (vis) {
      V::load(kbase + (int64_t)c * rs, kv);
      V::load(vbase + (int64_t)c * rs, vv);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) kv[e] = vv[e] = 0.f;
    }
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) x += qv[e] * kv[e];
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m, 64);
    const float y = vis ? x * logistic_scaled(x, c_exp) : 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += y * vv[e];
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
  if (rg == 0) {
    float* dst = partial + ((int64_t)(C.rb + C.chunk) * H + C.h) * D + sub * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[e] = acc[e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kWaves) void k_targets_bwd(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, T* __restrict__ dk, T* __restrict__ dv,
    float* __restrict__ partial, Prep P, const int4* __restrict__ units,
    int H, const int32_t* __restrict__ func, int nfunc,
    float alpha, float out_scale, const int32_t* __restrict__ target_rows) {
  using V = Vec16<T>;
  constexpr int VEC = V::N, LPR = D / VEC, RPW = 64 / LPR;
  ChunkCtx C;
  if (!chunk_ctx(units, target_rows, C)) return;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR, rg = lane / LPR;
  const int ni = (nfunc + 1) / 2;
  Candidate cd;
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    cd.lo[j] = C.L;
    cd.hi[j] = 0;
    if (j < ni) row_interval(func, P.total, C.s + C.cand, j, C.L, cd.lo[j], cd.hi[j]);
  }
  const int64_t rs = (int64_t)H * D;
  float qv[VEC], gv[VEC], acc[VEC];
  V::load(q + ((int64_t)C.b * H + C.h) * D + sub * VEC, qv);
  V::load(dout + ((int64_t)C.b * H + C.h) * D + sub * VEC, gv);
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const float c_exp = -alpha * kLog2e;
  const int64_t base = C.s * rs + (int64_t)C.h * D + sub * VEC;
  for (int it = 0; it < kChunk / RPW; ++it) {
    const int c = C.chunk * kChunk + it * RPW + rg;
    const bool in = c < C.L;
    const bool vis = in && cd.sees(c, ni);
    float kv[VEC], vv[VEC];
    if (vis) {
      V::load(k + base + (int64_t)c * rs, kv);
      V::load(v + base + (int64_t)c * rs, vv);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) kv[e] = vv[e] = 0.f;
    }
    float x = 0.f, ds = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      x += qv[e] * kv[e];
      ds += gv[e] * vv[e];
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
      x += __shfl_xor(x, m, 64);
      ds += __shfl_xor(ds, m, 64);
    }
    float y = 0.f, p = 0.f;
    if (vis) {
      const float sg = logistic_scaled(x, c_exp);
      const float ax = alpha * x;
      y = x * sg;
      p = ds * (sg * (1.0f + ax * (1.0f - sg)));
    }
    if (in) {
      float wk[VEC], wv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        wk[e] = out_scale * p * qv[e];
        wv[e] = out_scale * y * gv[e];
      }
      V::store(dk + base + (int64_t)c * rs, wk);
      V::store(dv + base + (int64_t)c * rs, wv);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += p * kv[e];
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
  if (rg == 0) {
    float* dst = partial + ((int64_t)(C.rb + C.chunk) * H + C.h) * D + sub * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[e] = acc[e];
  }
}

// out[b][h][:] = scale * sum over the sequence's chunks (in chunk order).
template <typename T, int D>
__global__ __launch_bounds__(D) void k_targets_reduce(const float* __restrict__ partial,
                                                      T* __restrict__ out, Prep P, int H,
                                                      float scale) {
  const int b = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int L = (int)(P.so[b + 1] - P.so[b]);
  const int nch = (L + kChunk - 1) / kChunk;
  const float* src = partial + ((int64_t)P.rb_off[b] * H + h) * D + d;
  float acc = 0.f;
  for (int c = 0; c < nch; ++c) acc += src[(int64_t)c * H * D];
  out[((int64_t)b * H + h) * D + d] = Vec16<T>::cvt(acc * scale);
}

template <typename T, int D>
hipError_t fwd_impl(const void* q, const void* k, const void* v, void* o, const Prep& P,
                    const Units& U, int H, const int32_t* func, int nfunc, float alpha,
                    float scale, const int32_t* target_rows, float* partial, hipStream_t stream) {
  if (U.cap > 0) {
    ProfScope ps(stream, "k_targets_fwd");
    hipLaunchKernelGGL((k_targets_fwd<T, D>), dim3(U.cap), dim3(64 * kWaves), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, partial, P, U.list, H,
                       func, nfunc, alpha, target_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps(stream, "k_targets_reduce");
  hipLaunchKernelGGL((k_targets_reduce<T, D>), dim3(P.B, H), dim3(D), 0, stream,
                     (const float*)partial, (T*)o, P, H, scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_impl(const void* q, const void* k, const void* v, const void* dout, void* dq,
                    void* dk, void* dv, const Prep& P, const Units& U, int H, const int32_t* func,
                    int nfunc, float alpha, float scale, const int32_t* target_rows,
                    float* partial, hipStream_t stream) {
  if (U.cap > 0) {
    ProfScope ps(stream, "k_targets_bwd");
    hipLaunchKernelGGL((k_targets_bwd<T, D>), dim3(U.cap), dim3(64 * kWaves), 0, stream,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)dout, (T*)dk, (T*)dv,
                       partial, P, U.list, H, func, nfunc, alpha, scale, target_rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope ps(stream, "k_targets_reduce");
  hipLaunchKernelGGL((k_targets_reduce<T, D>), dim3(P.B, H), dim3(D), 0, stream,
                     (const float*)partial, (T*)dq, P, H, scale);
  return hipGetLastError();
}

}  // namespace

int targets_chunk_rows() { return kChunk; }

#define HSTU_TARGETS_DISPATCH(FN, ...)                                  \
  if (dtype == 1) {                                                     \
    switch (D) {                                                        \
      case 32: return FN<float, 32>(__VA_ARGS__);                       \
      case 64: return FN<float, 64>(__VA_ARGS__);                       \
      case 128: return FN<float, 128>(__VA_ARGS__);                     \
    }                                                                   \
  } else {                                                              \
    switch (D) {                                                        \
      case 32: return FN<uint16_t, 32>(__VA_ARGS__);                    \
      case 64: return FN<uint16_t, 64>(__VA_ARGS__);                    \
      case 128: return FN<uint16_t, 128>(__VA_ARGS__);                  \
    }                                                                   \
  }                                                                     \
  return hipErrorInvalidValue;

hipError_t launch_targets_fwd(int dtype, int D, const void* q, const void* k, const void* v,
                              void* o, const Prep& P, const Units& U, int H, const int32_t* func,
                              int nfunc, float alpha, float inv_max_len,
                              const int32_t* target_rows, float* partial, hipStream_t stream) {
  HSTU_TARGETS_DISPATCH(fwd_impl, q, k, v, o, P, U, H, func, nfunc, alpha, alpha * inv_max_len,
                        target_rows, partial, stream)
}

hipError_t launch_targets_bwd(int dtype, int D, const void* q, const void* k, const void* v,
                              const void* dout, void* dq, void* dk, void* dv, const Prep& P,
                              const Units& U, int H, const int32_t* func, int nfunc, float alpha,
                              float inv_max_len, const int32_t* target_rows, float* partial,
                              hipStream_t stream) {
  HSTU_TARGETS_DISPATCH(bwd_impl, q, k, v, dout, dq, dk, dv, P, U, H, func, nfunc, alpha,
                        alpha * inv_max_len, target_rows, partial, stream)
}

}  // namespace hstu
