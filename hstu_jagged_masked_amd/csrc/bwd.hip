// Backward kernels, bf16 inputs, D = 128, bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// With x = <q_i, k_j>, sg = logistic(alpha x), y = x sg and, for visible pairs,
//   silu(alpha x) = alpha y,   silu'(alpha x) = sg (1 + alpha x (1 - sg)),
//   dS_ij = <dO_i, v_j>,       p_ij = dS_ij silu'(alpha x_ij)   (= max_len dP_ij),
// the gradients are
//   dV_j = (alpha/max_len) sum_i y_ij dO_i,   dK_j = (alpha/max_len) sum_i p_ij q_i,
//   dQ_i = (alpha/max_len) sum_j p_ij k_j.
// Masked pairs contribute nothing: y and p are zeroed there (silu'(0) = 1/2,
// so zeroing only y would be wrong).
//
// Two kernels, each output written by exactly one workgroup (no atomics), so
// every gradient is bitwise repeatable:
//   k_bwd_kv  one workgroup per (sequence, head, 128 key rows); wave w owns keys
//             [32w, 32w+32) and keeps their K and V rows in registers; it walks
//             the 64-row query blocks whose envelopes reach its keys:
//               S = Q K^T, dS = dO V^T          (A from LDS, B = K, V registers)
//               y, p in registers (mask via per-row bitmasks in LDS)
//               dV^T += dO^T Y,  dK^T += Q^T P  (A = transpose reads of the
//                                                row-major Q / dO tiles)
//   k_bwd_q   one workgroup per (sequence, head, 128 query rows), the forward's
//             walk over key tiles:
//               S^T = K Q^T, dS^T = V dO^T      (B = Q, dO registers)
//               p in registers
//               dQ^T += K^T P^T                 (A = transpose reads of K)
#include "common.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
// k_bwd_kv
constexpr int kKvBN = 128;         // key rows per workgroup
constexpr int kKvBM = 64;          // query rows per step (one row block)
constexpr int kQStr = kD + 8;      // LDS row stride of the Q / dO tiles (bf16)
// k_bwd_q
constexpr int kQBM = 128;          // query rows per workgroup
constexpr int kQBN = 64;           // key columns per tile
constexpr int kKStr = kD + 8;      // LDS row stride of K / V tiles (bf16)

__device__ __forceinline__ bf16x8 concat4(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__global__ __launch_bounds__(kThreads, 1) void k_bwd_kv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, Prep P, const int4* __restrict__ units,
    const int* __restrict__ unit_count, int H, const int32_t* __restrict__ func, int nfunc,
    float alpha, float out_scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kKvBM * kQStr];
  __shared__ __attribute__((aligned(16))) uint16_t sG[kKvBM * kQStr];  // dO tile
  __shared__ __attribute__((aligned(16))) uint32_t sMask[4][kKvBM];

  const int slot = xcd_slot(blockIdx.x, *unit_count);
  if (slot < 0) return;
  const int4 u = units[slot];
  const int b = u.x, kt = u.y, h = u.z;
  const int64_t s = P.so[b];
  const int L = (int)(P.so[b + 1] - s);
  const int c0 = kt * kKvBN;
  const int c1 = min(c0 + kKvBN, L);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;
  const float c_exp = -alpha * kLog2e;

  // this lane's key column and its K / V rows (B operands: [k = d][n = key])
  const int col = c0 + wave * 32 + n;
  const bool col_ok = col < L;
  bf16x8 kf[kD / 16], vf[kD / 16];
  {
    const uint16_t* kp = k + (s + col) * rs + (int64_t)h * kD + g * 8;
    const uint16_t* vp = v + (s + col) * rs + (int64_t)h * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      kf[ks] = col_ok ? *reinterpret_cast<const bf16x8*>(kp + ks * 16) : bf16x8{};
      vf[ks] = col_ok ? *reinterpret_cast<const bf16x8*>(vp + ks * 16) : bf16x8{};
    }
  }
  f32x16 dkacc[kD / 32], dvacc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }

  // tile loads: rows lrow + 16i of the block, dims lcol..lcol+7
  const int lrow = tid >> 4, lcol = (tid & 15) * 8;
  // transpose-read base: lane j of 16-lane group G -> row 4*(G/2) + j/4,
  // column (G%2)*16 + 4*(j%4)
  const int grp = lane >> 4, gl = lane & 15;
  const int tr_off = (4 * (grp >> 1) + (gl >> 2)) * kQStr + (grp & 1) * 16 + 4 * (gl & 3);

  const int nrb = (L + kRB - 1) / kRB;
  const int4* env = P.env + (int64_t)P.rb_off[b] * ni;
  for (int rb = 0; rb < nrb; ++rb) {
    bool live, full;
    block_vs_cols(env + (int64_t)rb * ni, ni, c0, c1, live, full);
    if (!live) continue;
    const int q0 = rb * kRB;
    // stage the Q and dO rows of this block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 16 * i;
      uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
      if (q0 + r < L) {
        a = *reinterpret_cast<const uint4*>(q + (s + q0 + r) * rs + (int64_t)h * kD + lcol);
        c = *reinterpret_cast<const uint4*>(dout + (s + q0 + r) * rs + (int64_t)h * kD + lcol);
      }
      *reinterpret_cast<uint4*>(&sQ[r * kQStr + lcol]) = a;
      *reinterpret_cast<uint4*>(&sG[r * kQStr + lcol]) = c;
    }
    if (!full) {
      // row q0 + lane: visibility of this wave's 32 key columns
      int lo[kMaxNI], hi[kMaxNI];
      const int r = q0 + lane;
#pragma unroll
      for (int j = 0; j < kMaxNI; ++j) {
        lo[j] = L;
        hi[j] = 0;
        if (j < ni && r < L) row_interval(func, P.total, s + r, j, L, lo[j], hi[j]);
      }
      sMask[wave][lane] = col_mask32(lo, hi, ni, c0 + wave * 32);
    }
    __syncthreads();

    // S = Q K^T and dS = dO V^T for the block's two 32-row halves
    f32x16 sacc[2], dsacc[2];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      sacc[mq] = f32x16{};
      dsacc[mq] = f32x16{};
      const uint16_t* qp = &sQ[(mq * 32 + n) * kQStr + g * 8];
      const uint16_t* gp = &sG[(mq * 32 + n) * kQStr + g * 8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        sacc[mq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(qp + ks * 16), kf[ks], sacc[mq], 0, 0, 0);
        dsacc[mq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(gp + ks * 16), vf[ks], dsacc[mq], 0, 0, 0);
      }
    }
    // y and p per element: row mq*32 + (r/4)*8 + g*4 + r%4, column `col`
    bf16x8 yb[4], pb[4];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint4 m4 = make_uint4(~0u, ~0u, ~0u, ~0u);
        if (!full) m4 = *reinterpret_cast<const uint4*>(&sMask[wave][mq * 32 + jj * 8 + g * 4]);
        const uint32_t mrow[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = jj * 4 + i;
          const float x = sacc[mq][r];
          const float sg = logistic_scaled(x, c_exp);
          const float ax = alpha * x;
          float y = x * sg;
          float p = dsacc[mq][r] * (sg * (1.0f + ax * (1.0f - sg)));
          if (!((mrow[i] >> n) & 1u)) {
            y = 0.f;
            p = 0.f;
          }
          yb[mq * 2 + (r >> 3)][r & 7] = (__bf16)y;
          pb[mq * 2 + (r >> 3)][r & 7] = (__bf16)p;
        }
      }
    }
    // dV^T += dO^T Y and dK^T += Q^T P: A operands by transpose reads, query
    // rows 16ss + 4g + {0..3} and 16ss + 8 + 4g + {0..3} (ss = 2mq + half)
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
#pragma unroll
      for (int mb = 0; mb < kD / 32; ++mb) {
        const int off = tr_off + 16 * ss * kQStr + mb * 32;
        const bf16x8 ag = concat4(lds_read_tr(&sG[off]), lds_read_tr(&sG[off + 8 * kQStr]));
        dvacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, yb[ss], dvacc[mb], 0, 0, 0);
        const bf16x8 aq = concat4(lds_read_tr(&sQ[off]), lds_read_tr(&sQ[off + 8 * kQStr]));
        dkacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, pb[ss], dkacc[mb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds d = mb*32 + j*8 + g*4 + 0..3 of key row `col`
  if (col_ok) {
    uint16_t* kp = dk + (s + col) * rs + (int64_t)h * kD + g * 4;
    uint16_t* vp = dv + (s + col) * rs + (int64_t)h * kD + g * 4;
#pragma unroll
    for (int mb = 0; mb < kD / 32; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 wk, wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wk[i] = (__bf16)(dkacc[mb][j * 4 + i] * out_scale);
          wv[i] = (__bf16)(dvacc[mb][j * 4 + i] * out_scale);
        }
        *reinterpret_cast<bf16x4*>(kp + mb * 32 + j * 8) = wk;
        *reinterpret_cast<bf16x4*>(vp + mb * 32 + j * 8) = wv;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_bwd_q(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    Prep P, const int4* __restrict__ units, const int* __restrict__ unit_count, int H,
    const int32_t* __restrict__ func, int nfunc, float alpha, float out_scale) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kQBN * kKStr];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kQBN * kKStr];

  const int slot = xcd_slot(blockIdx.x, *unit_count);
  if (slot < 0) return;
  const int4 u = units[slot];
  const int b = u.x, qt = u.y, h = u.z;
  const int64_t s = P.so[b];
  const int L = (int)(P.so[b + 1] - s);
  const int r0 = qt * kQBM;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;
  const float c_exp = -alpha * kLog2e;

  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < L;
  bf16x8 qf[kD / 16], gf[kD / 16];
  {
    const uint16_t* qp = q + (s + row) * rs + (int64_t)h * kD + g * 8;
    const uint16_t* gp = dout + (s + row) * rs + (int64_t)h * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + ks * 16) : bf16x8{};
      gf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(gp + ks * 16) : bf16x8{};
    }
  }
  int lo[kMaxNI], hi[kMaxNI];
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    lo[j] = L;
    hi[j] = 0;
    if (j < ni && row_ok) row_interval(func, P.total, s + row, j, L, lo[j], hi[j]);
  }
  TileRanges R;
  tile_ranges(P, b, r0, kQBM, L, ni, kQBN, R);

  f32x16 dqacc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) dqacc[mb] = f32x16{};

  const int krow = tid >> 4, kcol = (tid & 15) * 8;
  const int grp = lane >> 4, gl = lane & 15;
  const int tr_off = (4 * (grp >> 1) + (gl >> 2)) * kKStr + (grp & 1) * 16 + 4 * (gl & 3);

  for (int t = next_live(R, ni, 0); t >= 0; t = next_live(R, ni, t + 1)) {
    const int c0 = t * kQBN;
    const bool full = tile_full(R, ni, c0, min(c0 + kQBN, L));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kv = krow + 16 * i;
      uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
      if (c0 + kv < L) {
        a = *reinterpret_cast<const uint4*>(k + (s + c0 + kv) * rs + (int64_t)h * kD + kcol);
        c = *reinterpret_cast<const uint4*>(v + (s + c0 + kv) * rs + (int64_t)h * kD + kcol);
      }
      *reinterpret_cast<uint4*>(&sK[kv * kKStr + kcol]) = a;
      *reinterpret_cast<uint4*>(&sV[kv * kKStr + kcol]) = c;
    }
    __syncthreads();

    f32x16 sacc[2], dsacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      dsacc[kb] = f32x16{};
      const uint16_t* kp = &sK[(kb * 32 + n) * kKStr + g * 8];
      const uint16_t* vp = &sV[(kb * 32 + n) * kKStr + g * 8];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kp + ks * 16), qf[ks], sacc[kb], 0, 0, 0);
        dsacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(vp + ks * 16), gf[ks], dsacc[kb], 0, 0, 0);
      }
    }
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t mg = 0xffffffffu;
      if (!full) mg = col_mask32(lo, hi, ni, c0 + kb * 32) >> (g * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = sacc[kb][r];
        const float sg = logistic_scaled(x, c_exp);
        const float ax = alpha * x;
        float p = dsacc[kb][r] * (sg * (1.0f + ax * (1.0f - sg)));
        const int bit = (r >> 2) * 8 + (r & 3);
        if (!((mg >> bit) & 1u)) p = 0.f;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    }
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
#pragma unroll
      for (int mb = 0; mb < kD / 32; ++mb) {
        const int off = tr_off + 16 * ss * kKStr + mb * 32;
        const bf16x8 a = concat4(lds_read_tr(&sK[off]), lds_read_tr(&sK[off + 8 * kKStr]));
        dqacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ss], dqacc[mb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (row_ok) {
    uint16_t* op = dq + (s + row) * rs + (int64_t)h * kD + g * 4;
#pragma unroll
    for (int mb = 0; mb < kD / 32; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = (__bf16)(dqacc[mb][j * 4 + i] * out_scale);
        *reinterpret_cast<bf16x4*>(op + mb * 32 + j * 8) = w4;
      }
    }
  }
}

}  // namespace

hipError_t launch_mfma_bwd(const void* q, const void* k, const void* v, const void* dout,
                           void* dq, void* dk, void* dv, const Prep& P, const Units& Ukv,
                           const Units& Uq, int H, const int32_t* func, int nfunc, float alpha,
                           float inv_max_len, hipStream_t stream) {
  const float scale = alpha * inv_max_len;
  if (Ukv.cap > 0) {
    ProfScope ps(stream, "k_bwd_kv");
    hipLaunchKernelGGL(k_bwd_kv, dim3(Ukv.cap), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), P, Ukv.list,
                       P.flags + kSlotKvUnits, H, func, nfunc, alpha, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (Uq.cap > 0) {
    ProfScope ps(stream, "k_bwd_q");
    hipLaunchKernelGGL(k_bwd_q, dim3(Uq.cap), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                       static_cast<uint16_t*>(dq), P, Uq.list, P.flags + kSlotQUnits, H, func,
                       nfunc, alpha, scale);
  }
  return hipGetLastError();
}

}  // namespace hstu
