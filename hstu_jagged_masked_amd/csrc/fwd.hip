// Forward kernel, bf16 inputs, D = 128, bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
//   O_i = (alpha / max_len) * sum_{j in V_i} y_ij v_j,  y_ij = x_ij * logistic(alpha x_ij),
//   x_ij = <q_i, k_j>   (so that alpha * y_ij = silu(alpha x_ij)).
//
// One workgroup (4 waves) owns 128 query rows of one (sequence, head); wave w
// owns rows [32w, 32w+32) of the tile.  Wave 0 lists, 64 tiles at a time, the
// key tiles of 64 columns that the rows' interval envelopes reach (the rest are
// never loaded) and flags the tiles every row sees whole.  For each listed tile:
//   1. K and V tiles -> LDS, both row-major, by asynchronous buffer-to-LDS
//      DMA into one of two stages, so the next tile's copy runs during this
//      tile's math (one barrier per tile); the buffer range check zero-fills
//      rows past the sequence end;
//   2. S^T = K Q^T on MFMA: A = K from LDS, B = Q^T from registers (each lane
//      keeps its query row's 128 dims), so the accumulator holds one query row
//      per lane and 16 key columns;
//   3. y = x * logistic(alpha x) in registers (v_exp_f32, v_rcp_f32), the
//      interval mask applied only on tiles that some row sees partially, then
//      rounded to bf16 -- already in the B-operand layout of the next product;
//   4. O^T += V^T Y^T on MFMA: A = V^T read from the row-major V tile with the
//      LDS transpose read, B = Y^T from registers.
// The key index order inside each 16-wide MFMA step is permuted identically
// in both operands (it is a sum), which is what lets step 3 feed step 4
// without any data movement.
#include <type_traits>

#include "common.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kD = 128;
constexpr int kBM = 128;             // query rows per workgroup
constexpr int kBN = 64;              // key columns per tile
constexpr int kKStr = kD + 8;        // LDS row stride of K (bf16): 272 B, b128 reads conflict-free
constexpr int kVStr = kD + 32;       // LDS row stride of V (bf16): 320 B, transpose reads conflict-free
constexpr int kThreads = 256;
constexpr int kKStage = kBN * kKStr;         // bf16 elements per K stage
constexpr int kVStage = kBN * kVStr;
constexpr int kKSlots = kKStr * 2 / 16;      // 16-byte DMA slots per LDS row
constexpr int kVSlots = kVStr * 2 / 16;
constexpr int kKInstr = kBN * kKSlots / 64;  // wave DMA instructions per stage
constexpr int kVInstr = kBN * kVSlots / 64;
constexpr int kDmaPerWave = (kVInstr + 3) / 4;
static_assert(kBN * kKSlots % 64 == 0 && kBN * kVSlots % 64 == 0, "whole DMA instructions");
static_assert(kKInstr <= 4 * kDmaPerWave && kVInstr <= 4 * kDmaPerWave, "DMA split");

__global__ __launch_bounds__(kThreads, 2) void k_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, Prep P, const int4* __restrict__ units,
    int H, const int32_t* __restrict__ func, int nfunc, float alpha, float out_scale) {
  // two LDS stages as separate objects, so the compiler sees that the DMA
  // filling one stage does not alias the reads of the other
  __shared__ __attribute__((aligned(16))) uint16_t sK0[kKStage], sK1[kKStage];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[kVStage], sV1[kVStage];
  __shared__ int sPart[kListWin], sFull[kListWin];
  __shared__ int sCount[2];
  __shared__ Envelope sEnv;

  UnitRec u;
  if (!unit_of_block(units, u)) return;
  const int qt = u.tile, h = u.h, L = u.L;
  const int64_t s = u.s;
  const int r0 = qt * kBM;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;  // row stride (elements)
  const int rs2 = H * kD * 2;          // row stride (bytes)

  // the block's envelope first: the tile list, and with it the first copy,
  // then need not wait behind the q and func loads
  if (tid == 0) rows_envelope(P, u.rb, r0, kBM, L, ni, sEnv);
  // this lane's query row (B-operand column n of wave `wave`)
  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < L;
  bf16x8 qf[kD / 16];
  {
    const uint16_t* qp = q + (s + row) * rs + (int64_t)h * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + ks * 16) : bf16x8{};
  }
  int lo[kMaxNI], hi[kMaxNI];
#pragma unroll
  for (int j = 0; j < kMaxNI; ++j) {
    lo[j] = L;
    hi[j] = 0;
    if (j < ni && row_ok) row_interval(func, P.total, s + row, j, L, lo[j], hi[j]);
  }

  __syncthreads();
  int t_begin, t_end;
  envelope_tile_span(sEnv, ni, kBN, t_begin, t_end);

  f32x16 oacc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) oacc[mb] = f32x16{};

  const float c_exp = -alpha * kLog2e;
  const uint16_t* kh = k + s * rs + (int64_t)h * kD;
  const uint16_t* vh = v + s * rs + (int64_t)h * kD;

  // DMA: wave w issues instructions I = w + 4i of a stage; lane l of
  // instruction I fills LDS slot 64*I + l (padding slots read out of range)
  int koff[kDmaPerWave], voff[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int slot = (wave + 4 * i) * 64 + lane;
    koff[i] = dma_slot_offset(slot, kKSlots, rs2);
    voff[i] = dma_slot_offset(slot, kVSlots, rs2);
  }
  auto dma_tile = [&](int t, auto stage) {
    constexpr int st = decltype(stage)::value;
    const int c0 = t * kBN;
    const int rows = min(kBN, L - c0);
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kh + (int64_t)c0 * rs, rows, rs2, kD * 2);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vh + (int64_t)c0 * rs, rows, rs2, kD * 2);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int I = wave + 4 * i;
      if (I < kKInstr) lds_dma16(rk, (st ? sK1 : sK0) + I * 512, koff[i]);
      if (I < kVInstr) lds_dma16(rv, (st ? sV1 : sV0) + I * 512, voff[i]);
    }
  };
  // transpose-read addressing for the A operand V^T: lane j of each 16-lane
  // group points at row j/4 of a 4-row block, columns 4*(j%4)..+3
  const int grp = lane >> 4, gl = lane & 15;
  const int vrd = (4 * (grp >> 1) + (gl >> 2)) * kVStr + (grp & 1) * 16 + 4 * (gl & 3);
  const int krd = n * kKStr + g * 8;

  // one tile in LDS stage `stage`: S^T, SiLU (+ mask), O^T += V^T Y^T
  auto compute = [&](int c0, auto masked, auto stage) {
    constexpr bool kMasked = decltype(masked)::value;
    const uint16_t* kbase = (decltype(stage)::value ? sK1 : sK0) + krd;
    const uint16_t* vbase = (decltype(stage)::value ? sV1 : sV0) + vrd;
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbase + kb * 32 * kKStr + ks * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t mg = 0;
      if constexpr (kMasked) mg = col_mask32(lo, hi, ni, c0 + kb * 32) >> (g * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = sacc[kb][r];
        float y = x * logistic_scaled(x, c_exp);
        if constexpr (kMasked) y = keep_bits(y, bit_keep_imm(mg, (r >> 2) * 8 + (r & 3)));
        pf[kb * 2 + (r >> 3)][r & 7] = (__bf16)y;
      }
    }
    // A = V^T: lane (d = mb*32 + n, half g) takes key rows 16ss + 4g + {0..3}
    // and 16ss + 8 + 4g + {0..3}, the same order the Y^T operand uses.
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
#pragma unroll
      for (int mb = 0; mb < kD / 32; ++mb) {
        const uint16_t* vp = vbase + (16 * ss) * kVStr + mb * 32;
        const bf16x4 lo4 = lds_read_tr(vp);
        const bf16x4 hi4 = lds_read_tr(vp + 8 * kVStr);
        const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ss], oacc[mb], 0, 0, 0);
      }
    }
  };

  // walk a list of tiles, two LDS stages: the next tile's DMA runs while
  // this tile is computed; the barrier before each tile both publishes its
  // DMA (the barrier waits for outstanding memory operations) and retires the
  // stage the new DMA overwrites
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto walk = [&](const int* list, int cnt, auto masked) {
    if (cnt == 0) return;
    dma_tile(list[0], S0{});
    for (int i = 0; i < cnt; i += 2) {
      dma_barrier();
      if (i + 1 < cnt) dma_tile(list[i + 1], S1{});
      compute(list[i] * kBN, masked, S0{});
      if (i + 1 >= cnt) break;
      dma_barrier();
      if (i + 2 < cnt) dma_tile(list[i + 2], S0{});
      compute(list[i + 1] * kBN, masked, S1{});
    }
    __syncthreads();
  };

  for (int w0 = t_begin; w0 < t_end; w0 += kListWin) {
    if (wave == 0) {
      int np, nf;
      tile_window(sEnv, ni, kBN, L, w0, t_end, sPart, sFull, np, nf);
      if (lane == 0) {
        sCount[0] = np;
        sCount[1] = nf;
      }
    }
    __syncthreads();
    const int n_part = sCount[0], n_full = sCount[1];
    walk(sPart, n_part, std::true_type{});
    walk(sFull, n_full, std::false_type{});
    // the next window rewrites the lists and counts: every wave is done with them
    __syncthreads();
  }

  // epilogue: lane holds O[row][mb*32 + j*8 + g*4 + 0..3]
  if (row_ok) {
    uint16_t* op = o + (s + row) * rs + (int64_t)h * kD + g * 4;
#pragma unroll
    for (int mb = 0; mb < kD / 32; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = (__bf16)(oacc[mb][j * 4 + i] * out_scale);
        *reinterpret_cast<bf16x4*>(op + mb * 32 + j * 8) = w4;
      }
    }
  }
}

}  // namespace

hipError_t launch_mfma_fwd(const void* q, const void* k, const void* v, void* o, const Prep& P,
                           const Units& U, int H, const int32_t* func, int nfunc, float alpha,
                           float inv_max_len, hipStream_t stream) {
  if (U.cap == 0) return hipSuccess;
  ProfScope ps(stream, "k_fwd_bf16");
  hipLaunchKernelGGL(k_fwd_bf16, dim3(U.cap), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), P, U.list, H,
                     func, nfunc, alpha, alpha * inv_max_len);
  return hipGetLastError();
}

}  // namespace hstu
