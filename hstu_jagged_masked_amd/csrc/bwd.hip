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
//             [32w, 32w+32) and keeps their K and V rows in registers; wave 0
//             lists, with a ballot, the 64-row row blocks whose envelopes
//             reach these keys (partly seen blocks and wholly seen blocks in
//             separate lists); each block is one step (one LDS stage, one
//             barrier), computed as two halves of 32 query rows:
//               S = Q K^T, dS = dO V^T          (A from LDS, B = K, V registers)
//               y, p in registers (mask via per-row bitmasks in LDS, from
//               the func columns of the block's rows, which a partly seen
//               block's copy brings into LDS with its Q and dO tiles)
//               dV^T += dO^T Y,  dK^T += Q^T P  (A = transpose reads of the
//                                                row-major Q / dO tiles)
//   k_bwd_q   one workgroup per (sequence, head, 128 query rows), the forward's
//             walk over key tiles:
//               S^T = K Q^T, dS^T = V dO^T      (B = Q, dO registers)
//               p in registers
//               dQ^T += K^T P^T                 (A = transpose reads of K)
// Both stage their tiles in LDS with asynchronous buffer-to-LDS DMA into two
// stages: the next step's copy runs during this step's math, and the one
// barrier per step both publishes the copy and retires the other stage.
//
// The atomic-dQ variant (k_bwd_kv<false, true>) replaces k_bwd_q: after each
// half the four waves exchange their bf16 P through LDS, wave w forms
// dQ[32 rows][dims 32w..32w+31] = P[32 rows][128 keys] K[128 keys][those dims]
// with K from registers, and adds it to an fp32 accumulator with global
// atomics (in no fixed order: dq is not bitwise repeatable).
#include <type_traits>

#include "atomic_dq.h"
#include "common.h"
#include "pstore.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
using S0 = std::integral_constant<int, 0>;
using S1 = std::integral_constant<int, 1>;

// k_bwd_kv
constexpr int kKvBN = 128;                    // key rows per workgroup
constexpr int kKvBM = 32;                     // query rows per step (half a row block)
constexpr int kStepRows = 2 * kKvBM;          // query rows per step (one row block)
constexpr int kQStage = kStepRows * kD;       // bf16 elements per swizzled stage (16 KiB)
constexpr int kQInstr = kQStage / 512;        // 16 wave DMA instructions per tile
constexpr int kStepWin = kListWin;            // steps per list window (one per row block)

// k_bwd_q
constexpr int kQBM = 128;                     // query rows per workgroup
constexpr int kQBN = 64;                      // key columns per tile
constexpr int kKStage = kQBN * kD;            // bf16 elements per swizzled stage (16 KiB)
constexpr int kKInstr = kKStage / 512;        // 16 wave DMA instructions per tile

__device__ __forceinline__ bf16x8 concat4(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Wave-level: for the row blocks [w0, min(w0 + 64, nrb)) of a sequence of
// length L, lists the blocks (their first local row) that reach key columns
// [c0, c1): partly seen blocks into part, wholly seen ones into full; returns
// the counts in every lane.
__device__ __forceinline__ void step_window(const int4* env, int ni, int L, int nrb, int w0,
                                            int c0, int c1, int* part, int* full_list,
                                            int& n_part, int& n_full) {
  const int lane = threadIdx.x & 63;
  const int rb = w0 + lane;
  bool live = false, full = false;
  if (rb < nrb) block_vs_cols(env + (int64_t)rb * ni, ni, c0, c1, live, full);
  full = full && live;
  const bool partial = live && !full;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t mp = __ballot(partial), mf = __ballot(full);
  if (partial) part[__popcll(mp & below)] = rb * kRB;
  if (full) full_list[__popcll(mf & below)] = rb * kRB;
  n_part = __popcll(mp);
  n_full = __popcll(mf);
}

// kStoreP: also store each half's P (bf16, as rounded for the dK product)
// for the dQ pass, in the block layout of pstore.h (one 8 KiB block per
// (128-key tile, 32-row half)), through a buffer resource over this key
// tile's blocks clipped to the caller's buffer.  A block holds the
// registers pb[hh] of the four waves as they are: [wave w][hh][lane (n, g)][8
// bf16], i.e. key 32 w + n at row positions hh*16 + g*8 + 0..7, where row
// position hh*16 + g*8 + e is query row (2 hh + e/4)*8 + g*4 + e%4 of the
// half.  The dQ pass transposes it.  Each half's stores go out as soon as its
// P is formed (holding the second half's until after the next barrier
// measured the same).  Only the halves a key tile walks are written; the dQ
// pass reads exactly those.
//
// kAtomicDQ: also add each half's dQ contribution to dq_acc (fp32 [total, H,
// D]) with atomics, as described at the top.  The exchange buffers and the
// K operands of the dQ product do not fit beside two workgroups per CU, so
// this instantiation runs one workgroup (one wave per SIMD) per CU.
template <bool kStoreP, bool kAtomicDQ>
__global__ __launch_bounds__(kThreads, kAtomicDQ ? 1 : 2) void k_bwd_kv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, Prep P, const int4* __restrict__ units, int H,
    const int32_t* __restrict__ func, int nfunc, float alpha, float out_scale,
    uint16_t* __restrict__ pstore, uint64_t pstore_cap, float* __restrict__ dq_acc) {
  // two LDS stages as separate objects, so the compiler sees that the DMA
  // filling one stage does not alias the reads of the other
  __shared__ __attribute__((aligned(256))) uint16_t sQ0[kQStage], sQ1[kQStage];
  __shared__ __attribute__((aligned(256))) uint16_t sG0[kQStage], sG1[kQStage];  // dO
  __shared__ __attribute__((aligned(16))) uint32_t sMask[4][kStepRows];
  // func columns of the step's rows (masked walks), copied with its tiles
  __shared__ __attribute__((aligned(16))) int32_t sF0[kMaxNfunc][kStepRows],
      sF1[kMaxNfunc][kStepRows];
  __shared__ int sPart[kStepWin], sFull[kStepWin];
  __shared__ int sCount[2];
  // atomic dQ: per half, the four waves' P registers (2 KiB each)
  __shared__ __attribute__((aligned(16))) uint16_t sX[kAtomicDQ ? kXchgBytes / 2 : 8];

  UnitRec u;
  if (!unit_of_block(units, u)) return;
  const int kt = u.tile, h = u.h, L = u.L;
  const int64_t s = u.s;
  const int c0 = kt * kKvBN;
  const int c1 = min(c0 + kKvBN, L);
  const int tid = threadIdx.x;
  // the wave index in a scalar register: the copies' LDS addresses derive
  // from it and stay scalar
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;
  const int rs2 = H * kD * 2;
  const float c_exp = -alpha * kLog2e;

  // the first window's step lists before the K / V row loads, so that they
  // (and the first copy) do not wait behind them
  const int nrb = (L + kRB - 1) / kRB;
  const int4* env = P.env + (int64_t)u.rb * ni;
  auto list_window = [&](int w0) {
    if (wave == 0) {
      int np, nf;
      step_window(env, ni, L, nrb, w0, c0, c1, sPart, sFull, np, nf);
      if (lane == 0) {
        sCount[0] = np;
        sCount[1] = nf;
      }
    }
  };
  list_window(0);
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
  // atomic dQ: B operands of dQ[rows][dims] += P K, this wave's 32 dims
  // (32 wave + n) and the tile's 128 keys: lane (n, g) holds keys
  // 16 ks + 8 g + 0..7 (zero past the sequence end)
  bf16x8 kq[kAtomicDQ ? kKvBN / 16 : 1];
  if constexpr (kAtomicDQ) {
    const uint16_t* kd = k + s * rs + (int64_t)h * kD + wave * 32 + n;
#pragma unroll
    for (int ks = 0; ks < kKvBN / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = c0 + xchg_k_key(ks, g, e);
        const uint16_t bits = key < L ? kd[(int64_t)key * rs] : (uint16_t)0;
        kq[ks][e] = __builtin_bit_cast(__bf16, bits);
      }
    }
  }
  f32x16 dkacc[kD / 32], dvacc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }

  const uint16_t* qh = q + s * rs + (int64_t)h * kD;
  const uint16_t* gh = dout + s * rs + (int64_t)h * kD;
  // stored P: this workgroup's key tile's blocks, as a buffer resource
  // clipped to the caller's buffer (stores past it are dropped)
  const PRegion pr = kStoreP ? pstore_tile_region(u.pblk, H, h, L, kt, pstore_cap) : PRegion{0, 0};
  const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<char*>(pstore) + pr.base, (short)0, (int)pr.bytes, 0x00020000);
  // written once and read back by the dQ pass long after it has left L2:
  // non-temporal stores keep the Q / dO tiles cached instead
  auto p_store = [&](int r, const bf16x8* pv) {
    const int t = r / kKvBM;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const auto w = __builtin_bit_cast(
          __attribute__((ext_vector_type(4))) unsigned int, pv[hf]);
      __builtin_amdgcn_raw_buffer_store_b128(w, p_rsrc, (int)pstore_offset(t, 2 * wave + hf, lane),
                                             0, kCacheNT);
    }
  };
  // DMA of one 64-row step: wave w issues instructions I = w + 4i of each
  // tensor; lane l of instruction I fills LDS slot 64*I + l
  constexpr int kDmaPerWave = kQInstr / 4;
  int doff[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) doff[i] = swz_dma_offset((wave + 4 * i) * 64 + lane, rs2);
  auto dma_step = [&](int q0, auto stage, auto with_func) {
    constexpr int st = decltype(stage)::value;
    const int rows = min(kStepRows, L - q0);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(qh + (int64_t)q0 * rs, rows, rs2, kD * 2);
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(gh + (int64_t)q0 * rs, rows, rs2, kD * 2);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int I = wave + 4 * i;
      lds_dma16(rq, (st ? sQ1 : sQ0) + I * 512, doff[i]);
      lds_dma16(rg, (st ? sG1 : sG0) + I * 512, doff[i]);
    }
    if constexpr (decltype(with_func)::value) {
      // func column c of rows q0 + lane, 4 bytes per lane, through a
      // resource over the step's rows (rows past the sequence read 0); wave
      // w copies columns w, w + 4, w + 8
#pragma unroll
      for (int i = 0; i < (kMaxNfunc + 3) / 4; ++i) {
        const int c = wave + 4 * i;
        if (c < nfunc) {
          const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<int32_t*>(func + (int64_t)c * P.total + s + q0), (short)0, rows * 4,
              0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rf, (__attribute__((address_space(3))) void*)(st ? sF1[c] : sF0[c]), 4, lane * 4, 0,
              0, 0);
        }
      }
    }
  };

  // Byte offsets into a swizzled tile.  Row reads: lane (n, g) reads row n
  // (+ 32 kb), chunk 2 ks + g, at rd_b ^ 32 ks.  Transpose reads: lane j of
  // 16-lane group G reads row 4*(G/2) + j/4 (+ 16 per slab), column
  // (G%2)*16 + 4*(j%4) + 32 mb at tr_b ^ 64 mb, and the same rows + 8 at
  // tr_b ^ 64 mb ^ 32 + 2 KiB.  The XORs are applied at each read so only two
  // offsets stay live.
  const int grp = lane >> 4, gl = lane & 15;
  const int trow = 4 * (grp >> 1) + (gl >> 2);
  const int rd_b0 = n * 256 + ((g ^ swz(n)) << 4);
  const int tr_b0 = trow * 256 + 8 * (gl & 1) +
                    ((((grp & 1) * 2 + ((gl & 3) >> 1)) ^ swz(trow)) << 4);

  // Atomic dQ of one half (query rows from r0h), in the exchange layout of
  // atomic_dq.h.  The two halves use separate buffers; the barrier before
  // each step retires a buffer before the next step rewrites it.
  auto dq_atomic = [&](int r0h, int hf, const bf16x8* pv) {
    const int xw0 = xchg_write_offset(wave, n, g, 0), xw1 = xchg_write_offset(wave, n, g, 1);
    const int xr0 = xchg_read_offset(lane, 0, 0), xr1 = xchg_read_offset(lane, 0, 1);
    char* xb = reinterpret_cast<char*>(sX) + hf * kXchgHalfBytes;
    *reinterpret_cast<bf16x8*>(xb + xw0) = pv[0];
    *reinterpret_cast<bf16x8*>(xb + xw1) = pv[1];
    lds_barrier();
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kKvBN / 16; ++ks) {
      // xchg_read_offset(lane, ks, s) = xchg_read_offset(lane, 0, s) + this
      const uint16_t* rb = reinterpret_cast<const uint16_t*>(
          xb + (ks >> 1) * kXchgWaveBytes + (ks & 1) * 1024);
      const bf16x8 pt = concat4(lds_tr8(rb, xr0), lds_tr8(rb, xr1));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pt, kq[ks], acc, 0, 0, 0);
    }
    // element i of lane (n, g): dim 32 wave + n of query row r0h + xchg_acc_row(i, g)
    float* dst = dq_acc + s * rs + (int64_t)h * kD + wave * 32 + n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r0h + xchg_acc_row(i, g);
      if (row < L) unsafeAtomicAdd(dst + (int64_t)row * rs, acc[i]);
    }
  };

  // one 64-row step (two halves of 32 rows) from LDS stage `stage`; `next`
  // (>= 0) is the next step's first row, whose DMA is issued after this
  // step's func loads
  auto step = [&](int q0, int next, auto masked, auto stage) {
    constexpr bool kMasked = decltype(masked)::value;
    constexpr int st = decltype(stage)::value;
    const int nh = q0 + kKvBM < L ? 2 : 1;  // halves of 32 rows in this step
    if constexpr (kMasked) {
      // row q0 + 32 g + n (lane (n, g) takes one row of half g): visibility of
      // this wave's 32 key columns (wave-private LDS), from the func columns
      // copied with this step's tiles
      const int rr = g * kKvBM + n, r = q0 + rr;
      const int32_t(*sf)[kStepRows] = st ? sF1 : sF0;
      int lo[kMaxNI], hi[kMaxNI];
#pragma unroll
      for (int j = 0; j < kMaxNI; ++j) {
        lo[j] = L;
        hi[j] = 0;
        if (j < ni) {
          const int a = j > 0 ? max(sf[2 * j - 1][rr], 0) : 0;
          const int b = min(sf[2 * j][rr], L);
          if (b > a && r < L) {
            lo[j] = a;
            hi[j] = b;
          }
        }
      }
      sMask[wave][rr] = col_mask32(lo, hi, ni, c0 + wave * 32);
    }
    if (next >= 0) {
      if constexpr (st == 0) {
        dma_step(next, S1{}, masked);
      } else {
        dma_step(next, S0{}, masked);
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (hf >= nh) break;
      const uint16_t* sQ = (st ? sQ1 : sQ0) + hf * kKvBM * kD;
      const uint16_t* sG = (st ? sG1 : sG0) + hf * kKvBM * kD;
      const int rd_b = opaque(rd_b0), tr_b = opaque(tr_b0);
      f32x16 sacc = f32x16{}, dsacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const int off = rd_b ^ (32 * ks);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row16(sQ, off), kf[ks], sacc, 0, 0, 0);
        dsacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row16(sG, off), vf[ks], dsacc, 0, 0, 0);
      }
      // element r: query row (r/4)*8 + g*4 + r%4 of the half, key column `col`
      bf16x8 yb[2], pb[2];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint4 m4 = make_uint4(0, 0, 0, 0);
        if constexpr (kMasked)
          m4 = *reinterpret_cast<const uint4*>(&sMask[wave][hf * kKvBM + jj * 8 + g * 4]);
        const uint32_t mrow[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = jj * 4 + i;
          const float x = sacc[r];
          const float sg = logistic_scaled(x, c_exp);
          float y = x * sg;
          // silu'(alpha x) = sg + alpha * x sg (1 - sg) = sg + alpha * (y - y sg)
          float p = dsacc[r] * fmaf(alpha, fmaf(-y, sg, y), sg);
          if constexpr (kMasked) {
            const uint32_t keep = bit_keep(mrow[i], n);
            y = keep_bits(y, keep);
            p = keep_bits(p, keep);
          }
          yb[r >> 3][r & 7] = (__bf16)y;
          pb[r >> 3][r & 7] = (__bf16)p;
        }
      }
      if constexpr (kStoreP) p_store(q0 + hf * kKvBM, pb);
      if constexpr (kAtomicDQ) dq_atomic(q0 + hf * kKvBM, hf, pb);
      // dV^T += dO^T Y and dK^T += Q^T P: A operands by transpose reads, query
      // rows 16hh + 4g + {0..3} and 16hh + 8 + 4g + {0..3}; the operands of
      // step o + 1 (o = 4 hh + mb) are read before the products of step o so
      // that the LDS latency is not waited for right before each product
      auto ld = [&](int o, bf16x8& ag, bf16x8& aq) {
        const int hh = o >> 2, mb = o & 3;
        const int o0 = (tr_b ^ (64 * mb)) + 16 * hh * 256;
        const int o1 = (tr_b ^ (64 * mb) ^ 32) + (16 * hh + 8) * 256;
        ag = concat4(lds_tr8(sG, o0), lds_tr8(sG, o1));
        aq = concat4(lds_tr8(sQ, o0), lds_tr8(sQ, o1));
      };
      bf16x8 ag0, aq0, ag1, aq1;
      ld(0, ag0, aq0);
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        const int hh = o >> 2, mb = o & 3;
        if (o + 1 < 8) {
          if (o & 1)
            ld(o + 1, ag0, aq0);
          else
            ld(o + 1, ag1, aq1);
        }
        const bf16x8 ag = (o & 1) ? ag1 : ag0, aq = (o & 1) ? aq1 : aq0;
        dvacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, yb[hh], dvacc[mb], 0, 0, 0);
        dkacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, pb[hh], dkacc[mb], 0, 0, 0);
      }
    }
  };

  auto walk = [&](const int* list, int cnt, auto masked) {
    if (cnt == 0) return;
    dma_step(list[0], S0{}, masked);
    for (int i = 0; i < cnt; i += 2) {
      dma_barrier();
      step(list[i], i + 1 < cnt ? list[i + 1] : -1, masked, S0{});
      if (i + 1 >= cnt) break;
      dma_barrier();
      step(list[i + 1], i + 2 < cnt ? list[i + 2] : -1, masked, S1{});
    }
    __syncthreads();
  };

  for (int w0 = 0; w0 < nrb; w0 += kListWin) {
    if (w0 > 0) list_window(w0);
    __syncthreads();
    const int n_part = sCount[0], n_full = sCount[1];
    walk(sPart, n_part, std::true_type{});
    walk(sFull, n_full, std::false_type{});
    // the next window rewrites the lists and counts: every wave is done with them
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

__global__ __launch_bounds__(kThreads, 2) void k_bwd_q(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq,
    Prep P, const int4* __restrict__ units, int H, const int32_t* __restrict__ func, int nfunc,
    float alpha, float out_scale) {
  __shared__ __attribute__((aligned(256))) uint16_t sK0[kKStage], sK1[kKStage];
  __shared__ __attribute__((aligned(256))) uint16_t sV0[kKStage], sV1[kKStage];
  __shared__ int sPart[kListWin], sFull[kListWin];
  __shared__ int sCount[2];
  __shared__ Envelope sEnv;

  UnitRec u;
  if (!unit_of_block(units, u)) return;
  const int qt = u.tile, h = u.h, L = u.L;
  const int64_t s = u.s;
  const int r0 = qt * kQBM;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;
  const int rs2 = H * kD * 2;
  const float c_exp = -alpha * kLog2e;

  // the block's envelope first, so that the tile list does not wait behind
  // the q, dO and func loads
  if (tid == 0) rows_envelope(P, u.rb, r0, kQBM, L, ni, sEnv);
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
  __syncthreads();
  int t_begin, t_end;
  envelope_tile_span(sEnv, ni, kQBN, t_begin, t_end);

  f32x16 dqacc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) dqacc[mb] = f32x16{};

  const uint16_t* kh = k + s * rs + (int64_t)h * kD;
  const uint16_t* vh = v + s * rs + (int64_t)h * kD;
  constexpr int kDmaPerWave = kKInstr / 4;
  int doff[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) doff[i] = swz_dma_offset((wave + 4 * i) * 64 + lane, rs2);
  auto dma_tile = [&](int t, auto stage) {
    constexpr int st = decltype(stage)::value;
    const int c0 = t * kQBN;
    const int rows = min(kQBN, L - c0);
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kh + (int64_t)c0 * rs, rows, rs2, kD * 2);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vh + (int64_t)c0 * rs, rows, rs2, kD * 2);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int I = wave + 4 * i;
      lds_dma16(rk, (st ? sK1 : sK0) + I * 512, doff[i]);
      lds_dma16(rv, (st ? sV1 : sV0) + I * 512, doff[i]);
    }
  };

  // Byte offsets into a swizzled tile.  Row reads: lane (n, g) reads row n
  // (+ 32 kb), chunk 2 ks + g, at rd_b ^ 32 ks.  Transpose reads: lane j of
  // 16-lane group G reads row 4*(G/2) + j/4 (+ 16 per slab), column
  // (G%2)*16 + 4*(j%4) + 32 mb at tr_b ^ 64 mb, and the same rows + 8 at
  // tr_b ^ 64 mb ^ 32 + 2 KiB.  The XORs are applied at each read so only two
  // offsets stay live.
  const int grp = lane >> 4, gl = lane & 15;
  const int trow = 4 * (grp >> 1) + (gl >> 2);
  const int rd_b0 = n * 256 + ((g ^ swz(n)) << 4);
  const int tr_b0 = trow * 256 + 8 * (gl & 1) +
                    ((((grp & 1) * 2 + ((gl & 3) >> 1)) ^ swz(trow)) << 4);

  auto compute = [&](int c0, auto masked, auto stage) {
    constexpr bool kMasked = decltype(masked)::value;
    constexpr int st = decltype(stage)::value;
    const uint16_t* sK = st ? sK1 : sK0;
    const uint16_t* sV = st ? sV1 : sV0;
    const int rd_b = opaque(rd_b0), tr_b = opaque(tr_b0);
    f32x16 sacc[2], dsacc[2];
    // operands of (kb, ks) step o = 8 kb + ks read one step ahead
    auto ldr = [&](int o, bf16x8& a, bf16x8& b) {
      const int off = (rd_b ^ (32 * (o & 7))) + (o >> 3) * 32 * 256;
      a = lds_row16(sK, off);
      b = lds_row16(sV, off);
    };
    bf16x8 ra0, rb0, ra1, rb1;
    ldr(0, ra0, rb0);
#pragma unroll
    for (int o = 0; o < 16; ++o) {
      const int kb = o >> 3, ks = o & 7;
      if (ks == 0) {
        sacc[kb] = f32x16{};
        dsacc[kb] = f32x16{};
      }
      if (o + 1 < 16) {
        if (o & 1)
          ldr(o + 1, ra0, rb0);
        else
          ldr(o + 1, ra1, rb1);
      }
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((o & 1) ? ra1 : ra0, qf[ks], sacc[kb], 0,
                                                         0, 0);
      dsacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((o & 1) ? rb1 : rb0, gf[ks], dsacc[kb],
                                                          0, 0, 0);
    }
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t mg = 0;
      if constexpr (kMasked) mg = col_mask32(lo, hi, ni, c0 + kb * 32) >> (g * 4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = sacc[kb][r];
        const float sg = logistic_scaled(x, c_exp);
        // silu'(alpha x) = sg + alpha * x sg (1 - sg)
        const float y = x * sg;
        float p = dsacc[kb][r] * fmaf(alpha, fmaf(-y, sg, y), sg);
        if constexpr (kMasked) p = keep_bits(p, bit_keep_imm(mg, (r >> 2) * 8 + (r & 3)));
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    }
    auto ldk = [&](int o) {
      const int ss = o >> 2, mb = o & 3;
      const int o0 = (tr_b ^ (64 * mb)) + 16 * ss * 256;
      const int o1 = (tr_b ^ (64 * mb) ^ 32) + (16 * ss + 8) * 256;
      return concat4(lds_tr8(sK, o0), lds_tr8(sK, o1));
    };
    bf16x8 ka0 = ldk(0), ka1;
#pragma unroll
    for (int o = 0; o < 16; ++o) {
      if (o + 1 < 16) {
        if (o & 1)
          ka0 = ldk(o + 1);
        else
          ka1 = ldk(o + 1);
      }
      dqacc[o & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((o & 1) ? ka1 : ka0, pb[o >> 2],
                                                             dqacc[o & 3], 0, 0, 0);
    }
  };

  auto walk = [&](const int* list, int cnt, auto masked) {
    if (cnt == 0) return;
    dma_tile(list[0], S0{});
    for (int i = 0; i < cnt; i += 2) {
      dma_barrier();
      if (i + 1 < cnt) dma_tile(list[i + 1], S1{});
      compute(list[i] * kQBN, masked, S0{});
      if (i + 1 >= cnt) break;
      dma_barrier();
      if (i + 2 < cnt) dma_tile(list[i + 2], S0{});
      compute(list[i + 1] * kQBN, masked, S1{});
    }
    __syncthreads();
  };

  for (int w0 = t_begin; w0 < t_end; w0 += kListWin) {
    if (wave == 0) {
      int np, nf;
      tile_window(sEnv, ni, kQBN, L, w0, t_end, sPart, sFull, np, nf);
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
                           float inv_max_len, uint16_t* pstore, uint64_t pstore_cap,
                           hipStream_t stream) {
  const float scale = alpha * inv_max_len;
  if (Ukv.cap > 0) {
    ProfScope ps(stream, pstore ? "k_bwd_kv_p" : "k_bwd_kv");
    auto kern = pstore ? k_bwd_kv<true, false> : k_bwd_kv<false, false>;
    hipLaunchKernelGGL(kern, dim3(Ukv.cap), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), P, Ukv.list, H,
                       func, nfunc, alpha, scale, pstore, pstore_cap, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pstore) return launch_dq_from_p(k, dq, P, Uq, H, nfunc, pstore, pstore_cap, scale, stream);
  if (Uq.cap > 0) {
    ProfScope ps(stream, "k_bwd_q");
    hipLaunchKernelGGL(k_bwd_q, dim3(Uq.cap), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                       static_cast<uint16_t*>(dq), P, Uq.list, H, func, nfunc, alpha, scale);
  }
  return hipGetLastError();
}

namespace {

// fp32 accumulator of the atomic-dQ backward: cleared by a kernel (not a
// memset, so that the enqueued work can be captured in a graph) and turned
// into bf16 dq = acc * scale afterwards.  n4 = elements / 4 (D = 128, so a
// whole number).
__global__ __launch_bounds__(256) void k_fill_f32(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void k_dq_convert(const float4* __restrict__ acc,
                                                    uint16_t* __restrict__ dq, int64_t n4,
                                                    float scale) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    const float4 a = acc[i];
    bf16x4 w;
    w[0] = (__bf16)(a.x * scale);
    w[1] = (__bf16)(a.y * scale);
    w[2] = (__bf16)(a.z * scale);
    w[3] = (__bf16)(a.w * scale);
    *reinterpret_cast<bf16x4*>(dq + 4 * i) = w;
  }
}

}  // namespace

hipError_t launch_mfma_bwd_atomic(const void* q, const void* k, const void* v, const void* dout,
                                  void* dq, void* dk, void* dv, const Prep& P, const Units& Ukv,
                                  int H, const int32_t* func, int nfunc, float alpha,
                                  float inv_max_len, float* dq_acc, int64_t total,
                                  hipStream_t stream) {
  const float scale = alpha * inv_max_len;
  const int64_t n4 = total * H * kD / 4;
  const int grid = (int)std::min<int64_t>(std::max<int64_t>((n4 + 255) / 256, 1), 8192);
  if (n4 > 0) {
    ProfScope ps(stream, "k_fill_f32");
    hipLaunchKernelGGL(k_fill_f32, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<float4*>(dq_acc), n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (Ukv.cap > 0) {
    ProfScope ps(stream, "k_bwd_kv_atomic");
    hipLaunchKernelGGL((k_bwd_kv<false, true>), dim3(Ukv.cap), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), P, Ukv.list, H,
                       func, nfunc, alpha, scale, nullptr, (uint64_t)0, dq_acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n4 > 0) {
    ProfScope ps(stream, "k_dq_convert");
    hipLaunchKernelGGL(k_dq_convert, dim3(grid), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(dq_acc), static_cast<uint16_t*>(dq), n4,
                       scale);
  }
  return hipGetLastError();
}

}  // namespace hstu
