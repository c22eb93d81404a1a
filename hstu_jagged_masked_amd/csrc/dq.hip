// dQ from stored P, bf16 inputs, D = 128, bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
//   dQ_i = (alpha / max_len) * sum_j p_ij k_j,  p_ij = dS_ij silu'(alpha x_ij)
//
// with p as the key-owner backward kernel rounded it to bf16 for its dK product
// and stored it (masked pairs hold 0).  No S, dS or mask is recomputed here.
//
// One workgroup (4 waves) owns 128 query rows of one (sequence, head); wave w
// owns the 32 rows from r0 + 32w (one stored-P half).  The workgroup walks
// the 128-key tiles its row blocks reach.  Per tile:
//   * the K rows -> LDS (swizzled 256-byte rows) by buffer-to-LDS copies into
//     one of two stages, the next tile's copy in flight during this tile;
//   * each wave's stored P block (8 KiB, the key-owner kernel's registers as
//     they were: key-major, 8 row positions per 16 bytes) -> registers by
//     16-byte buffer loads (range-checked against the key tile's blocks and
//     the caller's buffer), two tiles ahead;
//   * P transposed through a wave-private LDS buffer, 32 keys at a time, into
//     the B operand of dQ^T += K^T P^T (row position per lane, 8 keys);
//   * dQ^T += K^T P^T on MFMA, A = K^T by LDS transpose reads.
// A wave whose row block the key tile does not reach has no P block for it
// and skips that tile.  The accumulator columns are P's row positions; the
// epilogue maps them back to query rows.
#include <type_traits>

#include "common.h"
#include "pstore.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kBM = 128;                     // query rows per workgroup
constexpr int kKT = 128;                     // keys per stored-P tile
constexpr int kStep = 32;                    // rows per stored-P step
constexpr int kKStage = kKT * kD;            // bf16 elements of K per stage (32 KiB)
constexpr int kKDma = kKStage / 512 / 4;     // K copy instructions per wave per stage
constexpr int kKSteps = kKT / 16;            // MFMA key steps per tile

using S0 = std::integral_constant<int, 0>;
using S1 = std::integral_constant<int, 1>;

__global__ __launch_bounds__(kThreads, 2) void k_bwd_dq(
    const uint16_t* __restrict__ k, uint16_t* __restrict__ dq, Prep P,
    const int4* __restrict__ units, int H, int nfunc, const uint16_t* __restrict__ pstore,
    uint64_t pstore_cap, float out_scale) {
  __shared__ __attribute__((aligned(256))) uint16_t sK0[kKStage], sK1[kKStage];
  // per wave: P of 32 keys as [key][32 row positions], 64-byte rows, 16-byte
  // chunk c of key row r at position c ^ ((r / 4) mod 4)
  __shared__ __attribute__((aligned(16))) uint16_t sPt[4 * 32 * 32];

  UnitRec u;
  if (!unit_of_block(units, u)) return;
  const int qt = u.tile, h = u.h, L = u.L;
  const int64_t s = u.s;
  const int r0 = qt * kBM;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int ni = (nfunc + 1) / 2;
  const int64_t rs = (int64_t)H * kD;
  const int rs2 = H * kD * 2;

  // this wave's step and the row block whose envelope decides its tiles
  const int q0 = r0 + wave * kStep;
  const bool wave_rows = q0 < L;

  // a stored-P buffer smaller than these lengths need held no complete P:
  // the rows get NaN, so that the failure cannot pass unseen
  if ((uint64_t)P.pblk[P.B] * (uint64_t)H * kPBlockBytes > pstore_cap) {
    const int row = r0 + wave * 32 + n;
    if (row < L) {
      uint16_t* op = dq + (s + row) * rs + (int64_t)h * kD + g * 64;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint4*>(op + j * 8) = make_uint4(0x7fc07fc0u, 0x7fc07fc0u,
                                                           0x7fc07fc0u, 0x7fc07fc0u);
    }
    return;
  }
  const int nrb = (L + kRB - 1) / kRB;
  const int4* env = P.env + (int64_t)u.rb * ni;
  const int rb_a = r0 / kRB, rb_b = rb_a + 1;  // the workgroup's two row blocks
  const bool has_b = rb_b < nrb;
  const bool in_b = wave >= 2;                 // waves 2, 3 own rows of the second
  auto block_live = [&](int rb, int c0, int c1) {
    bool live, full;
    block_vs_cols(env + (int64_t)rb * ni, ni, c0, c1, live, full);
    return live;
  };

  // every key tile of the sequence is a candidate: the window ballots below
  // pick the live ones (one round of envelope reads instead of two)
  const int kt_begin = 0, kt_end = (L + kKT - 1) / kKT;
  // Liveness of 64 key tiles at a time as ballot masks (bit j: tile w + j
  // reaches the first / second row block), so that the walk itself issues no
  // loads besides its copies and P loads.
  int win = -1;
  uint64_t live_a = 0, live_b = 0;
  auto window = [&](int w) {
    const int kt = w + lane;
    bool la = false, lb = false;
    if (kt < kt_end) {
      const int c0 = kt * kKT, c1 = min(c0 + kKT, L);
      la = block_live(rb_a, c0, c1);
      lb = has_b && block_live(rb_b, c0, c1);
    }
    live_a = __ballot(la);
    live_b = __ballot(lb);
    win = w;
  };
  // next key tile from kt on that some wave has P for (or -1); `mine`: this wave
  auto next_tile = [&](int kt, bool& mine) {
    while (kt < kt_end) {
      const int w = kt & ~63;
      if (w != win) window(w);
      const uint64_t rest = (live_a | live_b) >> (kt - w);
      if (rest) {
        kt += __builtin_ctzll(rest);
        mine = wave_rows && (((in_b ? live_b : live_a) >> (kt - w)) & 1);
        return kt;
      }
      kt = w + 64;
    }
    mine = false;
    return -1;
  };

  const uint16_t* kh = k + s * rs + (int64_t)h * kD;

  int kdoff[kKDma];
#pragma unroll
  for (int i = 0; i < kKDma; ++i) kdoff[i] = swz_dma_offset((wave + 4 * i) * 64 + lane, rs2);
  auto dma_k = [&](int kt, auto stage) {
    constexpr int st = decltype(stage)::value;
    const int c0 = kt * kKT;
    const __amdgpu_buffer_rsrc_t rk =
        rows_rsrc(kh + (int64_t)c0 * rs, min(kKT, L - c0), rs2, kD * 2);
#pragma unroll
    for (int i = 0; i < kKDma; ++i)
      lds_dma16_raw(rk, (st ? sK1 : sK0) + (wave + 4 * i) * 512, kdoff[i]);
  };
  // P is read exactly once: non-temporal loads, so that it does not push the
  // K tiles (re-read by every query block of the sequence) out of L2.  The
  // loads go through a resource over key tile kt's blocks (clipped to the
  // caller's buffer): a wave whose step lies past the sequence end reads
  // zeros there instead of another tile's blocks or memory past the buffer.
  auto load_p = [&](int kt, bf16x8* dst) {
    const PRegion pr = pstore_tile_region(u.pblk, H, h, L, kt, pstore_cap);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(pstore)) + pr.base, (short)0,
        (int)pr.bytes, 0x00020000);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(
          rp, (int)pstore_offset(q0 / kStep, ks, lane), 0, kCacheNT);
      dst[ks] = __builtin_bit_cast(bf16x8, w);
    }
  };

  // K^T transpose reads: lane j of 16-lane group G takes key rows 8*(G/2) + j/4
  // (+ 16 ks; + 4 for the second read) and d = 32 mb + (G%2)*16 + 4*(j%4), so
  // lane l holds keys 16 ks + 8 (l/32) + 0..7, the order of the stored P^T
  const int grp = lane >> 4, gl = lane & 15;
  const int trow = 8 * (grp >> 1) + (gl >> 2);
  const int tr_b0 = trow * 256 + 8 * (gl & 1) +
                    ((((grp & 1) * 2 + ((gl & 3) >> 1)) ^ swz(trow)) << 4);

  // P transpose.  Register j of a P block, lane (n, g), holds key 32 (j/2) + n
  // at row positions (2 (j%2) + g) * 8 + 0..7: written to row n, chunk
  // 2 (j%2) + g of the buffer.  Read back like K^T: lane j of 16-lane group G
  // reads key rows 8*(G/2) + j/4 (+ 16 ksl; + 4 for the second read), row
  // positions (G%2)*16 + 4*(j%4), so lane l holds keys 16 ks + 8 (l/32) + 0..7
  // of row position l%32.  (Rows + 4 flip the chunk swizzle's low bit.)
  char* const pbuf = reinterpret_cast<char*>(sPt + wave * 1024);
  const int pw_b0 = n * 64 + ((g ^ ((n >> 2) & 3)) << 4);
  const int pr_b0 = (8 * (grp >> 1) + (gl >> 2)) * 64 +
                    ((((grp & 1) * 2 + ((gl & 3) >> 1)) ^ (2 * (grp >> 1))) << 4) +
                    (gl & 1) * 8;
  auto p_tr = [&](int off) {
    return lds_read_tr(reinterpret_cast<const uint16_t*>(pbuf + off));
  };

  f32x16 acc[kD / 32];
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) acc[mb] = f32x16{};

  auto compute = [&](const bf16x8* pj, auto stage) {
    constexpr int st = decltype(stage)::value;
    const uint16_t* sK = st ? sK1 : sK0;
    const int tr_b = opaque(tr_b0);
    const int pw_b = opaque(pw_b0), pr_b = opaque(pr_b0);
    bf16x8 pt[kKSteps];
#pragma unroll
    for (int r = 0; r < kKT / 32; ++r) {
      // (one wave's LDS operations run in order: this round's writes follow
      // the previous round's reads)
      *reinterpret_cast<bf16x8*>(pbuf + pw_b) = pj[2 * r];
      *reinterpret_cast<bf16x8*>(pbuf + (pw_b ^ 32)) = pj[2 * r + 1];
#pragma unroll
      for (int ksl = 0; ksl < 2; ++ksl)
        pt[2 * r + ksl] = __builtin_shufflevector(p_tr(pr_b + ksl * 1024),
                                                  p_tr((pr_b ^ 16) + 256 + ksl * 1024), 0, 1,
                                                  2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int mb = 0; mb < kD / 32; ++mb) {
        // rows + 4: swz(r + 4) = swz(r) ^ 1 for these rows (r / 4 even)
        const int o0 = (tr_b ^ (64 * mb)) + 16 * ks * 256;
        const int o1 = (tr_b ^ (64 * mb) ^ 16) + (16 * ks + 4) * 256;
        const bf16x8 a = __builtin_shufflevector(lds_tr8(sK, o0), lds_tr8(sK, o1), 0, 1, 2, 3, 4,
                                                 5, 6, 7);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pt[ks], acc[mb], 0, 0, 0);
      }
    }
  };

  // walk: K in two LDS stages one tile ahead, P in three register sets two
  // tiles ahead (P comes from HBM).  P of every tile the workgroup visits is
  // loaded by every wave (a wave without a block there loads bytes it then
  // ignores), so each tile issues the same number of operations: at tile i
  // K(i+1) then P(i+2), and at the top of tile i only P(i+1)'s loads, issued
  // after K(i), may still be in flight (vector-memory loads complete in issue
  // order).
  bf16x8 p0[kKSteps], p1[kKSteps], p2[kKSteps];
  bool m0 = false, m1 = false, m2 = false;
  int t0 = next_tile(kt_begin, m0);
  int t1 = t0 >= 0 ? next_tile(t0 + 1, m1) : -1;
  if (t0 >= 0) {
    load_p(t0, p0);
    dma_k(t0, S0{});
    if (t1 >= 0) load_p(t1, p1);
  }
  // one tile: compute tile t (K stage st, P set pc) and prefetch
  auto tile = [&](int t, bool m, int tn, int& tnn, bool& mnn, const bf16x8* pc, bf16x8* pnn,
                  auto stage, auto nstage) {
    if (tn >= 0) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kKSteps) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();
    tnn = tn >= 0 ? next_tile(tn + 1, mnn) : -1;
    if (tn >= 0) dma_k(tn, nstage);
    if (tnn >= 0) load_p(tnn, pnn);
    if (m) compute(pc, stage);
  };
  // the stage of tile i is i % 2 and its P set i % 3: six tiles per round
  while (t0 >= 0) {
    int t2;
    bool mm2;
    tile(t0, m0, t1, t2, mm2, p0, p2, S0{}, S1{});
    if (t1 < 0) break;
    int t3;
    bool mm3;
    tile(t1, m1, t2, t3, mm3, p1, p0, S1{}, S0{});
    if (t2 < 0) break;
    int t4;
    bool mm4;
    tile(t2, mm2, t3, t4, mm4, p2, p1, S0{}, S1{});
    if (t3 < 0) break;
    int t5;
    bool mm5;
    tile(t3, mm3, t4, t5, mm5, p0, p2, S1{}, S0{});
    if (t4 < 0) break;
    int t6;
    bool mm6;
    tile(t4, mm4, t5, t6, mm6, p1, p0, S0{}, S1{});
    if (t5 < 0) break;
    int t7;
    bool mm7;
    tile(t5, mm5, t6, t7, mm7, p2, p1, S1{}, S0{});
    t0 = t6;
    m0 = mm6;
    t1 = t7;
    m1 = mm7;
  }

  // epilogue: column n is row position n = hh*16 + g'*8 + e of the step,
  // query row (2 hh + e/4)*8 + g'*4 + e%4; lane holds d = mb*32 + j*8 + g*4 + 0..3
  const int hh = n >> 4, gp = (n >> 3) & 1, e = n & 7;
  const int row = q0 + (2 * hh + (e >> 2)) * 8 + gp * 4 + (e & 3);
  if (wave_rows && row < L) {
    uint16_t* op = dq + (s + row) * rs + (int64_t)h * kD + g * 4;
#pragma unroll
    for (int mb = 0; mb < kD / 32; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 w4;
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = (__bf16)(acc[mb][j * 4 + i] * out_scale);
        *reinterpret_cast<bf16x4*>(op + mb * 32 + j * 8) = w4;
      }
    }
  }
}

}  // namespace

hipError_t launch_dq_from_p(const void* k, void* dq, const Prep& P, const Units& Uq, int H,
                            int nfunc, const uint16_t* pstore, uint64_t pstore_cap,
                            float out_scale, hipStream_t stream) {
  if (Uq.cap == 0) return hipSuccess;
  ProfScope ps(stream, "k_bwd_dq");
  hipLaunchKernelGGL(k_bwd_dq, dim3(Uq.cap), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<uint16_t*>(dq), P, Uq.list, H,
                     nfunc, pstore, pstore_cap, out_scale);
  return hipGetLastError();
}

}  // namespace hstu
