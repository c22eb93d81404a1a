/*
 * hstu_attn.h -- C ABI of the MI355X (gfx950) HSTU jagged masked attention
 * library (libhstu_attn.so).
 *
 * The operator.  Sequences are stored jagged: sequence b owns the global rows
 * [seq_offsets[b], seq_offsets[b+1]) of every [rows, H, D] tensor, and all row
 * and column indices below are local to their sequence.  Each query row i
 * carries a column mask given by `func`, the int32 interval encoding of
 * TorchEasyRec PR #670 ("move the HSTU arbitrary-mask path to NFUNC=5",
 * sections "Why" and "What changed"):
 *     interval 0 = [0, f0),  interval j = [f(2j-1), f(2j))  for j = 1..(nfunc-1)/2,
 * a pair whose end is <= its start is empty and skipped, and the visible set
 * V_i is the union of the intervals clipped to [0, L_b).  Any int32 value is
 * legal (it is clipped); func is shared by all heads (the review reply on that
 * PR shows the head dimension of func is never read), so it has no head axis.
 * For a visible pair (i, j) of head h:
 *     P_ij = alpha * <q_i, k_j>,   S_ij = silu(P_ij) / max_len,
 *     O_i  = sum_{j in V_i} S_ij v_j,
 * and the backward, with silu'(x) = s(x)(1 + x(1 - s(x))), s the logistic:
 *     dP_ij = <dO_i, v_j> silu'(P_ij) / max_len,
 *     dQ_i = alpha sum_j dP_ij k_j,  dK_j = alpha sum_i dP_ij q_i,
 *     dV_j = sum_i S_ij dO_i.
 * Rows with no visible column get O = dQ = 0; key rows no query sees get
 * dK = dV = 0 (always written).
 *
 * Targets-only mode (MLCommons training PR #903, "Summary" and "Gating"):
 * exactly one candidate row per sequence, i_b = target_rows[b], forms Q
 * against the full-length K and V.  Then q, o, dO and dq are compact [B, H, D]
 * (row b = candidate of sequence b) while k, v, dk, dv stay [total, H, D]; the
 * candidate's mask is func column seq_offsets[b] + i_b.  dK/dV rows that the
 * candidate does not see are written as 0.
 *
 * Layouts.  q, k, v, o, dout, dq, dk, dv: row-major [rows, H, D] (D fastest),
 * elements bf16 (HSTU_BF16) or fp32 (HSTU_FP32), 16-byte aligned.  func:
 * int32 [nfunc, total] row-major (column t = global row t).  seq_offsets:
 * int64 [B+1], seq_offsets[0] = 0, nondecreasing, seq_offsets[B] = total
 * (the "complete cumsum" of the lengths).  target_rows: int32 [B].  Every
 * pointer is a DEVICE pointer, except that `total_pairs` below is too.
 *
 * Supported: B >= 1, total >= 0, 1 <= H <= 255, D in {32, 64, 128},
 * 1 <= nfunc <= hstu_max_nfunc() and odd, max_len >= 1, alpha finite.
 * bf16 with D = 128 runs the MFMA kernels; the other combinations run plain
 * fp32 FMA kernels (correct at any size, tuned for none).
 *
 * Ownership.  The caller allocates and owns every buffer, including the
 * workspace (size from hstu_attn_workspace_size).  The library keeps no
 * pointer after a call returns and allocates no device memory itself.  Work is
 * enqueued on `stream` (a hipStream_t passed as void*; NULL = the default
 * stream) and runs asynchronously; buffers must stay valid until it completes.
 *
 * Errors.  Every entry point validates its arguments on the host before
 * enqueueing anything and returns a status; on failure nothing is enqueued and
 * hstu_last_error() describes the problem.  The library never aborts.  Device
 * contents (offsets, target rows) are not read by the host: kernels clamp them
 * into range, so malformed offsets give wrong results but no out-of-bounds
 * access; hstu_attn_check_inputs() reports them.
 */
#ifndef HSTU_ATTN_H
#define HSTU_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HSTU_BF16 = 0, HSTU_FP32 = 1 } hstu_dtype_t;

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID = -1,     /* bad argument (null, misaligned, out of range) */
  HSTU_ERR_UNSUPPORTED = -2, /* valid but not supported (e.g. D = 96, nfunc too large) */
  HSTU_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  HSTU_ERR_DEVICE = -4,      /* a HIP runtime call failed */
  HSTU_ERR_INPUT = -5        /* hstu_attn_check_inputs found malformed device data */
} hstu_status_t;

/* Largest nfunc accepted (odd).  The reference wheel fixed nfunc at build time
 * and a proposed query op reported it (PR #670 review thread); here nfunc is a
 * runtime argument up to this bound. */
int hstu_max_nfunc(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* hstu_last_error(void);

/* Bytes of device workspace a call needs (fwd: is_bwd = 0, bwd: 1) for these
 * sizes (either dtype); targets_only != 0 for the targets-only mode.  Returns
 * 0 for sizes the library does not support (the entry point then reports
 * why).  The workspace is scratch: its contents need not be preserved between
 * calls. */
size_t hstu_attn_workspace_size(int is_bwd, int64_t B, int64_t total, int H, int D, int nfunc,
                                int targets_only);

/* Forward: writes o ([total,H,D], or [B,H,D] when target_rows != NULL).
 * q has the shape of o; k, v are [total,H,D]. */
int hstu_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o,
                  const int64_t* seq_offsets, int64_t B, int64_t total, int H, int D,
                  const int32_t* func, int nfunc, float alpha, int64_t max_len,
                  const int32_t* target_rows, void* workspace, size_t workspace_bytes,
                  void* stream);

/* The forward of hstu_attn_fwd (same arguments, same kernels, same results)
 * without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Its workspace is a fixed 32 MiB array in device memory
 * that the library holds on every GPU it runs on until the process ends; the
 * call itself allocates nothing.  Sizes whose workspace
 * (hstu_attn_workspace_size) exceeds 32 MiB are rejected with
 * HSTU_ERR_UNSUPPORTED before anything is enqueued; full-length calls up to
 * about 8 million tokens at H = 4 fit.  The array is shared by every call on
 * a GPU: calls that overlap on one GPU (other streams, other threads) race
 * and must not be issued. */
int hstu_attn_fwd_noalloc(int dtype, const void* q, const void* k, const void* v, void* o,
                          const int64_t* seq_offsets, int64_t B, int64_t total, int H, int D,
                          const int32_t* func, int nfunc, float alpha, int64_t max_len,
                          const int32_t* target_rows, void* stream);

/* Backward: from dout (shape of o) writes dq (shape of q) and dk, dv
 * ([total,H,D]).  dk and dv are deterministic (bitwise repeatable); so is dq. */
int hstu_attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* dout,
                  void* dq, void* dk, void* dv, const int64_t* seq_offsets, int64_t B,
                  int64_t total, int H, int D, const int32_t* func, int nfunc, float alpha,
                  int64_t max_len, const int32_t* target_rows, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Stored-P backward (bf16, D = 128, full-length mode): the same outputs as
 * hstu_attn_bwd (dtype HSTU_BF16, target_rows NULL).  Instead of a query-owner
 * pass that recomputes <q_i, k_j> and <dO_i, v_j> for dQ, the key-owner pass
 * also writes, for every 32-row x 128-key block it visits, the bf16 values
 * max_len * dP_ij that it feeds its own dK product (0 for masked pairs) into
 * `pstore`, and dQ_i = alpha/max_len * sum_j (max_len dP_ij) k_j is formed
 * from them.  This trades HBM capacity and bandwidth (about 2 bytes per
 * (row, column) pair of each sequence's L x L square, per head) for 4*D of
 * the 14*D executed flops per visible pair.
 * pstore: device buffer, 256-byte aligned, of pstore_bytes bytes; scratch
 * (contents not preserved).  It must hold hstu_attn_pstore_bytes bytes for
 * the device offsets.  Those are known on the device only, so the call does
 * not wait for them: every access to pstore is range-checked against
 * pstore_bytes (nothing outside the buffer is read or written, whatever its
 * size), and if the buffer is smaller than the offsets need, dk and dv are
 * still correct and every row of dq is written as NaN.  The call enqueues
 * its work and returns without synchronizing `stream`.  dk, dv and dq are
 * deterministic. */
int hstu_attn_bwd_pstore(const void* q, const void* k, const void* v, const void* dout, void* dq,
                         void* dk, void* dv, const int64_t* seq_offsets, int64_t B, int64_t total,
                         int H, int D, const int32_t* func, int nfunc, float alpha,
                         int64_t max_len, void* workspace, size_t workspace_bytes, void* pstore,
                         size_t pstore_bytes, void* stream);

/* Bytes of `pstore` that hstu_attn_bwd_pstore needs: the sum over sequences of
 * ceil(L_b/128) * ceil(L_b/32) * 8192 * H.  seq_offsets is a HOST copy of the
 * int64 [B+1] offsets (sanitized exactly as the kernels do: clamped into
 * [0, total], running maximum).  Returns 0 for unsupported sizes. */
size_t hstu_attn_pstore_bytes(const int64_t* seq_offsets, int64_t B, int64_t total, int H);

/* Stored-P backward with a buffer of any size the caller picks: the batch is
 * cut into runs of consecutive sequences, each as long as the buffer holds
 * its stored P (ceil(L/128) * ceil(L/32) * 8192 * H bytes per sequence), and
 * hstu_attn_bwd_pstore's work runs once per run on `stream`, each run
 * reusing the buffer.  The outputs are bitwise those of hstu_attn_bwd_pstore
 * with a buffer that holds the whole batch; the footprint is pstore_bytes,
 * whatever the batch size (the pages' layer shapes reach 137 GB of stored P
 * for the whole batch at L = 4086: MLCommons training PR #903, "Evidence").
 * Each run launches its own prep and passes, so runs should hold many
 * sequences (a buffer of a few GB at the pages' shapes).
 * host_offsets: a HOST copy of seq_offsets (int64 [B+1], 0 = first <= ... <=
 * last = total), read before anything is enqueued to cut the runs; the
 * device offsets of each run are clamped into that run's rows, so a device
 * copy that disagrees with it gives wrong gradients but no access outside
 * the tensors.  Fails with HSTU_ERR_INVALID, before enqueueing anything, when
 * host_offsets is malformed or one sequence alone needs more than
 * pstore_bytes.  Other arguments, the workspace (hstu_attn_workspace_size
 * with is_bwd = 1) and the asynchronous, deterministic behaviour are those
 * of hstu_attn_bwd_pstore. */
int hstu_attn_bwd_pstore_chunked(const void* q, const void* k, const void* v, const void* dout,
                                 void* dq, void* dk, void* dv, const int64_t* seq_offsets,
                                 const int64_t* host_offsets, int64_t B, int64_t total, int H,
                                 int D, const int32_t* func, int nfunc, float alpha,
                                 int64_t max_len, void* workspace, size_t workspace_bytes,
                                 void* pstore, size_t pstore_bytes, void* stream);

/* Atomic-dQ backward (bf16, D = 128, full-length mode): the same dk and dv as
 * hstu_attn_bwd, bitwise, and dq up to the order of fp32 additions.  It is the
 * variant the pages rank against the deterministic dQ kernel (MLCommons
 * training PR #903, "Read First": gradients close rather than bitwise equal
 * are acceptable): the key-owner pass also forms, for every 32-row half it
 * walks, the dQ contribution of its 128 keys and adds it to dq_accum with
 * fp32 atomics, so there is neither a query-owner pass that recomputes
 * <q_i, k_j> and <dO_i, v_j> nor a stored P.  The additions reach each
 * element in no fixed order: dq is not bitwise repeatable.
 * dq_accum: device buffer of at least total*H*D*4 bytes (fp32 [total, H, D]),
 * 256-byte aligned; scratch (cleared and overwritten by the call).  dq is
 * written from it (times alpha/max_len, rounded to bf16) after the pass.
 * Workspace and other arguments as hstu_attn_bwd; the call enqueues its work
 * and returns without synchronizing `stream`. */
int hstu_attn_bwd_atomic(const void* q, const void* k, const void* v, const void* dout, void* dq,
                         void* dk, void* dv, const int64_t* seq_offsets, int64_t B, int64_t total,
                         int H, int D, const int32_t* func, int nfunc, float alpha,
                         int64_t max_len, void* workspace, size_t workspace_bytes, void* dq_accum,
                         size_t dq_accum_bytes, void* stream);

/* Visible-column count |V_i| of every query row: counts is int32 [total]
 * (or [B] with target_rows), total_pairs a device int64 receiving their sum.
 * Either output may be NULL.  Integer work: exact. */
int hstu_attn_visible_counts(const int64_t* seq_offsets, int64_t B, int64_t total,
                             const int32_t* func, int nfunc, const int32_t* target_rows,
                             int32_t* counts, int64_t* total_pairs, void* stream);

/* Validates device-resident inputs: seq_offsets[0] == 0, nondecreasing,
 * seq_offsets[B] == total, and (if given) 0 <= target_rows[b] < L_b for every
 * non-empty sequence.  Needs hstu_attn_workspace_size(0, ...) bytes of
 * workspace.  Synchronizes `stream`; returns HSTU_OK or HSTU_ERR_INPUT. */
int hstu_attn_check_inputs(const int64_t* seq_offsets, int64_t B, int64_t total,
                           const int32_t* target_rows, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Per-kernel timing (a profiling aid, not part of the operator).  While
 * enabled, every kernel an entry point enqueues is bracketed by a HIP event
 * pair recorded on the same stream.  hstu_profile_enable returns the previous
 * state.  hstu_profile_read waits for the recorded events, folds them into
 * per-kernel totals and writes lines "kernel_name count total_ms" into buf
 * (NUL-terminated, truncated to len); it returns the size needed including
 * the NUL.  hstu_profile_reset drops all totals. */
int hstu_profile_enable(int on);
size_t hstu_profile_read(char* buf, size_t len);
void hstu_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_ATTN_H */
