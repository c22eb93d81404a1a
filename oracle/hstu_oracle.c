/*
 * HSTU jagged masked attention -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (the plainest reading of the pages; every point where the
 * pages are silent is listed in the project's design notes):
 *
 *   Mask.  TorchEasyRec PR #670 ("move the HSTU arbitrary-mask path to
 *   NFUNC=5", sections "Why" and "What changed"): each query row carries nfunc
 *   int32 bounds laid out interleaved.  Interval 0 is [0, f0); interval j is
 *   [f(2j-1), f(2j)) for j = 1 .. (nfunc-1)/2; a pair whose end is <= its start
 *   is empty and skipped; the visible columns of a row are the OR (union) of
 *   its intervals.  Bounds are sequence-local and are clipped to [0, L_b), so
 *   a row never reaches into another sequence.  The same func column serves
 *   every head (the review reply on PR #670 shows the head dimension of func is
 *   never read).
 *
 *   Scores.  For a visible pair (i, j) of sequence b and head h:
 *       P_ij = alpha * <q_i, k_j>,  S_ij = silu(P_ij) / max_len,
 *       O_i  = sum over visible j of S_ij * v_j.
 *   Pairs that are not visible contribute nothing (outputs of a row with no
 *   visible column are exactly 0).
 *
 *   Backward, with silu'(x) = s(x) * (1 + x * (1 - s(x))), s = logistic:
 *       dS_ij = <dO_i, v_j>,  dP_ij = dS_ij * silu'(P_ij) / max_len,
 *       dV_j += S_ij dO_i,  dQ_i += alpha dP_ij k_j,  dK_j += alpha dP_ij q_i.
 *
 *   Targets-only mode (MLCommons training PR #903, "Summary"): one candidate
 *   row per sequence forms Q (q, o, dO, dq are [B, H, D]) against full-length
 *   K/V; its func column is the one of that row in the full-length layout.
 *
 * Layouts: q, k, v, o, dO, dq, dk, dv are row-major [rows, H, D] doubles;
 * func is [nfunc, total] int32; seq_offsets is int64 [B+1].  Loops run over
 * rows and columns in increasing order; OpenMP splits (sequence, head) pairs,
 * which own disjoint output rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS (-1)
#define ORACLE_ERR_OFFSETS (-2)
#define ORACLE_ERR_TARGET (-3)
#define ORACLE_ERR_NOMEM (-4)

static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * logistic(x); }
static double silu_grad(double x) {
  double s = logistic(x);
  return s * (1.0 + x * (1.0 - s));
}

/* Mark the columns of [lo, hi) clipped to [0, L). */
static void mark_interval(unsigned char* mark, int64_t L, int64_t lo, int64_t hi) {
  if (lo < 0) lo = 0;
  if (hi > L) hi = L;
  if (hi <= lo) return; /* empty pair: skipped */
  for (int64_t c = lo; c < hi; ++c) mark[c] = 1;
}

/* Visible-column set of the row whose func column is `fcol`, in a sequence of
 * length L.  mark[c] = 1 for every visible column c. */
static void decode_row(const int32_t* func, int nfunc, int64_t total, int64_t fcol, int64_t L,
                       unsigned char* mark) {
  memset(mark, 0, (size_t)L);
  mark_interval(mark, L, 0, func[fcol]);
  for (int j = 1; j <= (nfunc - 1) / 2; ++j) {
    int64_t lo = func[(int64_t)(2 * j - 1) * total + fcol];
    int64_t hi = func[(int64_t)(2 * j) * total + fcol];
    mark_interval(mark, L, lo, hi);
  }
}

static int check_common(const int64_t* off, int64_t B, int64_t total, int nfunc) {
  if (B < 0 || total < 0 || nfunc < 1 || (nfunc % 2) == 0) return ORACLE_ERR_ARGS;
  if (off[0] != 0 || off[B] != total) return ORACLE_ERR_OFFSETS;
  for (int64_t b = 0; b < B; ++b)
    if (off[b + 1] < off[b]) return ORACLE_ERR_OFFSETS;
  return ORACLE_OK;
}

static int check_targets(const int64_t* off, int64_t B, const int32_t* target_rows) {
  if (!target_rows) return ORACLE_OK;
  for (int64_t b = 0; b < B; ++b) {
    int64_t L = off[b + 1] - off[b];
    if (L > 0 && (target_rows[b] < 0 || target_rows[b] >= L)) return ORACLE_ERR_TARGET;
  }
  return ORACLE_OK;
}

static int64_t max_length(const int64_t* off, int64_t B) {
  int64_t m = 0;
  for (int64_t b = 0; b < B; ++b)
    if (off[b + 1] - off[b] > m) m = off[b + 1] - off[b];
  return m;
}

/* Number of visible columns per query row: counts[t] for global row t in
 * full-length mode, counts[b] for the candidate of sequence b in targets-only
 * mode.  Returns the total through *total_pairs. */
int oracle_visible_counts(const int64_t* off, int64_t B, int64_t total, const int32_t* func,
                          int nfunc, const int32_t* target_rows, int32_t* counts,
                          int64_t* total_pairs) {
  int st = check_common(off, B, total, nfunc);
  if (st) return st;
  if ((st = check_targets(off, B, target_rows))) return st;
  unsigned char* mark = (unsigned char*)malloc((size_t)(max_length(off, B) + 1));
  if (!mark) return ORACLE_ERR_NOMEM;
  int64_t sum = 0;
  for (int64_t b = 0; b < B; ++b) {
    int64_t L = off[b + 1] - off[b];
    int64_t r0 = target_rows ? target_rows[b] : 0;
    int64_t r1 = target_rows ? target_rows[b] + 1 : L;
    if (L == 0) {
      if (target_rows) counts[b] = 0;
      continue;
    }
    for (int64_t i = r0; i < r1; ++i) {
      decode_row(func, nfunc, total, off[b] + i, L, mark);
      int64_t n = 0;
      for (int64_t c = 0; c < L; ++c) n += mark[c];
      counts[target_rows ? b : off[b] + i] = (int32_t)n;
      sum += n;
    }
  }
  free(mark);
  if (total_pairs) *total_pairs = sum;
  return ORACLE_OK;
}

/* Forward.  o must hold rows x H x D doubles (rows = total, or B in
 * targets-only mode); it is fully overwritten. */
int oracle_fwd(const double* q, const double* k, const double* v, double* o, const int64_t* off,
               int64_t B, int64_t total, int H, int D, const int32_t* func, int nfunc,
               double alpha, double max_len, const int32_t* target_rows) {
  int st = check_common(off, B, total, nfunc);
  if (st) return st;
  if ((st = check_targets(off, B, target_rows))) return st;
  if (H < 1 || D < 1) return ORACLE_ERR_ARGS;
  int64_t rows = target_rows ? B : total;
  memset(o, 0, sizeof(double) * (size_t)(rows * H * D));
  int64_t maxL = max_length(off, B);
  int failed = 0;
#pragma omp parallel
  {
    unsigned char* mark = (unsigned char*)malloc((size_t)(maxL + 1));
    if (!mark) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < B * H; ++u) {
      if (!mark) continue;
      int64_t b = u / H;
      int h = (int)(u % H);
      int64_t L = off[b + 1] - off[b];
      if (L == 0) continue;
      int64_t r0 = target_rows ? target_rows[b] : 0;
      int64_t r1 = target_rows ? target_rows[b] + 1 : L;
      for (int64_t i = r0; i < r1; ++i) {
        int64_t qrow = target_rows ? b : off[b] + i;
        const double* qi = q + (qrow * H + h) * D;
        double* oi = o + (qrow * H + h) * D;
        decode_row(func, nfunc, total, off[b] + i, L, mark);
        for (int64_t c = 0; c < L; ++c) {
          if (!mark[c]) continue;
          const double* kc = k + ((off[b] + c) * H + h) * D;
          const double* vc = v + ((off[b] + c) * H + h) * D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qi[d] * kc[d];
          double s = silu(alpha * dot) / max_len;
          for (int d = 0; d < D; ++d) oi[d] += s * vc[d];
        }
      }
    }
    free(mark);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* Backward.  dq has the shape of q; dk and dv have the shape of k; all three
 * are fully overwritten (gradients of pairs that are never visible stay 0). */
int oracle_bwd(const double* q, const double* k, const double* v, const double* dout, double* dq,
               double* dk, double* dv, const int64_t* off, int64_t B, int64_t total, int H, int D,
               const int32_t* func, int nfunc, double alpha, double max_len,
               const int32_t* target_rows) {
  int st = check_common(off, B, total, nfunc);
  if (st) return st;
  if ((st = check_targets(off, B, target_rows))) return st;
  if (H < 1 || D < 1) return ORACLE_ERR_ARGS;
  int64_t rows = target_rows ? B : total;
  memset(dq, 0, sizeof(double) * (size_t)(rows * H * D));
  memset(dk, 0, sizeof(double) * (size_t)(total * H * D));
  memset(dv, 0, sizeof(double) * (size_t)(total * H * D));
  int64_t maxL = max_length(off, B);
  int failed = 0;
#pragma omp parallel
  {
    unsigned char* mark = (unsigned char*)malloc((size_t)(maxL + 1));
    if (!mark) failed = 1;
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < B * H; ++u) {
      if (!mark) continue;
      int64_t b = u / H;
      int h = (int)(u % H);
      int64_t L = off[b + 1] - off[b];
      if (L == 0) continue;
      int64_t r0 = target_rows ? target_rows[b] : 0;
      int64_t r1 = target_rows ? target_rows[b] + 1 : L;
      for (int64_t i = r0; i < r1; ++i) {
        int64_t qrow = target_rows ? b : off[b] + i;
        const double* qi = q + (qrow * H + h) * D;
        const double* doi = dout + (qrow * H + h) * D;
        double* dqi = dq + (qrow * H + h) * D;
        decode_row(func, nfunc, total, off[b] + i, L, mark);
        for (int64_t c = 0; c < L; ++c) {
          if (!mark[c]) continue;
          int64_t kr = ((off[b] + c) * H + h) * D;
          const double* kc = k + kr;
          const double* vc = v + kr;
          double dot = 0.0, ds = 0.0;
          for (int d = 0; d < D; ++d) dot += qi[d] * kc[d];
          for (int d = 0; d < D; ++d) ds += doi[d] * vc[d];
          double p = alpha * dot;
          double s = silu(p) / max_len;
          double dp = ds * silu_grad(p) / max_len;
          for (int d = 0; d < D; ++d) {
            dv[kr + d] += s * doi[d];
            dqi[d] += alpha * dp * kc[d];
            dk[kr + d] += alpha * dp * qi[d];
          }
        }
      }
    }
    free(mark);
  }
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}
