/*
 * Oracle A — the Gated DeltaNet recurrence evaluated token by token in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (FlashQLA talk transcript, "Qwen系列模型线性注意力高性能优化实践",
 * tokendh.com — the linear-attention section on the token recurrence into a
 * d x d state, the GDN section introducing the update gate beta and forget
 * gate alpha, and the sliding-window section naming the factor I - beta k k^T
 * with L2-normalised keys):
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t                      (post-update state)
 *
 * with S_t a dv x dk matrix and alpha_t = exp(g_t) (the pages store log alpha).
 * Expanding the product gives the equivalent per-token steps used below:
 *
 *     S <- alpha_t S
 *     u <- v_t - S k_t
 *     S <- S + beta_t u k_t^T
 *     o_t <- scale * S q_t
 *
 * Row j of S only ever touches row j (u_j = v_j - S[j,:].k), so value rows are
 * independent and the loop is parallelised over (sequence, head, row block).
 *
 * Layouts (all fp64, contiguous):
 *   q, k : [Ttot, H, dk]     v, o : [Ttot, H, dv]     g, beta : [Ttot, H]
 *   h0, hT : [N, H, dk, dv]  -- the state stored K-major: h[i][j] = S[j][i]
 *   cu : [N+1] token offsets of the N sequences inside Ttot
 * h0 may be NULL (zero initial state); hT may be NULL (not written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ROWS_PER_TASK 16

static void run_rows(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* h0, int64_t t0, int64_t t1, int64_t H,
                     int64_t h, int64_t dk, int64_t dv, int64_t j0, int64_t j1, double scale,
                     double* o, double* hT, int64_t state_off) {
  int64_t nr = j1 - j0;
  double* S = (double*)malloc(sizeof(double) * (size_t)(nr * dk));
  /* S[r][i] = S_{j0+r, i} = h0[i][j0+r] */
  for (int64_t r = 0; r < nr; ++r)
    for (int64_t i = 0; i < dk; ++i)
      S[r * dk + i] = h0 ? h0[state_off + i * dv + (j0 + r)] : 0.0;

  for (int64_t t = t0; t < t1; ++t) {
    const double* kt = k + (t * H + h) * dk;
    const double* qt = q + (t * H + h) * dk;
    const double* vt = v + (t * H + h) * dv;
    double alpha = exp(g[t * H + h]);
    double b = beta[t * H + h];
    double* ot = o + (t * H + h) * dv;
    for (int64_t r = 0; r < nr; ++r) {
      double* s = S + r * dk;
      double sk = 0.0;
      for (int64_t i = 0; i < dk; ++i) {
        s[i] *= alpha;
        sk += s[i] * kt[i];
      }
      double u = vt[j0 + r] - sk;
      double sq = 0.0;
      for (int64_t i = 0; i < dk; ++i) {
        s[i] += b * u * kt[i];
        sq += s[i] * qt[i];
      }
      ot[j0 + r] = scale * sq;
    }
  }
  if (hT)
    for (int64_t r = 0; r < nr; ++r)
      for (int64_t i = 0; i < dk; ++i) hT[state_off + i * dv + (j0 + r)] = S[r * dk + i];
  free(S);
}

/* Returns 0 on success, -1 on bad arguments. */
int gdn_oracle_token(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const double* h0, const int64_t* cu, int64_t N,
                     int64_t H, int64_t dk, int64_t dv, double scale, double* o, double* hT,
                     int nthreads) {
  if (!q || !k || !v || !g || !beta || !cu || !o || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
    return -1;
  int64_t nblk = (dv + ROWS_PER_TASK - 1) / ROWS_PER_TASK;
  int64_t ntask = N * H * nblk;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t task = 0; task < ntask; ++task) {
    int64_t blk = task % nblk;
    int64_t nh = task / nblk;
    int64_t h = nh % H;
    int64_t n = nh / H;
    int64_t j0 = blk * ROWS_PER_TASK;
    int64_t j1 = j0 + ROWS_PER_TASK < dv ? j0 + ROWS_PER_TASK : dv;
    run_rows(q, k, v, g, beta, h0, cu[n], cu[n + 1], H, h, dk, dv, j0, j1, scale, o, hT,
             (n * H + h) * dk * dv);
  }
  return 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
