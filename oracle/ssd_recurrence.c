/*
 * TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the Mamba-2 SSD forward.
 * Only the tests, the smoke check and the bench's CPU-baseline leg load it;
 * the product path never does.  It shares no code with the HIP library.
 *
 * What it computes: the selective state-space recurrence that the SSD
 * chunked scan reaches exactly in exact arithmetic.  The pages describe a
 * fixed-size hidden state updated with every token and its chunkwise form
 * (aiproviderindex.com, item on CUDA Tile Mamba-2 kernels, "Mamba-2 offers a
 * different scaling path": the state update, chunk-wise cumulative
 * parameters, state propagation and output construction) without writing
 * the update out; it is read as the plain Mamba-2 selective update.  For each
 * sequence s, head h (group g = h / (H / G)) and token t of the sequence:
 *
 *   delta_t   = clamp(softplus(dt[t,h] + dt_bias[h]), dt_min, dt_max)
 *   a_t       = exp(delta_t * A[h])
 *   h_{-1}    = initial_states[s,h]            (P x N), or 0
 *   h_t[p,n]  = a_t * h_{t-1}[p,n] + delta_t * x[t,h,p] * B[t,g,n]
 *   y[t,h,p]  = sum_n C[t,g,n] * h_t[p,n] + D[h] * x[t,h,p]
 *   final[s,h]= h_{T_s - 1}
 *
 * softplus(u) = max(u, 0) + log1p(exp(-|u|)), the overflow-free form of
 * log(1 + exp(u)).
 *
 * Plain loops, fp64 throughout, OpenMP over (sequence, selected head) only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus(double u) {
  return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)));
}

/*
 * Arrays (row-major, fp64):
 *   x        [Ttot, Hs, P]   the selected heads' inputs, all tokens
 *   dt       [Ttot, Hs]      raw dt of the selected heads
 *   dt_bias  [Hs] or NULL;  A [Hs];  D [Hs] or NULL
 *   grp      [Hs]            B/C group of each selected head
 *   B, C     [Ttot, G, N]
 *   init     [nseq, Hs, P, N] or NULL
 *   seq_start, seq_len [nseq]: token ranges in the flattened token axis
 * Outputs:
 *   y        [Ttot, Hs, P]   (tokens outside every sequence are left as is)
 *   final    [nseq, Hs, P, N] or NULL
 * Returns 0, or -1 for an out-of-range argument.
 */
int ssd_oracle_recurrence(int64_t nseq, const int64_t* seq_start, const int64_t* seq_len,
                          int64_t Ttot, int64_t Hs, int64_t P, int64_t N, int64_t G,
                          const double* x, const double* dt, const double* dt_bias,
                          const double* A, const int64_t* grp,
                          const double* B, const double* C, const double* D,
                          const double* init, double dt_min, double dt_max,
                          double* y, double* final_states, int nthreads) {
  if (nseq < 0 || Ttot < 0 || Hs < 0 || P <= 0 || N <= 0 || G <= 0) return -1;
  for (int64_t s = 0; s < nseq; ++s) {
    if (seq_start[s] < 0 || seq_len[s] < 0 || seq_start[s] + seq_len[s] > Ttot) return -1;
  }
  for (int64_t j = 0; j < Hs; ++j)
    if (grp[j] < 0 || grp[j] >= G) return -1;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t work = nseq * Hs;
#pragma omp parallel
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)(P * N));
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < work; ++w) {
      const int64_t s = w / Hs, j = w % Hs, g = grp[j];
      if (init)
        memcpy(h, init + ((s * Hs + j) * P) * N, sizeof(double) * (size_t)(P * N));
      else
        memset(h, 0, sizeof(double) * (size_t)(P * N));
      for (int64_t tt = 0; tt < seq_len[s]; ++tt) {
        const int64_t t = seq_start[s] + tt;
        double d = softplus(dt[t * Hs + j] + (dt_bias ? dt_bias[j] : 0.0));
        if (d < dt_min) d = dt_min;
        if (d > dt_max) d = dt_max;
        const double a = exp(d * A[j]);
        const double* xt = x + (t * Hs + j) * P;
        const double* bt = B + (t * G + g) * N;
        const double* ct = C + (t * G + g) * N;
        double* yt = y + (t * Hs + j) * P;
        for (int64_t p = 0; p < P; ++p) {
          const double dx = d * xt[p];
          double* hp = h + p * N;
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            hp[n] = a * hp[n] + dx * bt[n];
            acc += ct[n] * hp[n];
          }
          yt[p] = acc + (D ? D[j] : 0.0) * xt[p];
        }
      }
      if (final_states)
        memcpy(final_states + ((s * Hs + j) * P) * N, h, sizeof(double) * (size_t)(P * N));
    }
    free(h);
  }
  return 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
