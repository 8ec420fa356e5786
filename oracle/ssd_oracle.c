/*
 * Plain CPU oracle for the Mamba-2 SSD (state-space duality) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library and is written from the pages' description of the method:
 *
 *   [D2] devotd.net, news item on the Mamba-2 CUDA Tile forward-pass kernels,
 *        section 1 (recurrent model turned into chunks) and section 2 (three
 *        kernels, including the chunk_cumsum code figure);
 *   [DA] disconfirmai.com, "Jane Street ML Engineers Map Mamba-2 Recurrent
 *        State Computation to Tensor Cores with cuTile", body (fixed-size
 *        hidden state, jump formula, log-space cumulative decay).
 *
 * The method evaluates, chunk by chunk, a linear recurrence with a fixed-size
 * state.  Where the chunked evaluation reaches a result exactly (up to
 * rounding order), this file computes that result from its plain definition:
 * the token-by-token recurrence, in double precision, with natural exp and no
 * log-space cumulative sums.  For batch b, head h (group g = h / (H/G)),
 * headdim row p and state column n:
 *
 *     s_0      = h0[b,h]                     (zero when no initial state)
 *     a_t      = exp(dt[b,t,h] * A[h])        decay over one step: the product
 *                                             of decay rate and time interval
 *     s_t[p,n] = a_t * s_{t-1}[p,n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p] = sum_n s_t[p,n] * C[b,t,g,n] + D[h] * x[b,t,h,p]
 *
 * y reads the state after the update at step t.  Rows p of the state are
 * independent of each other, so the loops below run over (b, h, p) in
 * parallel; each row walks time in order.
 *
 * Parity status of each function (pins live in tests/test_oracle_pins.py):
 *   oracle_chunk_cumsum         pinned (hand-worked golden, decay identity)
 *   oracle_ssd_recurrence       pinned (hand-worked goldens, closed forms,
 *                               first-order IIR filter, brute force)
 *   oracle_chunk_local_states   pinned (no-decay matrix-product identity,
 *                               independent chunked form)
 *   oracle_state_passing        pinned (reproduces recurrence snapshots)
 *   oracle_chunk_outputs        pinned (reproduces recurrence outputs)
 *   oracle_ssd_backward         pinned (central finite differences of
 *                               oracle_ssd_recurrence, every input)
 * The head-to-group convention g = h / (H/G) is a stated convention: parity
 * unpinned against the pages, which do not fix it.
 *
 * Inputs are float32 arrays (bfloat16 values widen to float32 exactly);
 * all arithmetic is double.  Layouts are contiguous row-major:
 *   x[B,L,H,P]  dt[B,L,H]  A[H]  Bm,C[B,L,G,N]  D[H]  h0[B,H,P,N]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size;
} oracle_dims;

/* log2(e) in double: the pages scale the cumulative sum by LOG2E so that
 * consumers use base-2 exponentials ([D2] section 2, code figure). */
static const double ORACLE_LOG2E = 1.4426950408889634073599246810019;

static int dims_ok(const oracle_dims* d) {
  if (!d) return 0;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 ||
      d->dstate <= 0 || d->ngroups <= 0 || d->chunk_size <= 0)
    return 0;
  if (d->nheads % d->ngroups) return 0;
  return 1;
}

static int64_t nchunks(const oracle_dims* d) {
  return (d->seqlen + d->chunk_size - 1) / d->chunk_size;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * In-chunk cumulative sum of the log-decay ([D2] section 2: chunk_cumsum
 * accumulates decay rate times time interval within the chunk and stores it;
 * code figure: zero-padded dt tile, float cast, inclusive cumsum of A*dt
 * along time, then times LOG2E).  Positions past the sequence end read dt = 0
 * (zero padding), so the sum there stays at its last value.
 *   dA_cs[b,h,c,i] = LOG2E * sum_{j<=i} A[h] * dt[b, cQ+j, h]
 *   dt_T[b,h,c,i]  = dt[b, cQ+i, h]   (0 past the end)
 * Both outputs are [B,H,nc,Q] doubles.
 */
int oracle_chunk_cumsum(const oracle_dims* d, const float* dt, const float* A,
                        double* dA_cs, double* dt_T) {
  if (!dims_ok(d) || !dt || !A || !dA_cs) return 1;
  const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, Q = d->chunk_size;
  const int64_t nc = nchunks(d);
  for (int64_t b = 0; b < Bn; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t c = 0; c < nc; ++c) {
        double sum = 0.0;
        for (int64_t i = 0; i < Q; ++i) {
          const int64_t t = c * Q + i;
          const double dtv = (t < L) ? (double)dt[(b * L + t) * H + h] : 0.0;
          sum += (double)A[h] * dtv;
          const int64_t o = ((b * H + h) * nc + c) * Q + i;
          dA_cs[o] = sum * ORACLE_LOG2E;
          if (dt_T) dt_T[o] = dtv;
        }
      }
  return 0;
}

/* Resolves the selected head list: heads == NULL selects all heads. */
static int head_of(const oracle_dims* d, int nsel, const int* heads, int k) {
  (void)d; (void)nsel;
  return heads ? heads[k] : k;
}

static int heads_ok(const oracle_dims* d, int nsel, const int* heads) {
  if (nsel <= 0) return 0;
  if (!heads) return nsel == d->nheads;
  for (int k = 0; k < nsel; ++k)
    if (heads[k] < 0 || heads[k] >= d->nheads) return 0;
  return 1;
}

/*
 * The full forward pass by its definition: the token-by-token recurrence
 * written above ([DA] body: a fixed-size hidden state updated per token;
 * [D2] section 1).  Outputs are for the selected heads only (slot k holds
 * head heads[k]):
 *   y[B,L,nsel,P]                         outputs
 *   final_state[B,nsel,P,N]  (nullable)   state after the last token
 *   h_start[B,nc,nsel,P,N]   (nullable)   state before the first token of
 *                                         each chunk, i.e. s_{cQ}; the state
 *                                         fwd_pass_state produces at chunk
 *                                         starts ([D2] section 2)
 */
int oracle_ssd_recurrence(const oracle_dims* d, const float* x, const float* dt,
                          const float* A, const float* Bm, const float* C,
                          const float* D, const float* h0, int nsel,
                          const int* heads, double* y, double* final_state,
                          double* h_start) {
  if (!dims_ok(d) || !heads_ok(d, nsel, heads)) return 1;
  if (!x || !dt || !A || !Bm || !C || !y) return 1;
  const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
  const int64_t N = d->dstate, G = d->ngroups, Q = d->chunk_size;
  const int64_t nc = nchunks(d), hpg = H / G;
  const int64_t rows = Bn * (int64_t)nsel * P;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t p = r % P;
      const int64_t k = (r / P) % nsel;
      const int64_t b = r / (P * nsel);
      const int64_t h = head_of(d, nsel, heads, (int)k);
      const int64_t g = h / hpg;
      for (int64_t n = 0; n < N; ++n)
        s[n] = h0 ? (double)h0[((b * H + h) * P + p) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        if (h_start && t % Q == 0) {
          double* hs = h_start + (((b * nc + t / Q) * nsel + k) * P + p) * N;
          for (int64_t n = 0; n < N; ++n) hs[n] = s[n];
        }
        const double dtv = (double)dt[(b * L + t) * H + h];
        const double a = exp(dtv * (double)A[h]);
        const double xv = (double)x[((b * L + t) * H + h) * P + p];
        const float* Bt = Bm + ((b * L + t) * G + g) * N;
        const float* Ct = C + ((b * L + t) * G + g) * N;
        for (int64_t n = 0; n < N; ++n) s[n] = a * s[n] + dtv * xv * (double)Bt[n];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += s[n] * (double)Ct[n];
        if (D) acc += (double)D[h] * xv;
        y[((b * L + t) * nsel + k) * P + p] = acc;
      }
      if (final_state) {
        double* fs = final_state + ((b * nsel + k) * P + p) * N;
        for (int64_t n = 0; n < N; ++n) fs[n] = s[n];
      }
    }
    free(s);
  }
  return 0;
}

/*
 * Per-chunk local states: the same recurrence run over chunk c alone,
 * starting from a zero state; the result is the state at the chunk's end.
 * This is the per-chunk B X^T contribution of fwd_pass_state ([DA] body:
 * without decay the jump over a chunk is h(t+T) = h(t) + B X^T; with decay
 * the rows are pre-scaled).  Output S[B,nc,nsel,P,N].
 */
int oracle_chunk_local_states(const oracle_dims* d, const float* x,
                              const float* dt, const float* A, const float* Bm,
                              int nsel, const int* heads, double* S) {
  if (!dims_ok(d) || !heads_ok(d, nsel, heads)) return 1;
  if (!x || !dt || !A || !Bm || !S) return 1;
  const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
  const int64_t N = d->dstate, G = d->ngroups, Q = d->chunk_size;
  const int64_t nc = nchunks(d), hpg = H / G;
  const int64_t rows = Bn * (int64_t)nsel * P;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t p = r % P;
      const int64_t k = (r / P) % nsel;
      const int64_t b = r / (P * nsel);
      const int64_t h = head_of(d, nsel, heads, (int)k);
      const int64_t g = h / hpg;
      for (int64_t c = 0; c < nc; ++c) {
        for (int64_t n = 0; n < N; ++n) s[n] = 0.0;
        for (int64_t t = c * Q; t < (c + 1) * Q && t < L; ++t) {
          const double dtv = (double)dt[(b * L + t) * H + h];
          const double a = exp(dtv * (double)A[h]);
          const double xv = (double)x[((b * L + t) * H + h) * P + p];
          const float* Bt = Bm + ((b * L + t) * G + g) * N;
          for (int64_t n = 0; n < N; ++n) s[n] = a * s[n] + dtv * xv * (double)Bt[n];
        }
        double* o = S + (((b * nc + c) * nsel + k) * P + p) * N;
        for (int64_t n = 0; n < N; ++n) o[n] = s[n];
      }
    }
    free(s);
  }
  return 0;
}

/*
 * The jump across chunks, in chunk order ([D2] section 2: fwd_pass_state
 * computes the state at each chunk start and after the last chunk, keeping
 * chunk order; [DA] body: jump formula).  Given each chunk's local state
 * S[b,c,h] and the chunk's total decay factor decay[b,h,c] (the product of
 * the per-step decays inside the chunk):
 *   h_start[b,0,h]   = h0[b,h]  (zero when h0 is NULL)
 *   h_start[b,c+1,h] = decay[b,h,c] * h_start[b,c,h] + S[b,c,h]
 *   final[b,h]       = the value after the last chunk
 * Arrays: S, h_start [B,nc,H,P,N]; decay [B,H,nc]; h0, final [B,H,P,N].
 */
int oracle_state_passing(int64_t batch, int64_t nc, int64_t nheads,
                         int64_t headdim, int64_t dstate, const double* S,
                         const double* decay, const double* h0,
                         double* h_start, double* final_state) {
  if (batch < 0 || nc < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0) return 1;
  if (!S || !decay || !h_start) return 1;
  const int64_t PN = headdim * dstate;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t h = 0; h < nheads; ++h) {
      for (int64_t e = 0; e < PN; ++e) {
        double run = h0 ? h0[(b * nheads + h) * PN + e] : 0.0;
        for (int64_t c = 0; c < nc; ++c) {
          const int64_t o = ((b * nc + c) * nheads + h) * PN + e;
          h_start[o] = run;
          run = decay[(b * nheads + h) * nc + c] * run + S[o];
        }
        if (final_state) final_state[(b * nheads + h) * PN + e] = run;
      }
    }
  return 0;
}

/*
 * Outputs of each chunk given the state at its start ([D2] section 2:
 * compute_out produces the tokens' outputs from the chunk-start state).
 * Within chunk c the recurrence restarts from h_start[b,c,k] and runs over
 * the chunk's tokens; y is read after each update as in the definition.
 * h_start is [B,nc,nsel,P,N] doubles for the selected heads; y is
 * [B,L,nsel,P].
 */
int oracle_chunk_outputs(const oracle_dims* d, const float* x, const float* dt,
                         const float* A, const float* Bm, const float* C,
                         const float* D, int nsel, const int* heads,
                         const double* h_start, double* y) {
  if (!dims_ok(d) || !heads_ok(d, nsel, heads)) return 1;
  if (!x || !dt || !A || !Bm || !C || !h_start || !y) return 1;
  const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
  const int64_t N = d->dstate, G = d->ngroups, Q = d->chunk_size;
  const int64_t nc = nchunks(d), hpg = H / G;
  const int64_t rows = Bn * (int64_t)nsel * P;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t p = r % P;
      const int64_t k = (r / P) % nsel;
      const int64_t b = r / (P * nsel);
      const int64_t h = head_of(d, nsel, heads, (int)k);
      const int64_t g = h / hpg;
      for (int64_t c = 0; c < nc; ++c) {
        const double* hs = h_start + (((b * nc + c) * nsel + k) * P + p) * N;
        for (int64_t n = 0; n < N; ++n) s[n] = hs[n];
        for (int64_t t = c * Q; t < (c + 1) * Q && t < L; ++t) {
          const double dtv = (double)dt[(b * L + t) * H + h];
          const double a = exp(dtv * (double)A[h]);
          const double xv = (double)x[((b * L + t) * H + h) * P + p];
          const float* Bt = Bm + ((b * L + t) * G + g) * N;
          const float* Ct = C + ((b * L + t) * G + g) * N;
          for (int64_t n = 0; n < N; ++n) s[n] = a * s[n] + dtv * xv * (double)Bt[n];
          double acc = 0.0;
          for (int64_t n = 0; n < N; ++n) acc += s[n] * (double)Ct[n];
          if (D) acc += (double)D[h] * xv;
          y[((b * L + t) * nsel + k) * P + p] = acc;
        }
      }
    }
    free(s);
  }
  return 0;
}

/*
 * Gradients of the forward pass, by back-propagation through the same
 * token-by-token recurrence (reverse-mode differentiation of the definition
 * above).  The pages give no backward pass; the disconfirmai.com summary
 * ("Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
 * Tensor Cores with cuTile", lead paragraph) notes that the forward speedups
 * rest on a backward implementation that is not yet published.  For the scalar
 *     loss = sum_{t,p} dy[b,t,h,p] y[b,t,h,p] + sum dfinal[b,h] . s_L
 * with s_{t+1} = a_t s_t + dt_t x_t (outer) B_t (s_0 = h0) and
 * y_t = s_{t+1} . C_t + D x_t, a row p of the state walks time backwards
 * with g = d loss / d s_{t+1}:
 *     g          = dfinal row, then at each t (descending): g += dy_t[p] C_t
 *     dC_t      += dy_t[p] s_{t+1}         dx_t[p]  = D dy_t[p] + dt_t (g . B_t)
 *     dB_t      += dt_t x_t[p] g           ddt_t   += x_t[p] (g . B_t) + A a_t (g . s_t)
 *     dA        += dt_t a_t (g . s_t)      dD      += dy_t[p] x_t[p]
 *     g          = a_t g                   (after t = 0: dh0 row = g)
 * Outputs (double): dx[B,L,H,P], ddt[B,L,H], per-head parts of the group
 * gradients dBh, dCh[B,L,H,N] (the caller sums the heads of each group),
 * per-(batch, head) parts dA_part, dD_part[B,H], and dh0[B,H,P,N] (nullable).
 * dy[B,L,H,P] is required; dfinal[B,H,P,N], D and h0 may be NULL.
 * Each (b, h) runs in one thread, its rows in order, so every output element
 * has a single writer.
 */
int oracle_ssd_backward(const oracle_dims* d, const float* x, const float* dt,
                        const float* A, const float* Bm, const float* C, const float* D,
                        const float* h0, const float* dy, const float* dfinal, double* dx,
                        double* ddt, double* dBh, double* dCh, double* dA_part,
                        double* dD_part, double* dh0) {
  if (!dims_ok(d)) return 1;
  if (!x || !dt || !A || !Bm || !C || !dy || !dx || !ddt || !dBh || !dCh || !dA_part ||
      !dD_part)
    return 1;
  const int64_t Bn = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
  const int64_t N = d->dstate, G = d->ngroups, hpg = H / G;
  const int64_t units = Bn * H;
  int rc = 0;
#pragma omp parallel
  {
    /* states s_0 .. s_L of one row, and the running adjoint */
    double* s = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
    double* g = (double*)malloc(sizeof(double) * (size_t)N);
    if (!s || !g) {
#pragma omp atomic write
      rc = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      if (!s || !g) continue;
      const int64_t b = u / H, h = u % H, gr = h / hpg;
      const double Ah = (double)A[h], Dh = D ? (double)D[h] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        ddt[(b * L + t) * H + h] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          dBh[((b * L + t) * H + h) * N + n] = 0.0;
          dCh[((b * L + t) * H + h) * N + n] = 0.0;
        }
      }
      double dA_acc = 0.0, dD_acc = 0.0;
      for (int64_t p = 0; p < P; ++p) {
        for (int64_t n = 0; n < N; ++n)
          s[n] = h0 ? (double)h0[((b * H + h) * P + p) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
          const double dtv = (double)dt[(b * L + t) * H + h];
          const double a = exp(dtv * Ah);
          const double xv = (double)x[((b * L + t) * H + h) * P + p];
          const float* Bt = Bm + ((b * L + t) * G + gr) * N;
          const double* sp = s + t * N;
          double* sn = s + (t + 1) * N;
          for (int64_t n = 0; n < N; ++n) sn[n] = a * sp[n] + dtv * xv * (double)Bt[n];
        }
        for (int64_t n = 0; n < N; ++n)
          g[n] = dfinal ? (double)dfinal[((b * H + h) * P + p) * N + n] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
          const double dtv = (double)dt[(b * L + t) * H + h];
          const double a = exp(dtv * Ah);
          const double xv = (double)x[((b * L + t) * H + h) * P + p];
          const double dyv = (double)dy[((b * L + t) * H + h) * P + p];
          const float* Bt = Bm + ((b * L + t) * G + gr) * N;
          const float* Ct = C + ((b * L + t) * G + gr) * N;
          const double* sp = s + t * N;
          const double* sn = s + (t + 1) * N;
          double* dBt = dBh + ((b * L + t) * H + h) * N;
          double* dCt = dCh + ((b * L + t) * H + h) * N;
          double gB = 0.0, gs = 0.0;
          for (int64_t n = 0; n < N; ++n) {
            g[n] += dyv * (double)Ct[n];
            dCt[n] += dyv * sn[n];
            dBt[n] += dtv * xv * g[n];
            gB += g[n] * (double)Bt[n];
            gs += g[n] * sp[n];
          }
          dx[((b * L + t) * H + h) * P + p] = Dh * dyv + dtv * gB;
          ddt[(b * L + t) * H + h] += xv * gB + Ah * a * gs;
          dA_acc += dtv * a * gs;
          dD_acc += dyv * xv;
          for (int64_t n = 0; n < N; ++n) g[n] *= a;
        }
        if (dh0) {
          double* o = dh0 + ((b * H + h) * P + p) * N;
          for (int64_t n = 0; n < N; ++n) o[n] = g[n];
        }
      }
      dA_part[b * H + h] = dA_acc;
      dD_part[b * H + h] = dD_acc;
    }
    free(s);
    free(g);
  }
  return rc;
}
