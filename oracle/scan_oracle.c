/*
 * scan_oracle.c -- plain, slow fp64 CPU oracle of the selective (S6) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The product path
 * (the HIP library) shares no code, header, table or helper with it.
 *
 * Sources (web pages; cited by title and section):
 *   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block
 *          （面向医学图像分割的基础铺垫）" (eutaboo.com)
 *   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
 *   [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
 *   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
 *
 * What is computed, per batch b, channel d and scan direction k (everything in
 * double precision; bf16 inputs are widened from the same bit patterns the GPU
 * reads):
 *   x      = delta[b,k,t,d] + delta_bias[k,d]                  [MFS §4.1, Algorithm 2: Δ ← τΔ(Parameter + sΔ(x))]
 *   Δ      = softplus(x) (or x when softplus is off)           [MUN §4, discretisation: Δ = softplus(·)]
 *   Ā      = exp(Δ·A[k,d,n])                                    [MFS §6.2 Step 4, eq (4); VIM §1, ZOH]
 *   B̄·u    = Δ·B[b,k,t,n]·u  (simplified ZOH)                  [MUN §4: B̄ ≈ ΔB]
 *            or ((Ā−1)/A)·B·u when exact_zoh is set            [MFS eq (4) for a diagonal A]
 *   h[n]   = Ā·h[n] + B̄·u                                      [MFS §2.2 eq (2a); §5 scalar form h_t = a_t h_{t-1} + b_t]
 *   y      = Σ_n C[b,k,t,n]·h[n] + D[k,d]·u                    [MFS eq (2b); MUN §4 y = Ch + Dx]
 *   acc[t] += y, summed over directions k = 0,1,... in order   [VIM §2.2 VimBlock: y_forward + y_backward;
 *                                                               S4M §3 SS2D: four scan directions]
 *   out[t] = acc[t]·silu(z[b,t,d]) (or acc[t] if z is absent)  [MFS §6.2 Step 6: SSM(u) ⊙ φ(v), φ = SiLU]
 *   last_state[b,k,d,:] = h after the last step of direction k's scan.
 *
 * Scan orders (token index t for scan position p, L = seqlen):
 *   forward t = p; reversed t = L-1-p; bidirectional k=0 forward, k=1 reversed;
 *   2-D cross scan over an H×W grid with token t = row·W + col:
 *     k=0 row-major, k=1 column-major (t = (p mod H)·W + p div H),
 *     k=2 row-major reversed, k=3 column-major reversed.
 * Readings where the pages are silent (h starts at 0; y_t reads h after the
 * update; the gate multiplies the direction sum) are the plainest ones that
 * agree with the equations above.
 *
 * Work is split over (b, d) rows; every row is computed by one thread in a
 * fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t batch, dim, seqlen, dstate; /* B, D, L, N */
  int64_t height, width;              /* cross scan only: seqlen == height*width */
  int32_t dtype;                      /* 0: float32 values; 1: bfloat16 bit patterns (uint16) */
  int32_t dir_mode;                   /* 0 forward, 1 reversed, 2 bidirectional, 3 cross scan */
  int32_t delta_softplus;             /* 1: Δ = softplus(x); 0: Δ = x */
  int32_t exact_zoh;                  /* 1: B̄ = (Ā−1)/A·B; 0: B̄ = Δ·B */
} oracle_dims;

typedef struct {
  const void *u, *delta, *B, *C, *z; /* z may be NULL */
  const float *A, *D, *delta_bias;   /* D, delta_bias may be NULL */
  const float *initial_state;        /* [B][K][D][N] or NULL (zeros) */
} oracle_inputs;

/* Number of scan directions K for a direction mode. */
int oracle_num_dirs(int dir_mode) {
  switch (dir_mode) {
    case 0: case 1: return 1;
    case 2: return 2;
    case 3: return 4;
    default: return 0;
  }
}

/* Decode element i of an input array as double. */
static double ld(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* softplus(x) = log(1 + e^x), evaluated as max(x,0) + log1p(e^{-|x|}). */
double oracle_softplus(double x) {
  return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* silu(z) = z·σ(z) = z / (1 + e^{-z}). */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Token index visited at scan position p by direction k. */
int64_t oracle_token(const oracle_dims* g, int k, int64_t p) {
  const int64_t L = g->seqlen;
  switch (g->dir_mode) {
    case 0: return p;
    case 1: return L - 1 - p;
    case 2: return k == 0 ? p : L - 1 - p;
    case 3: {
      const int64_t q = (k >= 2) ? L - 1 - p : p;
      if (k == 0 || k == 2) return q;
      return (q % g->height) * g->width + q / g->height;
    }
    default: return -1;
  }
}

/* One (b, d) row over all directions.  out_row[t] (token order, L values),
 * state_row[k*N + n] (K*N values). acc is scratch of L doubles, h of N. */
static void scan_row(const oracle_dims* g, const oracle_inputs* in, int64_t b, int64_t d,
                     double* out_row, double* state_row, double* acc, double* h) {
  const int64_t L = g->seqlen, N = g->dstate, Dm = g->dim;
  const int K = oracle_num_dirs(g->dir_mode);
  const int Ku = (g->dir_mode == 3) ? 1 : K; /* u is shared by the four cross-scan directions */
  for (int64_t t = 0; t < L; ++t) acc[t] = 0.0;
  for (int k = 0; k < K; ++k) {
    for (int64_t n = 0; n < N; ++n)
      h[n] = in->initial_state ? (double)in->initial_state[((b * K + k) * Dm + d) * N + n] : 0.0;
    const double bias = in->delta_bias ? (double)in->delta_bias[k * Dm + d] : 0.0;
    const double Dk = in->D ? (double)in->D[k * Dm + d] : 0.0;
    const int ku = (Ku == 1) ? 0 : k;
    for (int64_t p = 0; p < L; ++p) {
      const int64_t t = oracle_token(g, k, p);
      const double x = ld(in->delta, g->dtype, ((b * K + k) * L + t) * Dm + d) + bias;
      const double dt = g->delta_softplus ? oracle_softplus(x) : x;
      const double v = ld(in->u, g->dtype, ((b * Ku + ku) * L + t) * Dm + d);
      const int64_t bc = ((b * K + k) * L + t) * N; /* B, C row of this token */
      double y = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double An = (double)in->A[(k * Dm + d) * N + n];
        const double abar = exp(dt * An);
        const double Bn = ld(in->B, g->dtype, bc + n);
        double bbar_u;
        if (g->exact_zoh && An != 0.0)
          bbar_u = ((abar - 1.0) / An) * Bn * v;
        else
          bbar_u = dt * Bn * v;
        h[n] = abar * h[n] + bbar_u;
      }
      for (int64_t n = 0; n < N; ++n) y += ld(in->C, g->dtype, bc + n) * h[n];
      y += Dk * v;
      acc[t] += y;
    }
    for (int64_t n = 0; n < N; ++n) state_row[k * N + n] = h[n];
  }
  for (int64_t t = 0; t < L; ++t) {
    double o = acc[t];
    if (in->z) o *= oracle_silu(ld(in->z, g->dtype, (b * L + t) * Dm + d));
    out_row[t] = o;
  }
}

typedef struct {
  const oracle_dims* g;
  const oracle_inputs* in;
  const int64_t *rows_b, *rows_d;
  int64_t nrows, first, stride;
  double *out_rows, *state_rows;
  int err;
} worker_arg;

static void* worker(void* p) {
  worker_arg* a = (worker_arg*)p;
  const int64_t L = a->g->seqlen, N = a->g->dstate;
  const int K = oracle_num_dirs(a->g->dir_mode);
  double* acc = (double*)malloc(sizeof(double) * (size_t)L);
  double* h = (double*)malloc(sizeof(double) * (size_t)N);
  if (!acc || !h) { a->err = 1; free(acc); free(h); return NULL; }
  for (int64_t r = a->first; r < a->nrows; r += a->stride)
    scan_row(a->g, a->in, a->rows_b[r], a->rows_d[r], a->out_rows + r * L,
             a->state_rows + r * K * N, acc, h);
  free(acc);
  free(h);
  return NULL;
}

/*
 * Computes the requested (b, d) rows.
 *   out_rows   [nrows][L]    output in token order
 *   state_rows [nrows][K][N] final state of each direction
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_scan_rows(const oracle_dims* g, const oracle_inputs* in, const int64_t* rows_b,
                     const int64_t* rows_d, int64_t nrows, double* out_rows, double* state_rows,
                     int nthreads) {
  if (!g || !in || !in->u || !in->delta || !in->A || !in->B || !in->C) return -1;
  if (g->batch <= 0 || g->dim <= 0 || g->seqlen <= 0 || g->dstate <= 0) return -1;
  if (oracle_num_dirs(g->dir_mode) == 0) return -1;
  if (g->dir_mode == 3 && (g->height <= 0 || g->width <= 0 || g->height * g->width != g->seqlen))
    return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows_b[r] < 0 || rows_b[r] >= g->batch || rows_d[r] < 0 || rows_d[r] >= g->dim) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  worker_arg* args = (worker_arg*)malloc(sizeof(worker_arg) * (size_t)nthreads);
  if (!th || !args) { free(th); free(args); return -2; }
  int err = 0;
  for (int i = 0; i < nthreads; ++i) {
    args[i] = (worker_arg){g, in, rows_b, rows_d, nrows, i, nthreads, out_rows, state_rows, 0};
    if (nthreads == 1) worker(&args[i]);
    else if (pthread_create(&th[i], NULL, worker, &args[i]) != 0) { worker(&args[i]); th[i] = 0; }
  }
  if (nthreads > 1)
    for (int i = 0; i < nthreads; ++i)
      if (th[i]) pthread_join(th[i], NULL);
  for (int i = 0; i < nthreads; ++i) err |= args[i].err;
  free(th);
  free(args);
  return err ? -2 : 0;
}

/*
 * One recurrent (decode) step of a forward scan for every (b, d)
 * [MFS §2.3: the recurrent form updates one token at a time].
 *   state [B][D][N] (double, in/out), u_t/delta_t/z_t [B][D], B_t/C_t [B][N],
 *   A [D][N], D/delta_bias [D]; out [B][D].
 */
int oracle_scan_step(const oracle_dims* g, double* state, const void* u_t, const void* delta_t,
                     const float* A, const void* B_t, const void* C_t, const float* D,
                     const void* z_t, const float* delta_bias, double* out) {
  if (!g || !state || !u_t || !delta_t || !A || !B_t || !C_t || !out) return -1;
  const int64_t Bn = g->batch, Dm = g->dim, N = g->dstate;
  for (int64_t b = 0; b < Bn; ++b)
    for (int64_t d = 0; d < Dm; ++d) {
      double* h = state + (b * Dm + d) * N;
      const double x = ld(delta_t, g->dtype, b * Dm + d) + (delta_bias ? (double)delta_bias[d] : 0.0);
      const double dt = g->delta_softplus ? oracle_softplus(x) : x;
      const double v = ld(u_t, g->dtype, b * Dm + d);
      double y = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double An = (double)A[d * N + n];
        const double abar = exp(dt * An);
        const double Bv = ld(B_t, g->dtype, b * N + n);
        const double bbar_u = (g->exact_zoh && An != 0.0) ? ((abar - 1.0) / An) * Bv * v : dt * Bv * v;
        h[n] = abar * h[n] + bbar_u;
      }
      for (int64_t n = 0; n < N; ++n) y += ld(C_t, g->dtype, b * N + n) * h[n];
      y += (D ? (double)D[d] : 0.0) * v;
      if (z_t) y *= oracle_silu(ld(z_t, g->dtype, b * Dm + d));
      out[b * Dm + d] = y;
    }
  return 0;
}

/*
 * Gradients of the forward scan, by reverse-mode differentiation in fp64.
 * For a loss L = Σ dout·out (dout = dL/dout, [B][L][D]) it returns dL/d of
 * every input.  The pages run the backward pass of the fused kernel by
 * recomputing the states [MFS §5; S4M §2.3]; here every state is simply
 * recomputed in full.  Per direction k, batch b, channel d and state n, with
 * scan position p visiting token t and h_{-1} the initial state:
 *   y_all[t] = Σ_k y_k[t];  g = silu(z);  dy = dout·g;  dz = dout·y_all·silu'(z)
 *   λ_p = C_t[n]·dy_t + Ā_{p+1}·λ_{p+1}  (λ_L = 0)   -- the adjoint of h_p
 *   dL/dĀ_p = λ_p·h_{p-1},  dL/d(B̄u)_p = λ_p
 *   Ā = e^{ΔA}; simplified rule B̄u = Δ·B·u; exact rule B̄u = c·B·u with
 *     c = (Ā - 1)/A, dc/dΔ = Ā, dc/dA = (Δ·Ā - c)/A  (c = Δ, dc/dA = Δ²/2 at A = 0)
 *   dΔ_p += λ h_{p-1} A Ā + λ (dc/dΔ or 1)·B·u;  dA += λ h_{p-1} Δ Ā (+ λ (dc/dA) B u, exact)
 *   dB_t += λ·(c or Δ)·u;  du_t += λ·(c or Δ)·B;  dC_t += dy_t·h_p
 *   du_t += D·dy_t;  dD += dy_t·u_t
 *   dx = dΔ·σ(x) with softplus (dx = dΔ without);  ddelta = dx;  ddelta_bias += dx
 *   dinit = Ā_0·λ_0
 * Outputs (double, zeroed here): du [B][Ku][L][D], ddelta [B][K][L][D],
 * dA [K][D][N], dB, dC [B][K][L][N], dD [K][D], dz [B][L][D] (may be NULL when
 * z is NULL), ddelta_bias [K][D], dinit [B][K][D][N].
 * Returns 0, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_scan_bwd(const oracle_dims* g, const oracle_inputs* in, const void* dout, double* du, double* ddelta,
                    double* dA, double* dB, double* dC, double* dD, double* dz, double* ddelta_bias, double* dinit) {
  if (!g || !in || !in->u || !in->delta || !in->A || !in->B || !in->C || !dout) return -1;
  if (!du || !ddelta || !dA || !dB || !dC || !dD || !ddelta_bias || !dinit || (in->z && !dz)) return -1;
  if (g->batch <= 0 || g->dim <= 0 || g->seqlen <= 0 || g->dstate <= 0) return -1;
  const int K = oracle_num_dirs(g->dir_mode);
  if (K == 0) return -1;
  if (g->dir_mode == 3 && (g->height <= 0 || g->width <= 0 || g->height * g->width != g->seqlen)) return -1;
  const int64_t Bn = g->batch, L = g->seqlen, Dm = g->dim, N = g->dstate;
  const int Ku = (g->dir_mode == 3) ? 1 : K;
  memset(du, 0, sizeof(double) * (size_t)(Bn * Ku * L * Dm));
  memset(ddelta, 0, sizeof(double) * (size_t)(Bn * K * L * Dm));
  memset(dA, 0, sizeof(double) * (size_t)(K * Dm * N));
  memset(dB, 0, sizeof(double) * (size_t)(Bn * K * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(Bn * K * L * N));
  memset(dD, 0, sizeof(double) * (size_t)(K * Dm));
  if (dz) memset(dz, 0, sizeof(double) * (size_t)(Bn * L * Dm));
  memset(ddelta_bias, 0, sizeof(double) * (size_t)(K * Dm));
  memset(dinit, 0, sizeof(double) * (size_t)(Bn * K * Dm * N));
  /* per row: states h[p][n] after step p, decays a[p][n], Δ, x and u per position */
  double* hs = (double*)malloc(sizeof(double) * (size_t)(K * L * N));
  double* as = (double*)malloc(sizeof(double) * (size_t)(K * L * N));
  double* dts = (double*)malloc(sizeof(double) * (size_t)(K * L));
  double* xs = (double*)malloc(sizeof(double) * (size_t)(K * L));
  double* vs = (double*)malloc(sizeof(double) * (size_t)(K * L));
  double* yall = (double*)malloc(sizeof(double) * (size_t)L);
  double* dy = (double*)malloc(sizeof(double) * (size_t)L);
  double* lam = (double*)malloc(sizeof(double) * (size_t)N);
  double* h0 = (double*)malloc(sizeof(double) * (size_t)N);
  if (!hs || !as || !dts || !xs || !vs || !yall || !dy || !lam || !h0) {
    free(hs); free(as); free(dts); free(xs); free(vs); free(yall); free(dy); free(lam); free(h0);
    return -2;
  }
  for (int64_t b = 0; b < Bn; ++b) {
    for (int64_t d = 0; d < Dm; ++d) {
      /* forward, keeping every state */
      for (int64_t t = 0; t < L; ++t) yall[t] = 0.0;
      for (int k = 0; k < K; ++k) {
        const int ku = (Ku == 1) ? 0 : k;
        const double bias = in->delta_bias ? (double)in->delta_bias[k * Dm + d] : 0.0;
        const double Dk = in->D ? (double)in->D[k * Dm + d] : 0.0;
        for (int64_t n = 0; n < N; ++n)
          h0[n] = in->initial_state ? (double)in->initial_state[((b * K + k) * Dm + d) * N + n] : 0.0;
        for (int64_t p = 0; p < L; ++p) {
          const int64_t t = oracle_token(g, k, p);
          const double x = ld(in->delta, g->dtype, ((b * K + k) * L + t) * Dm + d) + bias;
          const double dt = g->delta_softplus ? oracle_softplus(x) : x;
          const double v = ld(in->u, g->dtype, ((b * Ku + ku) * L + t) * Dm + d);
          xs[k * L + p] = x;
          dts[k * L + p] = dt;
          vs[k * L + p] = v;
          const int64_t bc = ((b * K + k) * L + t) * N;
          double y = Dk * v;
          for (int64_t n = 0; n < N; ++n) {
            const double An = (double)in->A[(k * Dm + d) * N + n];
            const double a = exp(dt * An);
            const double c = (g->exact_zoh && An != 0.0) ? (a - 1.0) / An : dt;
            const double hp = p > 0 ? hs[(k * L + p - 1) * N + n] : h0[n];
            const double hn = a * hp + c * ld(in->B, g->dtype, bc + n) * v;
            as[(k * L + p) * N + n] = a;
            hs[(k * L + p) * N + n] = hn;
            y += ld(in->C, g->dtype, bc + n) * hn;
          }
          yall[t] += y;
        }
      }
      /* gate */
      for (int64_t t = 0; t < L; ++t) {
        const double go = ld(dout, g->dtype, (b * L + t) * Dm + d);
        if (in->z) {
          const double zz = ld(in->z, g->dtype, (b * L + t) * Dm + d);
          const double sg = 1.0 / (1.0 + exp(-zz));
          dy[t] = go * zz * sg;
          dz[(b * L + t) * Dm + d] = go * yall[t] * sg * (1.0 + zz * (1.0 - sg));
        } else {
          dy[t] = go;
        }
      }
      /* reverse pass of each direction */
      for (int k = 0; k < K; ++k) {
        const int ku = (Ku == 1) ? 0 : k;
        const double Dk = in->D ? (double)in->D[k * Dm + d] : 0.0;
        for (int64_t n = 0; n < N; ++n) lam[n] = 0.0;
        for (int64_t n = 0; n < N; ++n)
          h0[n] = in->initial_state ? (double)in->initial_state[((b * K + k) * Dm + d) * N + n] : 0.0;
        for (int64_t p = L - 1; p >= 0; --p) {
          const int64_t t = oracle_token(g, k, p);
          const double dt = dts[k * L + p], v = vs[k * L + p], x = xs[k * L + p];
          const int64_t bc = ((b * K + k) * L + t) * N;
          double ddt = 0.0, duv = Dk * dy[t];
          dD[k * Dm + d] += dy[t] * v;
          for (int64_t n = 0; n < N; ++n) {
            const double An = (double)in->A[(k * Dm + d) * N + n];
            const double a = as[(k * L + p) * N + n];
            const double hp = p > 0 ? hs[(k * L + p - 1) * N + n] : h0[n];
            const double Bv = ld(in->B, g->dtype, bc + n);
            const double Cv = ld(in->C, g->dtype, bc + n);
            const double l = Cv * dy[t] + lam[n]; /* lam[n] holds Ā_{p+1}·λ_{p+1} */
            const int exact = g->exact_zoh;
            const double c = (exact && An != 0.0) ? (a - 1.0) / An : dt;
            const double dc_ddt = exact ? a : 1.0;
            const double dc_dA = !exact ? 0.0 : (An != 0.0 ? (dt * a - c) / An : 0.5 * dt * dt);
            ddt += l * hp * An * a + l * dc_ddt * Bv * v;
            dA[(k * Dm + d) * N + n] += l * hp * dt * a + l * dc_dA * Bv * v;
            dB[bc + n] += l * c * v;
            dC[bc + n] += dy[t] * hs[(k * L + p) * N + n];
            duv += l * c * Bv;
            lam[n] = a * l;
          }
          du[((b * Ku + ku) * L + t) * Dm + d] += duv;
          const double dx = g->delta_softplus ? ddt / (1.0 + exp(-x)) : ddt;
          ddelta[((b * K + k) * L + t) * Dm + d] = dx;
          ddelta_bias[k * Dm + d] += dx;
        }
        for (int64_t n = 0; n < N; ++n) dinit[((b * K + k) * Dm + d) * N + n] = lam[n];
      }
    }
  }
  free(hs); free(as); free(dts); free(xs); free(vs); free(yall); free(dy); free(lam); free(h0);
  return 0;
}
