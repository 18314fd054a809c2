/*
 * cfc_oracle.c -- plain, slow, float64 CPU oracle for the CfC K-loop.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP
 * library; it is written from the definitions alone, in the order the pages
 * give the steps, with no blocking, fusion or reordering.
 *
 * What it computes (per batch row b, rows fully independent, as in the
 * block-per-batch design of the "K-loop Parallelization Implementation Plan",
 * Tasks 2 and 3):
 *
 *   cell (this library's gated CfC cell; the pages fix the loop structure,
 *   buffers and invariants, the gate is a softplus rate instead of the pages'
 *   tau-decay):
 *     a      = W_in x_k + W_rec h_k + bias
 *     sp     = softplus(w_tau)                      (per unit)
 *     g      = sigmoid(-sp * a * dt)                (elementwise)
 *     c      = tanh(a)
 *     h_k+1  = g * h_k + (1 - g) * c
 *   loss      L_b = 1/2 |h_K - y_b|^2
 *   backward  exact reverse-mode gradient of L_b, one "+=" into the per-row
 *             scratch per timestep, in descending k, after the row is zeroed
 *             ("zero once per step, K invocations accumulate": Task 3 kernel
 *             comment and Task 5 Step 3); optionally also dL/dx_k and dL/dh_0.
 *   scratch row layout  [ dW_in (H x n_in, row-major) | dW_rec (H x H) |
 *                         db (H) | dw_tau (H) ]
 *   reduce_axis0  out[j] = sum_b in[b, j], b ascending, overwrite
 *             ("K-loop Parallelization Implementation Plan", Task 1).
 *
 * A second cell, the tau-decay cell the pages print ("K-loop
 * Parallelization Implementation Plan", Task 2 forward kernel and Task 3
 * backward kernel), replaces the gate with a per-unit constant:
 *     decay  = exp(-dt / max(tau, 1e-6))           (w_tau holds tau)
 *     h_k+1  = decay * h_k + (1 - decay) * tanh(a)
 * so dL/da has no gate term, and dL/dtau = dL/ddecay * decay * dt / tau^2
 * where tau > 1e-6, zero elsewhere (the pages' guard).  Its scratch row has
 * the same layout, with dL/dtau in the last slot.
 *
 * Everything is double precision.  The caller widens the float32 inputs.
 * Return value 0 = ok, -1 = bad argument.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CELL_GATED 0
#define ORACLE_CELL_TAU_DECAY 1
#define ORACLE_TAU_EPS 1e-6

/* softplus(w) = log(1 + e^w), written in the overflow-safe form
 * log1p(e^-|w|) + max(w, 0). */
static double oracle_softplus(double w)
{
    return log1p(exp(-fabs(w))) + (w > 0.0 ? w : 0.0);
}

/* logistic sigmoid 1 / (1 + e^-z); e^-z may overflow to +inf, giving 0. */
static double oracle_sigmoid(double z)
{
    return 1.0 / (1.0 + exp(-z));
}

/* Per-unit constants of the gate, from w_tau:
 *   gated cell:     sp = softplus(w_tau) (the rate), sw = sigmoid(w_tau)
 *                   (d softplus / d w_tau);
 *   tau-decay cell: sp = exp(-dt / max(tau, eps)) (the gate itself),
 *                   sw = dt / tau^2 where tau > eps, else 0, so that
 *                   d decay / d tau = decay * sw. */
static void oracle_unit_consts(int cell, int H, double dt, const double *w_tau,
                               double *sp, double *sw)
{
    for (int i = 0; i < H; ++i) {
        if (cell == ORACLE_CELL_TAU_DECAY) {
            const double tau_eff = w_tau[i] > ORACLE_TAU_EPS ? w_tau[i] : ORACLE_TAU_EPS;
            sp[i] = exp(-dt / tau_eff);
            sw[i] = w_tau[i] > ORACLE_TAU_EPS ? dt / (tau_eff * tau_eff) : 0.0;
        } else {
            sp[i] = oracle_softplus(w_tau[i]);
            sw[i] = oracle_sigmoid(w_tau[i]);
        }
    }
}

/* One cell step for one row: given x_k [n_in] and h [H], fill a, g, c and
 * h_next (each [H]).  sp holds the per-unit constants above. */
static void oracle_cell(int cell, int n_in, int H, double dt,
                        const double *w_in, const double *w_rec,
                        const double *bias, const double *sp,
                        const double *xk, const double *h,
                        double *a, double *g, double *c, double *h_next)
{
    for (int i = 0; i < H; ++i) {
        double s = bias[i];
        for (int j = 0; j < n_in; ++j)
            s += w_in[(size_t)i * n_in + j] * xk[j];
        for (int j = 0; j < H; ++j)
            s += w_rec[(size_t)i * H + j] * h[j];
        a[i] = s;
        if (cell == ORACLE_CELL_TAU_DECAY)
            g[i] = sp[i];   /* the unit's decay, independent of a */
        else
            g[i] = oracle_sigmoid(-sp[i] * s * dt);
        c[i] = tanh(s);
        h_next[i] = g[i] * h[i] + (1.0 - g[i]) * c[i];
    }
}

long long oracle_scratch_row_len(int n_in, int H)
{
    if (n_in < 1 || H < 1)
        return -1;
    return (long long)H * ((long long)n_in + H + 2);
}

/* Forward K-loop.  x [B,K,n_in], h0 [B,H] -> h_seq [B,K,H] holding h_1..h_K.
 * cell: ORACLE_CELL_GATED or ORACLE_CELL_TAU_DECAY. */
int oracle_cfc_forward(int B, int K, int n_in, int H, double dt,
                       const double *w_in, const double *w_rec,
                       const double *bias, const double *w_tau,
                       const double *x, const double *h0, double *h_seq, int cell)
{
    if (B < 0 || K < 1 || n_in < 1 || H < 1 || (cell != ORACLE_CELL_GATED && cell != ORACLE_CELL_TAU_DECAY))
        return -1;
    double *sp = malloc(sizeof(double) * H);
    double *sw = malloc(sizeof(double) * H);
    double *a = malloc(sizeof(double) * H);
    double *g = malloc(sizeof(double) * H);
    double *c = malloc(sizeof(double) * H);
    double *h = malloc(sizeof(double) * H);
    double *hn = malloc(sizeof(double) * H);
    oracle_unit_consts(cell, H, dt, w_tau, sp, sw);
    for (int b = 0; b < B; ++b) {
        memcpy(h, h0 + (size_t)b * H, sizeof(double) * H);
        for (int k = 0; k < K; ++k) {
            const double *xk = x + ((size_t)b * K + k) * n_in;
            oracle_cell(cell, n_in, H, dt, w_in, w_rec, bias, sp, xk, h, a, g, c, hn);
            memcpy(h, hn, sizeof(double) * H);
            memcpy(h_seq + ((size_t)b * K + k) * H, h, sizeof(double) * H);
        }
    }
    free(sp); free(sw); free(a); free(g); free(c); free(h); free(hn);
    return 0;
}

/* Backward through time for L = sum_b 1/2 |h_K - y_b|^2.
 * Inputs as for the forward plus h_seq [B,K,H] and y [B,H].
 * scratch [B, N] receives each row's parameter gradient (zeroed first, then
 * one += per timestep).  loss [B] (may be NULL) receives L_b.
 * The gradients with respect to the cell's inputs -- the per-step grad_x and
 * grad_h_old outputs of the pages' backward ("K-loop Parallelization
 * Implementation Plan", Task 3 kernel signature, grad_x nullable), carried
 * through the whole K-loop -- are optional:
 *   grad_x  [B,K,n_in] (may be NULL): dL/dx_k = W_in^T da_k for every k;
 *   grad_h0 [B,H]      (may be NULL): dL/dh_0, the delta left after step 0
 *                      (each step's grad_h_old is the next step's delta, so
 *                      only step 0's leaves the loop). */
int oracle_cfc_backward_inputs(int B, int K, int n_in, int H, double dt,
                               const double *w_in, const double *w_rec,
                               const double *bias, const double *w_tau,
                               const double *x, const double *h0,
                               const double *h_seq, const double *y,
                               double *scratch, double *loss,
                               double *grad_x, double *grad_h0, int cell)
{
    if (B < 0 || K < 1 || n_in < 1 || H < 1 || (cell != ORACLE_CELL_GATED && cell != ORACLE_CELL_TAU_DECAY))
        return -1;
    const size_t N = (size_t)oracle_scratch_row_len(n_in, H);
    double *sp = malloc(sizeof(double) * H);
    double *sw = malloc(sizeof(double) * H);   /* see oracle_unit_consts */
    double *a = malloc(sizeof(double) * H);
    double *g = malloc(sizeof(double) * H);
    double *c = malloc(sizeof(double) * H);
    double *hn = malloc(sizeof(double) * H);
    double *delta = malloc(sizeof(double) * H);
    double *delta_prev = malloc(sizeof(double) * H);
    double *dz = malloc(sizeof(double) * H);
    double *da = malloc(sizeof(double) * H);
    oracle_unit_consts(cell, H, dt, w_tau, sp, sw);
    for (int b = 0; b < B; ++b) {
        double *row = scratch + (size_t)b * N;
        double *g_win = row;                                  /* [H, n_in] */
        double *g_wrec = row + (size_t)H * n_in;              /* [H, H]    */
        double *g_b = g_wrec + (size_t)H * H;                 /* [H]       */
        double *g_wtau = g_b + H;                             /* [H]       */

        /* loss seed: dL/dh_K = h_K - y */
        const double *hK = h_seq + ((size_t)b * K + (K - 1)) * H;
        double l = 0.0;
        for (int i = 0; i < H; ++i) {
            delta[i] = hK[i] - y[(size_t)b * H + i];
            l += 0.5 * delta[i] * delta[i];
        }
        if (loss)
            loss[b] = l;

        /* the per-row scratch starts at zero for this step */
        for (size_t j = 0; j < N; ++j)
            row[j] = 0.0;

        for (int k = K - 1; k >= 0; --k) {
            const double *xk = x + ((size_t)b * K + k) * n_in;
            const double *hp = (k == 0) ? h0 + (size_t)b * H
                                        : h_seq + ((size_t)b * K + (k - 1)) * H;
            /* recompute the step's pre-activation and gates from h_k */
            oracle_cell(cell, n_in, H, dt, w_in, w_rec, bias, sp, xk, hp, a, g, c, hn);
            for (int i = 0; i < H; ++i) {
                if (cell == ORACLE_CELL_TAU_DECAY) {
                    /* dL/d(decay); the gate does not depend on a */
                    dz[i] = delta[i] * (hp[i] - c[i]);
                    da[i] = delta[i] * (1.0 - g[i]) * (1.0 - c[i] * c[i]);
                } else {
                    /* dL/dz with z = -sp*a*dt the gate's argument */
                    dz[i] = delta[i] * (hp[i] - c[i]) * g[i] * (1.0 - g[i]);
                    /* dL/da through tanh and through the gate */
                    da[i] = delta[i] * (1.0 - g[i]) * (1.0 - c[i] * c[i]) - dz[i] * sp[i] * dt;
                }
            }
            for (int i = 0; i < H; ++i) {
                for (int j = 0; j < n_in; ++j)
                    g_win[(size_t)i * n_in + j] += da[i] * xk[j];
                for (int j = 0; j < H; ++j)
                    g_wrec[(size_t)i * H + j] += da[i] * hp[j];
                g_b[i] += da[i];
                if (cell == ORACLE_CELL_TAU_DECAY)
                    g_wtau[i] += dz[i] * g[i] * sw[i];   /* dL/dtau */
                else
                    g_wtau[i] += dz[i] * (-a[i] * dt) * sw[i];
            }
            /* dL/dx_k = W_in^T da */
            if (grad_x) {
                double *gx = grad_x + ((size_t)b * K + k) * n_in;
                for (int j = 0; j < n_in; ++j) {
                    double t = 0.0;
                    for (int i = 0; i < H; ++i)
                        t += w_in[(size_t)i * n_in + j] * da[i];
                    gx[j] = t;
                }
            }
            /* dL/dh_k = delta * g (direct path) + W_rec^T da */
            for (int j = 0; j < H; ++j) {
                double s = delta[j] * g[j];
                for (int i = 0; i < H; ++i)
                    s += w_rec[(size_t)i * H + j] * da[i];
                delta_prev[j] = s;
            }
            memcpy(delta, delta_prev, sizeof(double) * H);
        }
        /* after step 0, delta is dL/dh_0 */
        if (grad_h0)
            memcpy(grad_h0 + (size_t)b * H, delta, sizeof(double) * H);
    }
    free(sp); free(sw); free(a); free(g); free(c); free(hn);
    free(delta); free(delta_prev); free(dz); free(da);
    return 0;
}


/* out[j] = sum_{b=0}^{B-1} in[b, j], b ascending; B = 0 gives zeros. */
int oracle_reduce_axis0(long long B, long long N, const double *in, double *out)
{
    if (B < 0 || N < 0)
        return -1;
    for (long long j = 0; j < N; ++j)
        out[j] = 0.0;
    for (long long b = 0; b < B; ++b)
        for (long long j = 0; j < N; ++j)
            out[j] += in[b * N + j];
    return 0;
}

/* The same column sum over float32 input rows, widened to double per term.
 * Used to check a float32 scratch produced elsewhere against its own exact-ish
 * sum without materialising a double copy of the whole matrix. */
int oracle_reduce_axis0_f32(long long B, long long N, const float *in, double *out)
{
    if (B < 0 || N < 0)
        return -1;
    for (long long j = 0; j < N; ++j)
        out[j] = 0.0;
    for (long long b = 0; b < B; ++b)
        for (long long j = 0; j < N; ++j)
            out[j] += (double)in[b * N + j];
    return 0;
}
