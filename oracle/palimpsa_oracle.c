/*
 * Palimpsa dual-state recurrence: plain, slow float64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the bench do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (all in float64, one attention head at a time):
 *
 *   gate      alpha_t = exp(-A_h * dt_t),  1 - alpha_t = -expm1(-A_h * dt_t)
 *             ("Learning to Remember, Learn, and Forget in Attention-Based
 *             Models", slides, frame "Forgetting discounts evidence and
 *             restores the prior", Eq. (9) / App. A.2)
 *
 *   importance  I_t = alpha_t I_{t-1} + (1 - alpha_t) I_prior + beta_t (x) k_t^2
 *   content     mu_t = alpha_t (I_{t-1} / I_t) . mu_{t-1}
 *                      + (1 / I_t) . [(beta_t . v_t) (x) k_t]
 *             (same slides, frame "Palimpsa updates content and importance
 *             together", Eq. (5); squares, products and divisions are
 *             elementwise, (x) is the outer product with rows indexed by the
 *             value channel i and columns by the key channel j)
 *
 *   readout   y_t = mu_t q_t, taken after token t has been written
 *             (same slides, frame "The attention state is an online
 *             regression model", posterior-mean read)
 *
 * Layouts (row-major, all float64):
 *   q, k   [B, T, H, dk]     v, beta  [B, T, H, dv]     dt  [B, T, H]
 *   A, Ip  [H]               mu, I    [B, H, dv, dk]    y   [B, T, H, dv]
 *
 * Heads (b, h) are independent; they are the only thing spread over OpenMP
 * threads.  Inside a head the loop is the sequential definition, token by
 * token, with no blocking, fusion or reordering.
 */
#include <math.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One token for one head: Eq. (5) applied in place, then the readout. */
static void oracle_token(int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *beta, double dt, double A, double Ip,
                         double *mu, double *I, double *y)
{
    const double a = exp(-A * dt);
    const double oma = -expm1(-A * dt);
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            const size_t e = (size_t)i * dk + j;
            const double I_old = I[e];
            const double I_new = a * I_old + oma * Ip + beta[i] * (k[j] * k[j]);
            const double write = (beta[i] * v[i]) * k[j];
            mu[e] = a * (I_old / I_new) * mu[e] + write / I_new;
            I[e] = I_new;
        }
    }
    for (int i = 0; i < dv; ++i) {
        double s = 0.0;
        for (int j = 0; j < dk; ++j)
            s += mu[(size_t)i * dk + j] * q[j];
        y[i] = s;
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Whole sequence for every head.  mu and I hold the initial state on entry
 * (the caller fills them with mu0 and I0) and the final state on return.
 * y receives every token's readout.
 */
void oracle_fwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *beta, const double *dt,
                const double *A, const double *Ip,
                double *mu, double *I, double *y, int nthreads)
{
    set_threads(nthreads);
    const long nheads = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nheads; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        double *mu_h = mu + (size_t)bh * dv * dk;
        double *I_h = I + (size_t)bh * dv * dk;
        for (int t = 0; t < T; ++t) {
            const size_t row = ((size_t)b * T + t) * H + h;
            oracle_token(dk, dv, q + row * dk, k + row * dk, v + row * dv,
                         beta + row * dv, dt[row], A[h], Ip[h],
                         mu_h, I_h, y + row * dv);
        }
    }
}

/*
 * One decode token for every head: the body of oracle_fwd for a single t.
 * q, k [B, H, dk]; v, beta, y [B, H, dv]; dt [B, H]; mu, I updated in place.
 */
void oracle_step(int B, int H, int dk, int dv,
                 const double *q, const double *k, const double *v,
                 const double *beta, const double *dt,
                 const double *A, const double *Ip,
                 double *mu, double *I, double *y, int nthreads)
{
    set_threads(nthreads);
    const long nheads = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < nheads; ++bh) {
        const int h = (int)(bh % H);
        oracle_token(dk, dv, q + (size_t)bh * dk, k + (size_t)bh * dk,
                     v + (size_t)bh * dv, beta + (size_t)bh * dv, dt[bh],
                     A[h], Ip[h], mu + (size_t)bh * dv * dk,
                     I + (size_t)bh * dv * dk, y + (size_t)bh * dv);
    }
}
