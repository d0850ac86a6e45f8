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
 * Options (the `opts` bit mask of every entry point):
 *   ORACLE_PRIOR_PER_ENTRY (2): Ip is [H, dv, dk], one prior precision per
 *       state entry instead of one per head (the reading notes' table of
 *       symbols allows a prior of the state's shape, broadcast from a scalar);
 *       the prior term is (1 - alpha) Ip[h, i, j].
 *   ORACLE_VSTAR (1): v holds v* = beta . v, the write itself (the slides'
 *       frame on the Mamba2 limit makes v* the kernel input); beta still
 *       scales k^2 in the importance.
 *
 *   backward  oracle_bwd: the reverse-mode derivative of all of the above
 *             for L = sum(gy . y) + sum(gmuT . mu_T) + sum(gIT . I_T), taken
 *             term by term of the same expressions (the pages print no
 *             backward; this is plain calculus on Eq. (5) and Eq. (9))
 *
 * Heads (b, h) are independent; they are the only thing spread over OpenMP
 * threads.  Inside a head the loop is the sequential definition, token by
 * token, with no blocking, fusion or reordering.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VSTAR 1
#define ORACLE_PRIOR_PER_ENTRY 2

/* One token for one head: Eq. (5) applied in place, then the readout.
 * Ip points at the head's prior: one value, or dv * dk values. */
static void oracle_token(int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *beta, double dt, double A, const double *Ip,
                         double *mu, double *I, double *y, int opts)
{
    const double a = exp(-A * dt);
    const double oma = -expm1(-A * dt);
    const int per_entry = (opts & ORACLE_PRIOR_PER_ENTRY) != 0;
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            const size_t e = (size_t)i * dk + j;
            const double I_old = I[e];
            const double prior = per_entry ? Ip[e] : Ip[0];
            const double I_new = a * I_old + oma * prior + beta[i] * (k[j] * k[j]);
            const double wv = (opts & ORACLE_VSTAR) ? v[i] : beta[i] * v[i];
            const double write = wv * k[j];
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

/* Threads of the OpenMP runtime's own default, taken before any call sets
 * them; nthreads <= 0 means that default, whatever an earlier call asked for. */
static int default_threads = 0;

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (default_threads == 0)
        default_threads = omp_get_max_threads();
    omp_set_num_threads(nthreads > 0 ? nthreads : default_threads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    if (default_threads == 0)
        default_threads = omp_get_max_threads();
    return default_threads;
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
                double *mu, double *I, double *y, int opts, int nthreads)
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
                         beta + row * dv, dt[row], A[h],
                         Ip + ((opts & ORACLE_PRIOR_PER_ENTRY) ? (size_t)h * dv * dk : (size_t)h),
                         mu_h, I_h, y + row * dv, opts);
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
                 double *mu, double *I, double *y, int opts, int nthreads)
{
    set_threads(nthreads);
    const long nheads = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < nheads; ++bh) {
        const int h = (int)(bh % H);
        oracle_token(dk, dv, q + (size_t)bh * dk, k + (size_t)bh * dk,
                     v + (size_t)bh * dv, beta + (size_t)bh * dv, dt[bh], A[h],
                     Ip + ((opts & ORACLE_PRIOR_PER_ENTRY) ? (size_t)h * dv * dk : (size_t)h),
                     mu + (size_t)bh * dv * dk, I + (size_t)bh * dv * dk, y + (size_t)bh * dv, opts);
    }
}

/*
 * ---------------------------------------------------------------------------
 * Backward: reverse-mode derivative of oracle_fwd.
 * ---------------------------------------------------------------------------
 *
 * The pages train through the recurrence but print no backward equations.
 * This is the vector-Jacobian product of the forward above, written for the
 * scalar
 *     L = sum(gy . y) + sum(gmuT . mu_T) + sum(gIT . I_T),
 * by differentiating Eq. (5) exactly as oracle_token evaluates it:
 *     I_new  = a I_old + oma Ip + beta_i k_j^2
 *     mu_new = a (I_old / I_new) mu_old + w / I_new,   w = (beta_i v_i) k_j
 *     y_i    = sum_j mu_new q_j
 * with a = exp(-A dt) and oma = -expm1(-A dt), so d a / d dt = -A a and
 * d oma / d dt = A a (and likewise for A with dt in place of A).
 */

/*
 * One token in reverse.  (mo, Io) is the state before the token and
 * (mn, In) after it.  On entry gm, gI hold dL/d(mn, In) from the later
 * tokens (and the final-state terms); on return they hold dL/d(mo, Io).
 * Writes the token's gq [dk], gk [dk], gv [dv], gbeta [dv], *gdt, and adds
 * its terms of dL/dA and dL/dIp to *gA, *gIp.
 */
static void oracle_token_bwd(int dk, int dv,
                             const double *q, const double *k, const double *v,
                             const double *beta, double dt, double A, const double *Ip,
                             const double *mo, const double *Io,
                             const double *mn, const double *In,
                             const double *gy, double *gm, double *gI,
                             double *gq, double *gk, double *gv, double *gbeta,
                             double *gdt, double *gA, double *gIp, int opts)
{
    const double a = exp(-A * dt);
    const double oma = -expm1(-A * dt);
    const int per_entry = (opts & ORACLE_PRIOR_PER_ENTRY) != 0;
    const int vstar = (opts & ORACLE_VSTAR) != 0;
    double ga = 0.0, goma = 0.0, gip = 0.0;
    for (int j = 0; j < dk; ++j) { gq[j] = 0.0; gk[j] = 0.0; }
    for (int i = 0; i < dv; ++i) {
        const double bv = vstar ? v[i] : beta[i] * v[i];
        double g_w_sum = 0.0;     /* sum_j dL/dw_ij k_j  -> d(beta_i v_i) */
        double g_b_sum = 0.0;     /* sum_j dL/dI_new_ij k_j^2 -> beta_i via k^2 term */
        for (int j = 0; j < dk; ++j) {
            const size_t e = (size_t)i * dk + j;
            /* readout */
            gq[j] += gy[i] * mn[e];
            const double g_mn = gm[e] + gy[i] * q[j];
            /* mu_new = a (I_old / I_new) mu_old + w / I_new */
            const double g_mo = g_mn * a * (Io[e] / In[e]);
            double g_Io = g_mn * a * mo[e] / In[e];
            const double g_In = gI[e] - g_mn * mn[e] / In[e];
            ga += g_mn * (Io[e] / In[e]) * mo[e];
            const double g_w = g_mn / In[e];
            g_w_sum += g_w * k[j];
            gk[j] += g_w * bv;
            /* I_new = a I_old + oma Ip + beta_i k_j^2 */
            const double prior = per_entry ? Ip[e] : Ip[0];
            g_Io += g_In * a;
            ga += g_In * Io[e];
            goma += g_In * prior;
            if (per_entry)
                gIp[e] += g_In * oma;
            else
                gip += g_In * oma;
            g_b_sum += g_In * (k[j] * k[j]);
            gk[j] += g_In * 2.0 * beta[i] * k[j];
            gm[e] = g_mo;
            gI[e] = g_Io;
        }
        /* the write is (beta_i v_i) k_j, or v*_i k_j */
        gv[i] = vstar ? g_w_sum : g_w_sum * beta[i];
        gbeta[i] = vstar ? g_b_sum : g_w_sum * v[i] + g_b_sum;
    }
    *gdt = A * a * (goma - ga);
    *gA += dt * a * (goma - ga);
    if (!per_entry)
        *gIp += gip;
}

/*
 * Whole-sequence backward for every head.
 *   inputs as oracle_fwd; mu0, I0 [B, H, dv, dk] hold the initial state;
 *   gy [B, T, H, dv]; gmuT, gIT [B, H, dv, dk] (NULL: zero).
 * Outputs: gq, gk [B, T, H, dk]; gv, gbeta [B, T, H, dv]; gdt [B, T, H];
 *   gA_bh [B, H] and gIp_bh [B, H] or, with a per-entry prior,
 *   [B, H, dv, dk] (per sequence; the caller sums over b);
 *   gmu0, gI0 [B, H, dv, dk].
 * States are needed newest first.  The forward pass keeps the state at the
 * start of every segment of `seg` tokens; each segment is then replayed with
 * oracle_token, keeping all its states, and differentiated token by token in
 * reverse.
 */
void oracle_bwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *beta, const double *dt,
                const double *A, const double *Ip,
                const double *mu0, const double *I0,
                const double *gy, const double *gmuT, const double *gIT,
                double *gq, double *gk, double *gv, double *gbeta, double *gdt,
                double *gA_bh, double *gIp_bh, double *gmu0, double *gI0,
                int opts, int nthreads)
{
    set_threads(nthreads);
    const long nheads = (long)B * H;
    const size_t S = (size_t)dv * dk;
    int seg = 1;
    while ((long)seg * seg < T) ++seg;
    const int nseg = T > 0 ? (T + seg - 1) / seg : 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nheads; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        double *ck_mu = malloc(sizeof(double) * S * (size_t)(nseg > 0 ? nseg : 1));
        double *ck_I = malloc(sizeof(double) * S * (size_t)(nseg > 0 ? nseg : 1));
        double *st_mu = malloc(sizeof(double) * S * (size_t)(seg + 1));
        double *st_I = malloc(sizeof(double) * S * (size_t)(seg + 1));
        double *mu = malloc(sizeof(double) * S), *I = malloc(sizeof(double) * S);
        double *ysc = malloc(sizeof(double) * (size_t)dv);
        double *gm = gmu0 + (size_t)bh * S, *gI = gI0 + (size_t)bh * S;
        const int per_entry = (opts & ORACLE_PRIOR_PER_ENTRY) != 0;
        const double *Ip_h = Ip + (per_entry ? (size_t)h * S : (size_t)h);
        if (per_entry)
            for (size_t e = 0; e < S; ++e) gIp_bh[(size_t)bh * S + e] = 0.0;
        for (size_t e = 0; e < S; ++e) {
            mu[e] = mu0[(size_t)bh * S + e];
            I[e] = I0[(size_t)bh * S + e];
        }
        /* forward, keeping segment starts */
        for (int t = 0; t < T; ++t) {
            if (t % seg == 0) {
                for (size_t e = 0; e < S; ++e) {
                    ck_mu[(size_t)(t / seg) * S + e] = mu[e];
                    ck_I[(size_t)(t / seg) * S + e] = I[e];
                }
            }
            const size_t row = ((size_t)b * T + t) * H + h;
            oracle_token(dk, dv, q + row * dk, k + row * dk, v + row * dv,
                         beta + row * dv, dt[row], A[h], Ip_h, mu, I, ysc, opts);
        }
        /* adjoint of the final state */
        for (size_t e = 0; e < S; ++e) {
            gm[e] = gmuT ? gmuT[(size_t)bh * S + e] : 0.0;
            gI[e] = gIT ? gIT[(size_t)bh * S + e] : 0.0;
        }
        double gA_acc = 0.0, gIp_acc = 0.0;
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const int t0 = sg * seg;
            const int len = (t0 + seg <= T) ? seg : T - t0;
            for (size_t e = 0; e < S; ++e) {
                st_mu[e] = ck_mu[(size_t)sg * S + e];
                st_I[e] = ck_I[(size_t)sg * S + e];
            }
            for (int u = 0; u < len; ++u) {
                const size_t row = ((size_t)b * T + t0 + u) * H + h;
                double *nm = st_mu + (size_t)(u + 1) * S, *nI = st_I + (size_t)(u + 1) * S;
                for (size_t e = 0; e < S; ++e) { nm[e] = st_mu[(size_t)u * S + e]; nI[e] = st_I[(size_t)u * S + e]; }
                oracle_token(dk, dv, q + row * dk, k + row * dk, v + row * dv,
                             beta + row * dv, dt[row], A[h], Ip_h, nm, nI, ysc, opts);
            }
            for (int u = len - 1; u >= 0; --u) {
                const size_t row = ((size_t)b * T + t0 + u) * H + h;
                oracle_token_bwd(dk, dv, q + row * dk, k + row * dk, v + row * dv,
                                 beta + row * dv, dt[row], A[h], Ip_h,
                                 st_mu + (size_t)u * S, st_I + (size_t)u * S,
                                 st_mu + (size_t)(u + 1) * S, st_I + (size_t)(u + 1) * S,
                                 gy + row * dv, gm, gI,
                                 gq + row * dk, gk + row * dk, gv + row * dv,
                                 gbeta + row * dv, gdt + row, &gA_acc,
                                 per_entry ? gIp_bh + (size_t)bh * S : &gIp_acc, opts);
            }
        }
        gA_bh[bh] = gA_acc;
        if (!per_entry)
            gIp_bh[bh] = gIp_acc;
        free(ck_mu); free(ck_I); free(st_mu); free(st_I); free(mu); free(I); free(ysc);
    }
}
