/*
 * CPU oracle for the selective scan and its scalar-decay (SSD) variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call this code.  It shares no source,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Plain, slow, single-threaded, float64 throughout, libm exp.  Every loop is
 * the definition written out; nothing is blocked, fused or reordered.
 *
 * What is computed (page titles and sections are those of the pages that
 * define the method):
 *   - "We brought Mamba to Trainium", section "Mamba: bringing an unsupported
 *     model to the chip": the running state is updated every step,
 *     h_t = Abar_t * h_{t-1} + Bbar_t * x_t, and read out as y_t = sum_n C_t h_t.
 *   - "Mamba-3 NKI Kernels for AWS Neuron", section "How it works", Phase 0:
 *     the decay is alpha = exp(dt * A); the input weight is gamma = lam * dt,
 *     which is dt for the plain (lam = 1) form used here, so Bbar_t x_t is
 *     dt_t * B_t * x_t.
 *   - same page and section, Phase 5: the D skip is added, then the silu gate
 *     is applied: y = (C.h + D x) * silu(z), silu(z) = z / (1 + exp(-z)).
 *   - the state before the first step is h0 (zero when h0 is NULL); h_last is
 *     the state after the last step, before the readout.
 *
 * Parity of this code is pinned by the CPU tests (closed forms, brute force,
 * a hand-derived worked example, invariants); it is never compared with
 * itself.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Selective scan.
 *   u, delta, z : (batch, dim, seqlen)          y    : (batch, dim, seqlen)
 *   B, C        : (batch, ngroups, dstate, seqlen)
 *   A           : (dim, dstate)                  Dskip: (dim)         (nullable)
 *   h0, h_last  : (batch, dim, dstate)           (h0 and h_last nullable)
 * Channel d reads group g = d / (dim / ngroups).
 * Returns 0, or -1 on a bad shape.
 */
int oracle_scan_f64(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                    int64_t ngroups, const double *u, const double *delta,
                    const double *A, const double *B, const double *C,
                    const double *Dskip, const double *z, const double *h0,
                    double *y, double *h_last)
{
    if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0 || ngroups < 1 ||
        dim % ngroups != 0 || dstate > 4096)
        return -1;
    double h[4096];
    const int64_t dpg = dim / ngroups;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t g = d / dpg;
            for (int64_t n = 0; n < dstate; ++n)
                h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t i = (b * dim + d) * seqlen + t;
                const double dl = delta[i];
                const double x = u[i];
                double acc = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    const int64_t j = ((b * ngroups + g) * dstate + n) * seqlen + t;
                    const double abar = exp(dl * A[d * dstate + n]);
                    h[n] = abar * h[n] + dl * B[j] * x;
                    acc += C[j] * h[n];
                }
                if (Dskip) acc += Dskip[d] * x;
                if (z) acc *= silu(z[i]);
                y[i] = acc;
            }
            if (h_last)
                for (int64_t n = 0; n < dstate; ++n)
                    h_last[(b * dim + d) * dstate + n] = h[n];
        }
    }
    return 0;
}

/*
 * Scalar-decay (SSD) form: one decay per (batch, time, head), shared by the
 * head's headdim x dstate states.  This is the recurrence the chunked SSD of
 * "Mamba-3 NKI Kernels for AWS Neuron" (section "Kernel details",
 * mamba3_siso_ssd_kernel, Mamba-2 structure) reaches, with the trapezoidal
 * and rotary extras switched off.  It takes no chunk argument: chunking only
 * reorganises the arithmetic.
 *   x, z, y : (batch, seqlen, nheads, headdim)   dt : (batch, seqlen, nheads)
 *   B, C    : (batch, seqlen, ngroups, dstate)    A, Dskip : (nheads)
 *   h0, h_last : (batch, nheads, headdim, dstate)
 * Head h reads group g = h / (nheads / ngroups).
 */
int oracle_ssd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups, const double *x, const double *dt,
                   const double *A, const double *B, const double *C,
                   const double *Dskip, const double *z, const double *h0,
                   double *y, double *h_last)
{
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1 ||
        ngroups < 1 || nheads % ngroups != 0 || headdim * dstate > 65536)
        return -1;
    static double H[65536];
    const int64_t hpg = nheads / ngroups;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t hd = 0; hd < nheads; ++hd) {
            const int64_t g = hd / hpg;
            for (int64_t k = 0; k < headdim * dstate; ++k)
                H[k] = h0 ? h0[(b * nheads + hd) * headdim * dstate + k] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const double d = dt[(b * seqlen + t) * nheads + hd];
                const double alpha = exp(d * A[hd]);
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
                    const double xv = x[i];
                    double acc = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        double *hp = &H[p * dstate + n];
                        *hp = alpha * *hp + d * Bt[n] * xv;
                        acc += Ct[n] * *hp;
                    }
                    if (Dskip) acc += Dskip[hd] * xv;
                    if (z) acc *= silu(z[i]);
                    y[i] = acc;
                }
            }
            if (h_last)
                for (int64_t k = 0; k < headdim * dstate; ++k)
                    h_last[(b * nheads + hd) * headdim * dstate + k] = H[k];
        }
    }
    return 0;
}

/*
 * Gradients of the selective scan above (reverse mode), float64.
 *
 * For a loss with upstream gradients dy (batch, dim, seqlen) on y and dh_last
 * (batch, dim, dstate; nullable = zero) on h_last, returns the loss gradient
 * with respect to every input: du, ddelta, dz (batch, dim, seqlen; dz only
 * when z is given), dA (dim, dstate), dB, dC (batch, ngroups, dstate,
 * seqlen), dD (dim; when Dskip is given) and dh0 (batch, dim, dstate).
 *
 * The pages report that the implementations' gradients are checked against a
 * reference ("Mamba-3 NKI Kernels for AWS Neuron", section "Correctness",
 * backward parity) but print no formulas: this is the chain rule applied to
 * the forward definition, step by step.  With yhat_t = C_t.h_t + D x_t the
 * output before the gate and lambda_t = dL/dh_t, walking t backwards:
 *   dyhat_t   = dy_t silu(z_t);   dz_t = dy_t yhat_t silu'(z_t)
 *   lambda_t  = dyhat_t C_t + abar_{t+1} lambda_{t+1}   (lambda_{L-1} also
 *               receives dh_last)
 *   dC_t     += dyhat_t h_t;      dB_t += lambda_t delta_t x_t
 *   dx_t      = dyhat_t D + sum_n lambda_t delta_t B_t
 *   ddelta_t  = sum_n lambda_t (B_t x_t + A abar_t h_{t-1})
 *   dA       += lambda_t delta_t abar_t h_{t-1};   dD += dyhat_t x_t
 *   dh0       = abar_0 lambda_0
 * The forward states of one channel are recomputed and kept (seqlen + 1 rows).
 * Returns 0, -1 on a bad shape, -2 if memory runs out.
 */
#include <stdlib.h>

int oracle_scan_bwd_f64(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                        int64_t ngroups, const double *u, const double *delta,
                        const double *A, const double *B, const double *C,
                        const double *Dskip, const double *z, const double *h0,
                        const double *dy, const double *dh_last,
                        double *du, double *ddelta, double *dA, double *dB,
                        double *dC, double *dD, double *dz, double *dh0)
{
    if (batch < 0 || dim < 0 || dstate < 1 || seqlen < 0 || ngroups < 1 ||
        dim % ngroups != 0)
        return -1;
    const int64_t dpg = dim / ngroups;
    double *hs = malloc(sizeof(double) * (size_t)((seqlen + 1) * dstate));
    double *yhat = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
    double *lam = malloc(sizeof(double) * (size_t)dstate);
    if (!hs || !yhat || !lam) {
        free(hs); free(yhat); free(lam);
        return -2;
    }
    for (int64_t k = 0; k < dim * dstate; ++k) dA[k] = 0.0;
    for (int64_t k = 0; k < batch * ngroups * dstate * seqlen; ++k) {
        dB[k] = 0.0;
        dC[k] = 0.0;
    }
    if (Dskip)
        for (int64_t d = 0; d < dim; ++d) dD[d] = 0.0;

    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t g = d / dpg;
            /* forward, keeping every state: hs[t + 1] is h after step t */
            for (int64_t n = 0; n < dstate; ++n)
                hs[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t i = (b * dim + d) * seqlen + t;
                double acc = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    const int64_t j = ((b * ngroups + g) * dstate + n) * seqlen + t;
                    const double abar = exp(delta[i] * A[d * dstate + n]);
                    hs[(t + 1) * dstate + n] = abar * hs[t * dstate + n] + delta[i] * B[j] * u[i];
                    acc += C[j] * hs[(t + 1) * dstate + n];
                }
                if (Dskip) acc += Dskip[d] * u[i];
                yhat[t] = acc;
            }
            /* backward */
            for (int64_t n = 0; n < dstate; ++n)
                lam[n] = dh_last ? dh_last[(b * dim + d) * dstate + n] : 0.0;
            for (int64_t t = seqlen - 1; t >= 0; --t) {
                const int64_t i = (b * dim + d) * seqlen + t;
                const double dl = delta[i], x = u[i];
                double dyh = dy[i];
                if (z) {
                    const double s = 1.0 / (1.0 + exp(-z[i]));
                    dyh = dy[i] * z[i] * s;
                    dz[i] = dy[i] * yhat[t] * s * (1.0 + z[i] * (1.0 - s));
                }
                double dx = 0.0, ddl = 0.0;
                if (Dskip) {
                    dD[d] += dyh * x;
                    dx = dyh * Dskip[d];
                }
                for (int64_t n = 0; n < dstate; ++n) {
                    const int64_t j = ((b * ngroups + g) * dstate + n) * seqlen + t;
                    const double a = A[d * dstate + n];
                    const double abar = exp(dl * a);
                    const double hprev = hs[t * dstate + n];
                    const double l = lam[n] + dyh * C[j];
                    dC[j] += dyh * hs[(t + 1) * dstate + n];
                    dB[j] += l * dl * x;
                    dx += l * dl * B[j];
                    ddl += l * (B[j] * x + a * abar * hprev);
                    dA[d * dstate + n] += l * dl * abar * hprev;
                    lam[n] = abar * l;
                }
                du[i] = dx;
                ddelta[i] = ddl;
            }
            for (int64_t n = 0; n < dstate; ++n)
                dh0[(b * dim + d) * dstate + n] = lam[n];
        }
    }
    free(hs);
    free(yhat);
    free(lam);
    return 0;
}

/*
 * Gradients of the scalar-decay SSD above (reverse mode), float64.
 *
 * For a loss with upstream gradients dy (batch, seqlen, nheads, headdim) on y
 * and dh_last (batch, nheads, headdim, dstate; nullable = zero) on h_last,
 * returns the gradient with respect to every input: dx, dz (like x; dz only
 * with z), ddt (batch, seqlen, nheads), dA, dD (nheads; dD only with Dskip),
 * dB, dC (batch, seqlen, ngroups, dstate) and dh0 (batch, nheads, headdim,
 * dstate).  "Mamba-3 NKI Kernels for AWS Neuron", section "Correctness",
 * reports backward parity of the SSD against a reference but prints no
 * formulas: this is the chain rule on the recurrence of oracle_ssd_f64,
 * walked backwards with Lam_t = dL/dS_t (P x N):
 *   yhat_t = S_t C_t + D x_t;  dyhat_t = dy_t silu(z_t);  dz_t = dy_t yhat_t silu'(z_t)
 *   Lam_t  = dyhat_t C_t^T + alpha_{t+1} Lam_{t+1}   (Lam_{L-1} also receives dh_last)
 *   dx_t   = dt_t Lam_t B_t + D dyhat_t;   dB_t += dt_t Lam_t^T x_t;   dC_t += S_t^T dyhat_t
 *   ddt_t  = sum_{p,n} Lam_t (x_t B_t^T + A alpha_t S_{t-1});   dA += dt_t sum Lam_t alpha_t S_{t-1}
 *   dD    += dyhat_t . x_t;   dh0 = alpha_0 Lam_0
 * The forward states of one head are recomputed and kept (seqlen + 1 of them).
 * Returns 0, -1 on a bad shape, -2 if memory runs out.
 */
int oracle_ssd_bwd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, const double *x, const double *dt,
                       const double *A, const double *B, const double *C,
                       const double *Dskip, const double *z, const double *h0,
                       const double *dy, const double *dh_last,
                       double *dx, double *ddt, double *dA, double *dB, double *dC,
                       double *dD, double *dz, double *dh0)
{
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1 ||
        ngroups < 1 || nheads % ngroups != 0)
        return -1;
    const int64_t PN = headdim * dstate, hpg = nheads / ngroups;
    double *S = malloc(sizeof(double) * (size_t)((seqlen + 1) * PN));
    double *yhat = malloc(sizeof(double) * (size_t)((seqlen > 0 ? seqlen : 1) * headdim));
    double *lam = malloc(sizeof(double) * (size_t)PN);
    double *dyh = malloc(sizeof(double) * (size_t)headdim);
    if (!S || !yhat || !lam || !dyh) {
        free(S); free(yhat); free(lam); free(dyh);
        return -2;
    }
    for (int64_t k = 0; k < nheads; ++k) dA[k] = 0.0;
    if (Dskip)
        for (int64_t k = 0; k < nheads; ++k) dD[k] = 0.0;
    for (int64_t k = 0; k < batch * seqlen * ngroups * dstate; ++k) {
        dB[k] = 0.0;
        dC[k] = 0.0;
    }
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t hd = 0; hd < nheads; ++hd) {
            const int64_t g = hd / hpg;
            /* forward, keeping every state: S[t + 1] is the state after step t */
            for (int64_t k = 0; k < PN; ++k)
                S[k] = h0 ? h0[(b * nheads + hd) * PN + k] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const double d = dt[(b * seqlen + t) * nheads + hd];
                const double alpha = exp(d * A[hd]);
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
                    double acc = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const int64_t k = p * dstate + n;
                        S[(t + 1) * PN + k] = alpha * S[t * PN + k] + d * Bt[n] * x[i];
                        acc += Ct[n] * S[(t + 1) * PN + k];
                    }
                    if (Dskip) acc += Dskip[hd] * x[i];
                    yhat[t * headdim + p] = acc;
                }
            }
            /* backward */
            for (int64_t k = 0; k < PN; ++k)
                lam[k] = dh_last ? dh_last[(b * nheads + hd) * PN + k] : 0.0;
            for (int64_t t = seqlen - 1; t >= 0; --t) {
                const double d = dt[(b * seqlen + t) * nheads + hd];
                const double alpha = exp(d * A[hd]);
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                double *dBt = dB + ((b * seqlen + t) * ngroups + g) * dstate;
                double *dCt = dC + ((b * seqlen + t) * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
                    dyh[p] = dy[i];
                    if (z) {
                        const double sg = 1.0 / (1.0 + exp(-z[i]));
                        dyh[p] = dy[i] * z[i] * sg;
                        dz[i] = dy[i] * yhat[t * headdim + p] * sg * (1.0 + z[i] * (1.0 - sg));
                    }
                    if (Dskip) dD[hd] += dyh[p] * x[i];
                }
                double ddl = 0.0;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
                    double dxp = Dskip ? Dskip[hd] * dyh[p] : 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const int64_t k = p * dstate + n;
                        const double l = lam[k] + dyh[p] * Ct[n];
                        dCt[n] += S[(t + 1) * PN + k] * dyh[p];
                        dBt[n] += l * d * x[i];
                        dxp += l * d * Bt[n];
                        ddl += l * (x[i] * Bt[n] + A[hd] * alpha * S[t * PN + k]);
                        dA[hd] += l * d * alpha * S[t * PN + k];
                        lam[k] = alpha * l;
                    }
                    dx[i] = dxp;
                }
                ddt[(b * seqlen + t) * nheads + hd] = ddl;
            }
            for (int64_t k = 0; k < PN; ++k)
                dh0[(b * nheads + hd) * PN + k] = lam[k];
        }
    }
    free(S);
    free(yhat);
    free(lam);
    free(dyh);
    return 0;
}

/*
 * Trapezoidal (Mamba-3 SISO) form of the scalar-decay SSD, float64.
 *
 * "Mamba-3 NKI Kernels for AWS Neuron": section "How it works", Phase 0 gives
 * the per-token coefficients alpha = exp(dt A), gamma = lam dt and
 * beta = (dt - gamma) alpha (lam already through its sigmoid, dt through its
 * softplus); the decode path is the three-term recurrence of its Eq. 9,
 *   H_t = alpha_t H_{t-1} + beta_t (B_{t-1} x_{t-1}) + gamma_t (B_t x_t),
 * read out as y_t = C_t . H_t; Phase 5 adds the D skip and the silu gate.
 * Before the first token H is h0 (zero when NULL) and the previous input
 * B_{-1} x_{-1} is the outer product of the token before the sequence,
 * x_prev (batch, nheads, headdim) and B_prev (batch, ngroups, dstate), or zero
 * when both are NULL (the step() decode path of the same section carries this
 * previous-token term from call to call).  h_last is H after the last token.
 *   lam : (batch, seqlen, nheads); other layouts as oracle_ssd_f64.
 * Returns 0, or -1 on a bad shape (or only one of x_prev, B_prev given).
 */
int oracle_ssd_trap_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int64_t ngroups, const double *x, const double *dt,
                        const double *lam, const double *A, const double *B, const double *C,
                        const double *Dskip, const double *z, const double *h0,
                        const double *x_prev, const double *B_prev,
                        double *y, double *h_last)
{
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1 ||
        ngroups < 1 || nheads % ngroups != 0 || headdim * dstate > 65536 ||
        (x_prev == NULL) != (B_prev == NULL))
        return -1;
    static double H[65536], prev[65536];
    const int64_t hpg = nheads / ngroups;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t hd = 0; hd < nheads; ++hd) {
            const int64_t g = hd / hpg;
            for (int64_t k = 0; k < headdim * dstate; ++k)
                H[k] = h0 ? h0[(b * nheads + hd) * headdim * dstate + k] : 0.0;
            for (int64_t p = 0; p < headdim; ++p)
                for (int64_t n = 0; n < dstate; ++n)
                    prev[p * dstate + n] = x_prev ? B_prev[(b * ngroups + g) * dstate + n] *
                                                        x_prev[(b * nheads + hd) * headdim + p]
                                                  : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const double d = dt[(b * seqlen + t) * nheads + hd];
                const double lm = lam[(b * seqlen + t) * nheads + hd];
                const double alpha = exp(d * A[hd]);
                const double gamma = lm * d;
                const double beta = (d - gamma) * alpha;
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
                    const double xv = x[i];
                    double acc = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const int64_t k = p * dstate + n;
                        const double bx = Bt[n] * xv;
                        H[k] = alpha * H[k] + beta * prev[k] + gamma * bx;
                        prev[k] = bx;
                        acc += Ct[n] * H[k];
                    }
                    if (Dskip) acc += Dskip[hd] * xv;
                    if (z) acc *= silu(z[i]);
                    y[i] = acc;
                }
            }
            if (h_last)
                for (int64_t k = 0; k < headdim * dstate; ++k)
                    h_last[(b * nheads + hd) * headdim * dstate + k] = H[k];
        }
    }
    return 0;
}

/*
 * Gradients of the trapezoidal SSD above (reverse mode), float64.
 *
 * Upstream gradients dy on y and dh_last (nullable = zero) on h_last; returns
 * dx, dz (dz only with z), ddt, dlam (batch, seqlen, nheads), dA, dD (dD only
 * with Dskip), dB, dC, dh0, and with the token before the sequence dx_prev
 * (batch, nheads, headdim) and dB_prev (batch, ngroups, dstate) (NULL without
 * it).  As for oracle_ssd_bwd_f64, "Mamba-3 NKI Kernels for AWS Neuron",
 * section "Correctness", reports backward parity but prints no formulas: this
 * is the chain rule on the three-term recurrence of oracle_ssd_trap_f64 (its
 * Eq. 9 with alpha, beta, gamma of Phase 0), walked backwards.  With
 * Q_t = x_t B_t^T (P x N), P_{t-1} = Q_{t-1} (P_{-1} = x_prev B_prev^T or 0) and
 * Lam_t = dL/dH_t:
 *   Lam_t  = dyhat_t C_t^T + alpha_{t+1} Lam_{t+1}        (Lam_{L-1} also receives dh_last)
 *   dQ_t   = gamma_t Lam_t + beta_{t+1} Lam_{t+1}          (beta_L = 0)
 *   dx_t   = dQ_t B_t + D dyhat_t;   dB_t += dQ_t^T x_t;   dC_t += H_t^T dyhat_t
 *   dalpha_t = <Lam_t, H_{t-1}>,  dbeta_t = <Lam_t, P_{t-1}>,  dgamma_t = <Lam_t, Q_t>
 * and through alpha = exp(dt A), beta = dt (1 - lam) alpha, gamma = lam dt:
 *   ddt_t  = A alpha_t dalpha_t + (1 - lam_t) alpha_t (1 + dt_t A) dbeta_t + lam_t dgamma_t
 *   dlam_t = dt_t (dgamma_t - alpha_t dbeta_t),   dA += dt_t (alpha_t dalpha_t + beta_t dbeta_t)
 *   dh0 = alpha_0 Lam_0;   dP_{-1} = beta_0 Lam_0 gives dx_prev = dP_{-1} B_prev and
 *   dB_prev = sum over the group's heads of dP_{-1}^T x_prev.
 * Returns 0, -1 on a bad shape, -2 if memory runs out.
 */
int oracle_ssd_trap_bwd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups, const double *x, const double *dt,
                            const double *lam, const double *A, const double *B, const double *C,
                            const double *Dskip, const double *z, const double *h0,
                            const double *x_prev, const double *B_prev,
                            const double *dy, const double *dh_last,
                            double *dx, double *ddt, double *dlam, double *dA, double *dB, double *dC,
                            double *dD, double *dz, double *dh0, double *dx_prev, double *dB_prev)
{
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1 ||
        ngroups < 1 || nheads % ngroups != 0 || (x_prev == NULL) != (B_prev == NULL))
        return -1;
    const int64_t PN = headdim * dstate, hpg = nheads / ngroups;
    double *Hs = malloc(sizeof(double) * (size_t)((seqlen + 1) * PN));
    double *yhat = malloc(sizeof(double) * (size_t)((seqlen > 0 ? seqlen : 1) * headdim));
    double *Lm = malloc(sizeof(double) * (size_t)PN);      /* Lam_t */
    double *Ln = malloc(sizeof(double) * (size_t)PN);      /* Lam_{t+1} */
    double *dyh = malloc(sizeof(double) * (size_t)headdim);
    if (!Hs || !yhat || !Lm || !Ln || !dyh) {
        free(Hs); free(yhat); free(Lm); free(Ln); free(dyh);
        return -2;
    }
    for (int64_t k = 0; k < nheads; ++k) dA[k] = 0.0;
    if (Dskip)
        for (int64_t k = 0; k < nheads; ++k) dD[k] = 0.0;
    for (int64_t k = 0; k < batch * seqlen * ngroups * dstate; ++k) {
        dB[k] = 0.0;
        dC[k] = 0.0;
    }
    if (B_prev)
        for (int64_t k = 0; k < batch * ngroups * dstate; ++k) dB_prev[k] = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t hd = 0; hd < nheads; ++hd) {
            const int64_t g = hd / hpg;
            const double *xp = x_prev ? x_prev + (b * nheads + hd) * headdim : NULL;
            const double *bp = B_prev ? B_prev + (b * ngroups + g) * dstate : NULL;
            /* forward, keeping every state: Hs[t + 1] is H_t */
            for (int64_t k = 0; k < PN; ++k) Hs[k] = h0 ? h0[(b * nheads + hd) * PN + k] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t it = (b * seqlen + t) * nheads + hd;
                const double d = dt[it], alpha = exp(d * A[hd]), gamma = lam[it] * d;
                const double beta = (d - gamma) * alpha;
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Bq = t > 0 ? B + ((b * seqlen + t - 1) * ngroups + g) * dstate : bp;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = it * headdim + p;
                    const double xq = t > 0 ? x[i - nheads * headdim] : (xp ? xp[p] : 0.0);
                    double acc = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const int64_t k = p * dstate + n;
                        const double prev = Bq ? Bq[n] * xq : 0.0;
                        Hs[(t + 1) * PN + k] = alpha * Hs[t * PN + k] + beta * prev + gamma * Bt[n] * x[i];
                        acc += Ct[n] * Hs[(t + 1) * PN + k];
                    }
                    if (Dskip) acc += Dskip[hd] * x[i];
                    yhat[t * headdim + p] = acc;
                }
            }
            /* backward */
            for (int64_t k = 0; k < PN; ++k) {
                Ln[k] = 0.0;  /* Lam_L: nothing after the sequence */
                Lm[k] = 0.0;
            }
            double beta_next = 0.0, alpha_next = 0.0;
            for (int64_t t = seqlen - 1; t >= 0; --t) {
                const int64_t it = (b * seqlen + t) * nheads + hd;
                const double d = dt[it], lm = lam[it], alpha = exp(d * A[hd]), gamma = lm * d;
                const double beta = (d - gamma) * alpha;
                const double *Bt = B + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Ct = C + ((b * seqlen + t) * ngroups + g) * dstate;
                const double *Bq = t > 0 ? B + ((b * seqlen + t - 1) * ngroups + g) * dstate : bp;
                double *dBt = dB + ((b * seqlen + t) * ngroups + g) * dstate;
                double *dCt = dC + ((b * seqlen + t) * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = it * headdim + p;
                    dyh[p] = dy[i];
                    if (z) {
                        const double sg = 1.0 / (1.0 + exp(-z[i]));
                        dyh[p] = dy[i] * z[i] * sg;
                        dz[i] = dy[i] * yhat[t * headdim + p] * sg * (1.0 + z[i] * (1.0 - sg));
                    }
                    if (Dskip) dD[hd] += dyh[p] * x[i];
                }
                double dal = 0.0, dbe = 0.0, dga = 0.0;
                for (int64_t p = 0; p < headdim; ++p) {
                    const int64_t i = it * headdim + p;
                    const double xq = t > 0 ? x[i - nheads * headdim] : (xp ? xp[p] : 0.0);
                    double dxp = Dskip ? Dskip[hd] * dyh[p] : 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const int64_t k = p * dstate + n;
                        /* Lam_t = dyhat_t C_t^T + alpha_{t+1} Lam_{t+1} (+ dh_last at the end) */
                        double l = dyh[p] * Ct[n] + alpha_next * Ln[k];
                        if (t == seqlen - 1 && dh_last) l += dh_last[(b * nheads + hd) * PN + k];
                        Lm[k] = l;
                        const double dq = gamma * l + beta_next * Ln[k];
                        dxp += dq * Bt[n];
                        dBt[n] += dq * x[i];
                        dCt[n] += Hs[(t + 1) * PN + k] * dyh[p];
                        dal += l * Hs[t * PN + k];
                        dbe += l * (Bq ? Bq[n] * xq : 0.0);
                        dga += l * Bt[n] * x[i];
                    }
                    dx[i] = dxp;
                }
                ddt[it] = A[hd] * alpha * dal + (1.0 - lm) * alpha * (1.0 + d * A[hd]) * dbe + lm * dga;
                dlam[it] = d * (dga - alpha * dbe);
                dA[hd] += d * (alpha * dal + beta * dbe);
                for (int64_t k = 0; k < PN; ++k) Ln[k] = Lm[k];
                alpha_next = alpha;
                beta_next = beta;
            }
            /* the state before the first step, and the previous token's input */
            for (int64_t k = 0; k < PN; ++k) {
                double l = seqlen > 0 ? Ln[k] : (dh_last ? dh_last[(b * nheads + hd) * PN + k] : 0.0);
                dh0[(b * nheads + hd) * PN + k] = seqlen > 0 ? alpha_next * l : l;
            }
            if (xp) {
                double *dxq = dx_prev + (b * nheads + hd) * headdim;
                double *dbq = dB_prev + (b * ngroups + g) * dstate;
                for (int64_t p = 0; p < headdim; ++p) {
                    double v = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        const double dp = seqlen > 0 ? beta_next * Ln[p * dstate + n] : 0.0;
                        v += dp * bp[n];
                        dbq[n] += dp * xp[p];
                    }
                    dxq[p] = v;
                }
            }
        }
    }
    free(Hs); free(yhat); free(Lm); free(Ln); free(dyh);
    return 0;
}

/*
 * Phase-0 maps of the raw step and trapezoid inputs ("Mamba-3 NKI Kernels for
 * AWS Neuron", section "How it works", Phase 0: dt_softplus = softplus(dt +
 * dt_bias), lam_sigmoid = sigmoid(lam)).
 *
 * For n raw values laid out with the biased index the slowest of `inner`
 * consecutive elements and `nb` biases repeating: element i uses bias
 * bias[(i / inner) % nb] (bias NULL: 0).
 *   softplus(v) = log(1 + exp(v)), written as v + log1p(exp(-v)) for v > 0.
 *   sigmoid(v)  = 1 / (1 + exp(-v)), the derivative of softplus.
 */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

void oracle_softplus_f64(int64_t n, int64_t inner, int64_t nb, const double *raw, const double *bias,
                         double *out) {
  for (int64_t i = 0; i < n; ++i) {
    const double bv = bias ? bias[(i / inner) % nb] : 0.0;
    out[i] = softplus(raw[i] + bv);
  }
}

/* grad_out[i] = grad_in[i] * sigmoid(raw[i] + bias): the chain rule through
 * softplus, from the gradient of the step to that of the raw value. */
void oracle_softplus_grad_f64(int64_t n, int64_t inner, int64_t nb, const double *raw, const double *bias,
                              const double *grad_in, double *grad_out) {
  for (int64_t i = 0; i < n; ++i) {
    const double bv = bias ? bias[(i / inner) % nb] : 0.0;
    grad_out[i] = grad_in[i] * sigmoid(raw[i] + bv);
  }
}

void oracle_sigmoid_f64(int64_t n, const double *raw, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = sigmoid(raw[i]);
}

/*
 * Rotary step on B and C: the complex-valued state of Mamba-3.
 *   "Mamba-3 NKI Kernels for AWS Neuron", section "How it works", Phase 1:
 *   the angles are the negated running sum of dt * theta over the sequence,
 *   and B and C are rotated by them; the same page lists a complex-valued
 *   state via data-dependent RoPE among the Mamba-3 features.
 * The page gives no formula for the rotation itself; read plainly:
 *   phi_t[k] = angle0[k] - sum_{s <= t} dt_s * theta_s[k]   (k < dstate / 2,
 *     per batch row and head; dt is the step, after any softplus),
 *   and each state pair (k, k + dstate / 2), taken as the complex number
 *   v1 + i v2, is multiplied by exp(i phi_t):
 *     (v1, v2) -> (v1 cos phi - v2 sin phi, v1 sin phi + v2 cos phi),
 *   B and C of step t with the same angle.  The rotated B and C differ from
 *   head to head, so they are stored per head.
 *   dt           : (batch, seqlen, nheads)
 *   theta        : (batch, seqlen, theta_heads, dstate / 2), theta_heads 1
 *                  (one set of angles for every head) or nheads
 *   B, C         : (batch, seqlen, ngroups, dstate); head h reads group
 *                  h / (nheads / ngroups)
 *   angle0       : (batch, nheads, dstate / 2) angle before the first step
 *                  (nullable: 0)
 *   B_rot, C_rot : (batch, seqlen, nheads, dstate)
 *   angle_last   : (batch, nheads, dstate / 2) angle after the last step
 */
int oracle_rope_bc_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups, int64_t dstate,
                       int64_t theta_heads, const double *dt, const double *theta, const double *B,
                       const double *C, const double *angle0, double *B_rot, double *C_rot,
                       double *angle_last) {
  if (batch < 0 || seqlen < 0 || nheads < 1 || ngroups < 1 || nheads % ngroups != 0 || dstate < 2 ||
      dstate % 2 != 0 || (theta_heads != 1 && theta_heads != nheads))
    return -1;
  const int64_t half = dstate / 2, hpg = nheads / ngroups;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < nheads; ++h) {
      const int64_t g = h / hpg;
      const int64_t th = theta_heads == 1 ? 0 : h;
      for (int64_t k = 0; k < half; ++k) {
        double phi = angle0 ? angle0[(b * nheads + h) * half + k] : 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
          phi -= dt[(b * seqlen + t) * nheads + h] * theta[((b * seqlen + t) * theta_heads + th) * half + k];
          const double c = cos(phi), s = sin(phi);
          const int64_t src = ((b * seqlen + t) * ngroups + g) * dstate;
          const int64_t dst = ((b * seqlen + t) * nheads + h) * dstate;
          const double b1 = B[src + k], b2 = B[src + k + half];
          const double c1 = C[src + k], c2 = C[src + k + half];
          B_rot[dst + k] = b1 * c - b2 * s;
          B_rot[dst + k + half] = b1 * s + b2 * c;
          C_rot[dst + k] = c1 * c - c2 * s;
          C_rot[dst + k + half] = c1 * s + c2 * c;
        }
        angle_last[(b * nheads + h) * half + k] = phi;
      }
    }
  }
  return 0;
}

/*
 * Gradients of the rotary step (oracle_rope_bc_f64) for upstream gradients
 * dB_rot, dC_rot (batch, seqlen, nheads, dstate) and dangle_last (batch,
 * nheads, dstate / 2; nullable: 0).  The pages print no backward; this is
 * the chain rule on the forward written above ("Mamba-3 NKI Kernels for AWS
 * Neuron", section "How it works", Phase 1, as read there):
 *   B and C: the rotation by phi_t is orthogonal, so each pair's gradient is
 *     the upstream gradient turned back by -phi_t, summed over the heads that
 *     read the group;
 *   phi_t: d(v1 cos - v2 sin)/dphi = -(rotated v2) and d(v1 sin + v2 cos)/dphi
 *     = rotated v1, so dL/dphi_t, per pair, is the sum over B and C of
 *     -dRot1 * rot2 + dRot2 * rot1;
 *   phi_t = angle0 - sum_{s <= t} dt_s theta_s: with R_s = dangle_last +
 *     sum_{t >= s} dL/dphi_t, dtheta_s += -dt_s R_s (summed over heads when
 *     theta is shared), ddt_s += -sum_k theta_s[k] R_s[k], dangle0 = R_0.
 * ddt is the gradient of the step (the caller chains any softplus).
 * Outputs: ddt (batch, seqlen, nheads), dtheta like theta, dB and dC like B
 * and C, dangle0 like angle0; all are written (zeroed first).
 */
int oracle_rope_bc_bwd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups, int64_t dstate,
                           int64_t theta_heads, const double *dt, const double *theta, const double *B,
                           const double *C, const double *angle0, const double *dB_rot, const double *dC_rot,
                           const double *dangle_last, double *ddt, double *dtheta, double *dB, double *dC,
                           double *dangle0) {
  if (batch < 0 || seqlen < 0 || nheads < 1 || ngroups < 1 || nheads % ngroups != 0 || dstate < 2 ||
      dstate % 2 != 0 || (theta_heads != 1 && theta_heads != nheads))
    return -1;
  const int64_t half = dstate / 2, hpg = nheads / ngroups;
  for (int64_t i = 0; i < batch * seqlen * nheads; ++i) ddt[i] = 0.0;
  for (int64_t i = 0; i < batch * seqlen * theta_heads * half; ++i) dtheta[i] = 0.0;
  for (int64_t i = 0; i < batch * seqlen * ngroups * dstate; ++i) dB[i] = dC[i] = 0.0;
  double *phis = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  double *dphi = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  if (!phis || !dphi) {
    free(phis); free(dphi);
    return -2;
  }
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < nheads; ++h) {
      const int64_t g = h / hpg;
      const int64_t th = theta_heads == 1 ? 0 : h;
      for (int64_t k = 0; k < half; ++k) {
        /* The forward angles. */
        double phi = angle0 ? angle0[(b * nheads + h) * half + k] : 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
          phi -= dt[(b * seqlen + t) * nheads + h] * theta[((b * seqlen + t) * theta_heads + th) * half + k];
          phis[t] = phi;
        }
        /* Each step: B and C turned back, and the gradient of its angle. */
        for (int64_t t = 0; t < seqlen; ++t) {
          const double c = cos(phis[t]), s = sin(phis[t]);
          const int64_t src = ((b * seqlen + t) * ngroups + g) * dstate;
          const int64_t dst = ((b * seqlen + t) * nheads + h) * dstate;
          const double b1 = B[src + k], b2 = B[src + k + half];
          const double c1 = C[src + k], c2 = C[src + k + half];
          const double gb1 = dB_rot[dst + k], gb2 = dB_rot[dst + k + half];
          const double gc1 = dC_rot[dst + k], gc2 = dC_rot[dst + k + half];
          dB[src + k] += gb1 * c + gb2 * s;
          dB[src + k + half] += -gb1 * s + gb2 * c;
          dC[src + k] += gc1 * c + gc2 * s;
          dC[src + k + half] += -gc1 * s + gc2 * c;
          /* rotated pair (r1, r2) = (v1 c - v2 s, v1 s + v2 c): dr1/dphi = -r2, dr2/dphi = r1 */
          const double rb1 = b1 * c - b2 * s, rb2 = b1 * s + b2 * c;
          const double rc1 = c1 * c - c2 * s, rc2 = c1 * s + c2 * c;
          dphi[t] = -gb1 * rb2 + gb2 * rb1 - gc1 * rc2 + gc2 * rc1;
        }
        /* The running sum, walked backwards. */
        double R = dangle_last ? dangle_last[(b * nheads + h) * half + k] : 0.0;
        for (int64_t t = seqlen - 1; t >= 0; --t) {
          R += dphi[t];
          const int64_t it = (b * seqlen + t) * nheads + h;
          const int64_t ith = ((b * seqlen + t) * theta_heads + th) * half + k;
          dtheta[ith] += -dt[it] * R;
          ddt[it] += -theta[ith] * R;
        }
        dangle0[(b * nheads + h) * half + k] = R;
      }
    }
  }
  free(phis);
  free(dphi);
  return 0;
}
