/*
 * Plain fp64 CPU oracle for the selective-scan (S6) forward path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code with the HIP library.
 *
 * What it computes, per batch row b and channel d, as a plain sequential loop
 * over time t and state index n (no blocking, no reordering):
 *
 *   c_t  = conv_b[d] + sum_k conv_w[d,k] * x_{t-(K-1)+k}     causal depthwise conv,
 *          history from conv_state (or zeros)                 conv_w[d,K-1] multiplies x_t
 *   u_t  = c_t * sigmoid(c_t)                                 SiLU
 *   D_t  = softplus(delta_t + b_delta[d])                     selection of the step size
 *   h_t  = exp(D_t * A[d,n]) * h_{t-1} + Bbar_t[n] * u_t      discretised recurrence
 *          Bbar = D_t * B_t[n]                                 (Euler write term), or
 *          Bbar = (1 - exp(D_t A[d,n])) / (-A[d,n]) * B_t[n]    (zero-order hold; D_t * B when A = 0)
 *   y_t  = sum_n C_t[n] * h_t[n] + Dskip[d] * u_t             readout after the update
 *   out_t = y_t * z_t * sigmoid(z_t)                          SiLU(z) gate
 *
 * Sources (the pages, cited by title and section):
 *  - ai360xpert.com "Mamba", "The selection mechanism": step size is softplus of
 *    an affine function of the input (bias inside the softplus); A_bar = exp(Delta A),
 *    B_bar ~ Delta B (the Euler write term, the default); its "Show Me the Code"
 *    loop and inferensys.com "Mamba" (zero-order hold rule) give the ZOH form
 *    B_bar = (1 - A_bar)/(-A) B (selected by `zoh`).
 *  - ozercemkelahmet.com "Mamba", "A minimal selective scan in PyTorch": state per
 *    (batch, channel, state index), zero initial state, dA = exp(delta*A),
 *    dB = delta*B, h = dA*h + dB*x, output read from the updated state as sum over n
 *    of h*C; "Deployment notes": state passed from one chunk to the next.
 *  - bembew.net "Overview of Mamba (SSM) Model", "How the Mamba Block Works":
 *    depthwise convolution then SiLU before the SSM; a SiLU branch gates the
 *    SSM output elementwise.
 *  - ozercemkelahmet.com "Mamba", "Glossary": the causal convolution looks only at
 *    the current and past positions.
 *  - The D*u skip term is not on the pages; it is part of the computation this
 *    library implements and is added before the gate.
 * Readings where the pages are silent: SiLU(v) = v/(1+exp(-v)); softplus in the
 * overflow-free form max(v,0) + log1p(exp(-|v|)); conv zero history, bias before
 * SiLU; NaN/Inf propagate.
 *
 * Optional pieces: conv_w == NULL means no conv and no SiLU (u = x) and then
 * conv_state must be NULL; conv_b / delta_bias / Dskip NULL mean zero;
 * z == NULL means no gate; ssm_state / conv_state NULL mean zero initial state
 * and nothing returned, otherwise they are read as the initial state and
 * overwritten with the final one.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_MAX_K 16

static double silu(double v) { return v / (1.0 + exp(-v)); }

static double softplus(double v) {
    double m = v > 0.0 ? v : 0.0;
    return m + log1p(exp(-fabs(v)));
}

/* One channel (b,d) over the whole sequence. Strides are in elements. */
static void scan_channel(int64_t L, int64_t D, int64_t N, int64_t K,
                         const double* x, const double* conv_w, const double* conv_b,
                         const double* delta, const double* delta_bias, const double* A,
                         const double* Bm, const double* Cm, const double* Dskip,
                         const double* z, double* y, double* ssm_state, double* conv_state,
                         int zoh, int64_t b, int64_t d, double* h) {
    double win[ORACLE_MAX_K];            /* win[0..K-2]: x_{t-(K-1)} .. x_{t-1} */
    for (int64_t k = 0; k < K - 1; ++k)
        win[k] = conv_state ? conv_state[(b * D + d) * (K - 1) + k] : 0.0;
    for (int64_t n = 0; n < N; ++n)
        h[n] = ssm_state ? ssm_state[(b * D + d) * N + n] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = (b * L + t) * D + d;     /* [B,L,D] */
        const int64_t bc = (b * L + t) * N;          /* [B,L,N] */
        const double xt = x[row];

        double u;
        if (conv_w) {
            double c = conv_b ? conv_b[d] : 0.0;
            for (int64_t k = 0; k < K - 1; ++k) c += conv_w[d * K + k] * win[k];
            c += conv_w[d * K + (K - 1)] * xt;
            u = silu(c);
            for (int64_t k = 0; k + 1 < K - 1; ++k) win[k] = win[k + 1];
            if (K > 1) win[K - 2] = xt;
        } else {
            u = xt;
        }

        const double dt = softplus(delta[row] + (delta_bias ? delta_bias[d] : 0.0));

        for (int64_t n = 0; n < N; ++n) {
            const double a = A[d * N + n];
            const double abar = exp(dt * a);
            double bcoef = dt;                                   /* Euler: Delta */
            if (zoh && a != 0.0) bcoef = expm1(dt * a) / a;      /* (1 - exp(Delta a)) / (-a) */
            h[n] = abar * h[n] + bcoef * Bm[bc + n] * u;
        }

        double yt = 0.0;
        for (int64_t n = 0; n < N; ++n) yt += Cm[bc + n] * h[n];
        yt += (Dskip ? Dskip[d] : 0.0) * u;

        if (z) yt *= silu(z[row]);
        y[row] = yt;
    }

    if (ssm_state)
        for (int64_t n = 0; n < N; ++n) ssm_state[(b * D + d) * N + n] = h[n];
    if (conv_state)
        for (int64_t k = 0; k < K - 1; ++k) conv_state[(b * D + d) * (K - 1) + k] = win[k];
}

/* Returns 0 on success, -1 on bad arguments. nthreads <= 0 means the OpenMP default. */
int oracle_conv_scan_fwd(int64_t Bsz, int64_t L, int64_t D, int64_t N, int64_t K,
                         const double* x, const double* conv_w, const double* conv_b,
                         const double* delta, const double* delta_bias, const double* A,
                         const double* Bm, const double* Cm, const double* Dskip,
                         const double* z, double* y, double* ssm_state, double* conv_state,
                         int zoh, int nthreads) {
    if (Bsz < 0 || L < 0 || D < 0 || N < 1 || N > 1024 || K < 1 || K > ORACLE_MAX_K) return -1;
    if (!x || !delta || !A || !Bm || !Cm || !y) return -1;
    if (!conv_w && conv_state) return -1;
    const int64_t channels = Bsz * D;

#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    {
        double h[1024];
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < channels; ++i)
            scan_channel(L, D, N, K, x, conv_w, conv_b, delta, delta_bias, A, Bm, Cm, Dskip,
                         z, y, ssm_state, conv_state, zoh, i / D, i % D, h);
    }
    return 0;
}

/* One decode step: the same computation with L = 1 and both states required
 * (x, delta, z, y are [B,D]; B, C are [B,N]). */
int oracle_step(int64_t Bsz, int64_t D, int64_t N, int64_t K,
                const double* x, const double* conv_w, const double* conv_b,
                const double* delta, const double* delta_bias, const double* A,
                const double* Bm, const double* Cm, const double* Dskip,
                const double* z, double* y, double* ssm_state, double* conv_state,
                int zoh, int nthreads) {
    if (!ssm_state || (conv_w && !conv_state)) return -1;
    return oracle_conv_scan_fwd(Bsz, 1, D, N, K, x, conv_w, conv_b, delta, delta_bias, A,
                                Bm, Cm, Dskip, z, y, ssm_state, conv_state, zoh, nthreads);
}

int oracle_version(void) { return 2; }
