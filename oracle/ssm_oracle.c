/*
 * ssm_oracle.c -- plain, slow, sequential fp64 reference ("oracle") for the
 * selective state-space scan.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline leg load this library. The HIP product path never calls it, and the
 * two share no code, headers or tables.
 *
 * What is computed
 * ----------------
 * The state-space recurrence of "Jamba — SSM-Transformer Híbrido"
 * (ai-engineering.academy), section "Um SSM em uma página", also given in the
 * zh lesson page "马巴 混合型SSM变压器" (Phase 10 · 21), section "一页的SSM":
 *
 *     h_t = Abar_t h_{t-1} + Bbar_t x_t ,        y_t = C_t h_t
 *
 * Both pages state that Mamba makes A, B, C data-dependent (the "selective"
 * part) and that y_t needs only h_{t-1} and x_t (constant-size state).
 *
 * The discretisation, the skip term D and the gate follow the MambaBlock of
 * "【大模型】- Jamba 混合 SSM-Transformer", section 4.1 "Mamba 层":
 *     Abar = exp(dt * A)   (A diagonal: one value per channel d and state n)
 *     Bbar = dt * B        (B and C shared by all channels of a (batch, step))
 *     y    = (sum_n C[n] h[n] + D[d] x) * silu(z),  silu(z) = z / (1 + exp(-z)).
 * The page's own loop sums (h * D) and never forms C or the D*x skip; the
 * reading taken here is the recurrence's y_t = C_t h_t plus the D skip, and
 * the whole is gated, as the MambaBlock gates the scan's output.
 *
 * The complex-state variant is the data-dependent rotation of the Mamba-3
 * item "Atualização de estado com valores complexos" on the same pt page:
 * A = (-a + i*theta) per (d, n), Abar = exp(dt * A) = exp(-dt a)(cos(dt theta)
 * + i sin(dt theta)), h complex, y = Re(sum_n C[n] h[n]) + D x (C not
 * conjugated), then the optional gate.
 *
 * Order of operations (fixed, so that special cases hold bit for bit):
 *     dA = exp(dt * A[d][n]);  dB = dt * B[n];
 *     h[n] = (dA * h[n]) + (dB * x);  acc = acc + C[n] * h[n]   (n ascending)
 *     y = acc + D[d] * x;  if gated: y = y * (z / (1 + exp(-z)))
 * Compiled with -ffp-contract=off: no fused multiply-adds.
 *
 * Layouts (row-major, contiguous, channel index fastest):
 *     x, dt, z, y : [batch][L][Dn]          B, C : [batch][L][N]   (complex: [..][N][2])
 *     A           : [Dn][N]   (complex: [Dn][N][2] = (re, im))     Dv : [Dn]
 *     h0, h_final : [batch][Dn][N]           (complex: [batch][Dn][N][2])
 * z and h0 may be NULL: no gate, zero initial state.
 * Decode (one token): h [n_layers][n_seq][Dn][N] updated in place;
 *     x, dt, z, y : [n_layers][n_seq][Dn];  B, C : [n_layers][n_seq][N];
 *     A : [n_layers][Dn][N];  Dv : [n_layers][Dn].
 * Return value: 0 on success, -1 on invalid sizes or allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Prefill over a whole sequence, real diagonal state. */
int oracle_scan_f64(int64_t batch, int64_t L, int64_t Dn, int64_t N,
                    const double *x, const double *dt, const double *A,
                    const double *B, const double *C, const double *Dv,
                    const double *z, const double *h0,
                    double *y, double *h_final)
{
    if (batch < 0 || L < 0 || Dn < 0 || N <= 0) return -1;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    if (!h) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * Dn + d;   /* (b, t, d) */
                const int64_t s = (b * L + t) * N;        /* (b, t, 0) */
                const double xv = x[i], dv = dt[i];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * A[d * N + n]);
                    const double dB = dv * B[s + n];
                    h[n] = dA * h[n] + dB * xv;
                    acc = acc + C[s + n] * h[n];
                }
                double yv = acc + Dv[d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
            }
            if (h_final)
                for (int64_t n = 0; n < N; ++n) h_final[(b * Dn + d) * N + n] = h[n];
        }
    }
    free(h);
    return 0;
}

/* One decode token for every (layer, sequence, channel); h updated in place. */
int oracle_step_f64(int64_t n_layers, int64_t n_seq, int64_t Dn, int64_t N,
                    double *h, const double *x, const double *dt, const double *A,
                    const double *B, const double *C, const double *Dv,
                    const double *z, double *y)
{
    if (n_layers < 0 || n_seq < 0 || Dn < 0 || N <= 0) return -1;
    for (int64_t l = 0; l < n_layers; ++l) {
        for (int64_t q = 0; q < n_seq; ++q) {
            const int64_t s = (l * n_seq + q) * N;            /* (l, q, 0) of B, C */
            for (int64_t d = 0; d < Dn; ++d) {
                const int64_t i = (l * n_seq + q) * Dn + d;   /* (l, q, d) */
                double *hs = h + i * N;
                const double *Ad = A + (l * Dn + d) * N;
                const double xv = x[i], dv = dt[i];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * Ad[n]);
                    const double dB = dv * B[s + n];
                    hs[n] = dA * hs[n] + dB * xv;
                    acc = acc + C[s + n] * hs[n];
                }
                double yv = acc + Dv[l * Dn + d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
            }
        }
    }
    return 0;
}

/* Prefill with a complex diagonal state, written with explicit re/im parts. */
int oracle_scan_c128(int64_t batch, int64_t L, int64_t Dn, int64_t N,
                     const double *x, const double *dt, const double *A,
                     const double *B, const double *C, const double *Dv,
                     const double *z, const double *h0,
                     double *y, double *h_final)
{
    if (batch < 0 || L < 0 || Dn < 0 || N <= 0) return -1;
    double *hr = (double *)malloc((size_t)N * sizeof(double));
    double *hi = (double *)malloc((size_t)N * sizeof(double));
    if (!hr || !hi) { free(hr); free(hi); return -1; }
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            for (int64_t n = 0; n < N; ++n) {
                hr[n] = h0 ? h0[((b * Dn + d) * N + n) * 2 + 0] : 0.0;
                hi[n] = h0 ? h0[((b * Dn + d) * N + n) * 2 + 1] : 0.0;
            }
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * Dn + d;
                const int64_t s = (b * L + t) * N;
                const double xv = x[i], dv = dt[i];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double are = A[(d * N + n) * 2 + 0];
                    const double aim = A[(d * N + n) * 2 + 1];
                    const double mag = exp(dv * are);
                    const double dAr = mag * cos(dv * aim);
                    const double dAi = mag * sin(dv * aim);
                    const double dBr = dv * B[(s + n) * 2 + 0];
                    const double dBi = dv * B[(s + n) * 2 + 1];
                    const double nr = (dAr * hr[n] - dAi * hi[n]) + dBr * xv;
                    const double ni = (dAr * hi[n] + dAi * hr[n]) + dBi * xv;
                    hr[n] = nr;
                    hi[n] = ni;
                    acc = acc + (C[(s + n) * 2 + 0] * hr[n] - C[(s + n) * 2 + 1] * hi[n]);
                }
                double yv = acc + Dv[d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
            }
            if (h_final)
                for (int64_t n = 0; n < N; ++n) {
                    h_final[((b * Dn + d) * N + n) * 2 + 0] = hr[n];
                    h_final[((b * Dn + d) * N + n) * 2 + 1] = hi[n];
                }
        }
    }
    free(hr);
    free(hi);
    return 0;
}

/* One decode token with a complex state; h [n_layers][n_seq][Dn][N][2] in place. */
int oracle_step_c128(int64_t n_layers, int64_t n_seq, int64_t Dn, int64_t N,
                     double *h, const double *x, const double *dt, const double *A,
                     const double *B, const double *C, const double *Dv,
                     const double *z, double *y)
{
    if (n_layers < 0 || n_seq < 0 || Dn < 0 || N <= 0) return -1;
    for (int64_t l = 0; l < n_layers; ++l) {
        for (int64_t q = 0; q < n_seq; ++q) {
            const int64_t s = (l * n_seq + q) * N;
            for (int64_t d = 0; d < Dn; ++d) {
                const int64_t i = (l * n_seq + q) * Dn + d;
                double *hs = h + i * N * 2;
                const double *Ad = A + (l * Dn + d) * N * 2;
                const double xv = x[i], dv = dt[i];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double mag = exp(dv * Ad[2 * n + 0]);
                    const double dAr = mag * cos(dv * Ad[2 * n + 1]);
                    const double dAi = mag * sin(dv * Ad[2 * n + 1]);
                    const double dBr = dv * B[(s + n) * 2 + 0];
                    const double dBi = dv * B[(s + n) * 2 + 1];
                    const double nr = (dAr * hs[2 * n] - dAi * hs[2 * n + 1]) + dBr * xv;
                    const double ni = (dAr * hs[2 * n + 1] + dAi * hs[2 * n]) + dBi * xv;
                    hs[2 * n] = nr;
                    hs[2 * n + 1] = ni;
                    acc = acc + (C[(s + n) * 2 + 0] * nr - C[(s + n) * 2 + 1] * ni);
                }
                double yv = acc + Dv[l * Dn + d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
            }
        }
    }
    return 0;
}

/* Bytes of a fixed-size SSM state: layers x channels x state size x bytes per
 * value. It does not depend on the sequence length (the memory-budget section,
 * "O orçamento de memória", of the pt page). */
int64_t oracle_state_bytes(int64_t n_layers, int64_t channels, int64_t d_state,
                           int64_t bytes_per_value)
{
    return n_layers * channels * d_state * bytes_per_value;
}

/* ------------------------------------------------------------------ input stage
 * What the MambaBlock ("【大模型】- Jamba 混合 SSM-Transformer", section 4.1
 * "Mamba 层") does to its inputs before the scan:
 *  - x: a depthwise 1-D convolution over time (one filter of K taps and one bias
 *    per channel), with K-1 zeros of padding in front and the output cut back to
 *    the first L steps, so output t sees inputs t-K+1 .. t only; then silu.
 *  - dt: softplus of the dt projection's output, softplus(v) = log(1 + e^v).
 * A convolution in the deep-learning sense takes no flip: tap k multiplies the
 * input k steps after the window's first one, i.e. x_{t-(K-1)+k}.
 *
 * Inputs before step 0 come from a carried "conv state" (the last K-1 inputs of
 * the previous call, oldest first) or are zero, which is the padding above. The
 * state after the call is the last K-1 inputs, so that calls can be chained.
 *
 * Layouts: x, u [batch][L][Dn]; w [Dn][K]; cb [Dn] (NULL = no bias);
 * state0, state_out [batch][K-1][Dn] (state0 NULL = zeros; state_out NULL = not
 * wanted); K >= 1. */
static double conv_input(const double *x, const double *state0, int64_t b, int64_t s,
                         int64_t d, int64_t L, int64_t Dn, int64_t K)
{
    if (s >= 0) return x[(b * L + s) * Dn + d];
    if (!state0) return 0.0;
    return state0[(b * (K - 1) + (K - 1 + s)) * Dn + d];
}

int oracle_conv_silu_f64(int64_t batch, int64_t L, int64_t Dn, int64_t K,
                         const double *x, const double *w, const double *cb,
                         const double *state0, double *u, double *state_out)
{
    if (batch < 0 || L < 0 || Dn < 0 || K < 1) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t t = 0; t < L; ++t) {
            for (int64_t d = 0; d < Dn; ++d) {
                double acc = cb ? cb[d] : 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc = acc + w[d * K + k] * conv_input(x, state0, b, t - (K - 1) + k, d, L, Dn, K);
                u[(b * L + t) * Dn + d] = silu(acc);
            }
        }
        if (state_out)
            for (int64_t j = 0; j < K - 1; ++j)
                for (int64_t d = 0; d < Dn; ++d)
                    state_out[(b * (K - 1) + j) * Dn + d] =
                        conv_input(x, state0, b, L - (K - 1) + j, d, L, Dn, K);
    }
    return 0;
}

/* softplus(v) = log(1 + e^v), written as max(v, 0) + log(1 + e^-|v|) so that it
 * neither overflows for large v nor loses the small result for very negative v;
 * the two forms are equal (for v > 0, 1 + e^v = e^v (1 + e^-v)). */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* dt[i][d] = softplus(raw[i][d] + bias[d]) for rows i < rows (bias NULL = 0). The
 * bias is that of the dt projection, applied here so the projection itself can run
 * without one. */
int oracle_softplus_f64(int64_t rows, int64_t Dn, const double *raw, const double *bias,
                        double *dt)
{
    if (rows < 0 || Dn < 0) return -1;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t d = 0; d < Dn; ++d)
            dt[i * Dn + d] = softplus(raw[i * Dn + d] + (bias ? bias[d] : 0.0));
    return 0;
}

/* Gradients through the input stage above, for training: the chain rule of
 * oracle_conv_silu_f64 and oracle_softplus_f64 written out. With xe the K-1 carried
 * inputs followed by x (xe_s = conv_input(s), s = -(K-1) .. L-1),
 *     a_t = cb + sum_k w[k] xe_{t-(K-1)+k},  u_t = silu(a_t),  dt_t = softplus(r_t + bias),
 * and given du = dLoss/du, ddt = dLoss/ddt:
 *     da_t = du_t s (1 + a_t (1 - s)),  s = 1 / (1 + e^-a_t)       (silu')
 *     dxe_{t-(K-1)+k} += w[k] da_t,  dw[k] += da_t xe_{t-(K-1)+k},  dcb += da_t
 *     dr_t = ddt_t / (1 + e^-(r_t + bias)),  dbias += dr_t        (softplus' = sigmoid)
 * dx = dxe_0 .. dxe_{L-1}; dstate0 = dxe_{-(K-1)} .. dxe_{-1} (NULL: not wanted).
 * dw, dcb, dbias are summed over batch and steps. K = 0 means no convolution and no
 * silu (u = x): dx = du, and w, cb, dw, dcb, state0, dstate0 are unused. cb, bias,
 * state0 NULL: zero (their gradients then not written when NULL). Every output given
 * is overwritten. Layouts as oracle_conv_silu_f64; r, ddt, dr [batch][L][Dn]. */
int oracle_input_stage_bwd_f64(int64_t batch, int64_t L, int64_t Dn, int64_t K,
                               const double *x, const double *r, const double *w,
                               const double *cb, const double *state0, const double *bias,
                               const double *du, const double *ddt, double *dx, double *dr,
                               double *dw, double *dcb, double *dbias, double *dstate0)
{
    if (batch < 0 || L < 0 || Dn < 0 || K < 0) return -1;
    const int64_t H = K > 0 ? K - 1 : 0;
    for (int64_t i = 0; i < batch * L * Dn; ++i) dx[i] = 0.0;
    if (dstate0) for (int64_t i = 0; i < batch * H * Dn; ++i) dstate0[i] = 0.0;
    if (K > 0) {
        for (int64_t i = 0; i < Dn * K; ++i) dw[i] = 0.0;
        if (dcb) for (int64_t d = 0; d < Dn; ++d) dcb[d] = 0.0;
    }
    if (dbias) for (int64_t d = 0; d < Dn; ++d) dbias[d] = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t t = 0; t < L; ++t) {
            for (int64_t d = 0; d < Dn; ++d) {
                const int64_t e = (b * L + t) * Dn + d;
                if (K == 0) {
                    dx[e] = du[e];
                } else {
                    double pre = cb ? cb[d] : 0.0;  /* a_t, the convolution before silu */
                    for (int64_t k = 0; k < K; ++k)
                        pre = pre + w[d * K + k] * conv_input(x, state0, b, t - H + k, d, L, Dn, K);
                    const double sg = 1.0 / (1.0 + exp(-pre));
                    const double da = du[e] * sg * (1.0 + pre * (1.0 - sg));
                    for (int64_t k = 0; k < K; ++k) {
                        const int64_t s = t - H + k;
                        dw[d * K + k] += da * conv_input(x, state0, b, s, d, L, Dn, K);
                        if (s >= 0) dx[(b * L + s) * Dn + d] += w[d * K + k] * da;
                        else if (dstate0) dstate0[(b * H + (H + s)) * Dn + d] += w[d * K + k] * da;
                    }
                    if (dcb) dcb[d] += da;
                }
                const double v = r[e] + (bias ? bias[d] : 0.0);
                dr[e] = ddt[e] / (1.0 + exp(-v));
                if (dbias) dbias[d] += dr[e];
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ backward
 * Gradients of the real-state prefill, for training: given dy = dLoss/dy and
 * optionally dh_final = dLoss/dh_final, the gradients of
 *     Loss = sum dy * y + sum dh_final * h_final
 * with respect to x, dt, z [batch][L][Dn], A [Dn][N], B, C [batch][L][N],
 * Dv [Dn] and h0 [batch][Dn][N]. The pages name the training-time evaluation of
 * the SSM ("Jamba — SSM-Transformer Híbrido", section "Um SSM em uma página", the
 * convolution form used in training) but print no backward; this is the chain
 * rule through the forward loop above, written out step by step:
 *     h_t = a_t h_{t-1} + dt_t B_t x_t,  a_t = exp(dt_t A),  o_t = C_t.h_t + D x_t,
 *     y_t = o_t g(z_t),  g = silu,  g'(z) = s (1 + z (1 - s)),  s = 1 / (1 + e^-z).
 * The adjoint lam_t = dLoss/dh_t obeys lam_t = do_t C_t + a_{t+1} lam_{t+1}, run
 * backwards from lam = dh_final, with do_t = dy_t g(z_t). Then, per step,
 *     dx_t  = do_t D + sum_n lam_t[n] dt_t B_t[n]
 *     ddt_t = sum_n lam_t[n] (x_t B_t[n] + A[n] a_t[n] h_{t-1}[n])
 *     dz_t  = dy_t o_t g'(z_t)
 *     dA[n] += lam_t[n] dt_t a_t[n] h_{t-1}[n]      dD += do_t x_t
 *     dB_t[n] += lam_t[n] dt_t x_t                  dC_t[n] += do_t h_t[n]
 * (dA, dD summed over batch and steps; dB, dC over channels), and
 * dh0 = a_0 lam_0. The states h_t are kept from a forward pass over the channel.
 * dh_final, z, h0 may be NULL (zero, ungated, zero); dz, dh0 may be NULL (not
 * wanted). Every output is overwritten. */
int oracle_scan_bwd_f64(int64_t batch, int64_t L, int64_t Dn, int64_t N,
                        const double *x, const double *dt, const double *A,
                        const double *B, const double *C, const double *Dv,
                        const double *z, const double *h0, const double *dy,
                        const double *dh_final, double *dx, double *ddt, double *dA,
                        double *dB, double *dC, double *dD, double *dz, double *dh0)
{
    if (batch < 0 || L < 0 || Dn < 0 || N <= 0) return -1;
    double *hs = (double *)malloc((size_t)(L + 1) * (size_t)N * sizeof(double));
    double *lam = (double *)malloc((size_t)N * sizeof(double));
    if (!hs || !lam) { free(hs); free(lam); return -1; }
    memset(dA, 0, (size_t)(Dn * N) * sizeof(double));
    memset(dD, 0, (size_t)Dn * sizeof(double));
    memset(dB, 0, (size_t)(batch * L * N) * sizeof(double));
    memset(dC, 0, (size_t)(batch * L * N) * sizeof(double));
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            /* forward, keeping every state: hs[t + 1] = h_t, hs[0] = h0 */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * Dn + d;
                const int64_t s = (b * L + t) * N;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(dt[i] * A[d * N + n]);
                    hs[(t + 1) * N + n] = a * hs[t * N + n] + (dt[i] * B[s + n]) * x[i];
                }
            }
            /* backward */
            for (int64_t n = 0; n < N; ++n) lam[n] = dh_final ? dh_final[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t i = (b * L + t) * Dn + d;
                const int64_t s = (b * L + t) * N;
                const double xv = x[i], dv = dt[i];
                double o = Dv[d] * xv;
                for (int64_t n = 0; n < N; ++n) o = o + C[s + n] * hs[(t + 1) * N + n];
                double dout = dy[i];
                if (z) {
                    const double sg = 1.0 / (1.0 + exp(-z[i]));
                    dout = dy[i] * (z[i] * sg);
                    if (dz) dz[i] = dy[i] * o * (sg * (1.0 + z[i] * (1.0 - sg)));
                }
                dD[d] += dout * xv;
                double gx = dout * Dv[d], gdt = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double lt = lam[n] + dout * C[s + n];       /* lam_t[n] */
                    const double a = exp(dv * A[d * N + n]);
                    const double hp = hs[t * N + n];                   /* h_{t-1}[n] */
                    dC[s + n] += dout * hs[(t + 1) * N + n];
                    dB[s + n] += lt * dv * xv;
                    gx += lt * dv * B[s + n];
                    gdt += lt * (xv * B[s + n] + A[d * N + n] * a * hp);
                    dA[d * N + n] += lt * dv * a * hp;
                    lam[n] = a * lt;                                  /* a_t lam_t */
                }
                dx[i] = gx;
                ddt[i] = gdt;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[(b * Dn + d) * N + n] = lam[n];
        }
    }
    if (z == NULL && dz != NULL) memset(dz, 0, (size_t)(batch * L * Dn) * sizeof(double));
    free(hs);
    free(lam);
    return 0;
}

/*
 * Exponential-trapezoidal discretisation (real diagonal state).
 *
 * "Jamba — SSM-Transformer Híbrido", section "Mamba-3: a linha de base de SSM puro
 * em 2026", item 1: Mamba-3 replaces the Euler discretisation (Bbar = dt B, above)
 * by a more expressive recurrence in which a convolution-like operation acts on the
 * state input inside the recurrence. The key-terms tables of the zh and hi lessons
 * ("Phase 10 · 21 Jamba hybrid SSM-Transformer") add that this recurrence subsumes
 * Mamba-2's Euler discretisation, so Euler must be one of its settings. No page gives
 * a formula; the reading taken here is the rule the name describes, with a weight.
 * Over a step of length dt the exact update of h' = A h + B(s) x(s) adds the integral
 * of exp(A (dt - s)) B(s) x(s) over [0, dt]. A two-point rule over the step's ends,
 * the current input with weight lambda and the older one (decayed across the step)
 * with weight 1 - lambda, gives
 *
 *     h_t = dA h_{t-1} + dt ((1 - lam_t) dA B_{t-1} x_{t-1} + lam_t B_t x_t),
 *     dA = exp(dt A):
 *
 * a two-tap filter over the state inputs B x. lam_t = 1 is Euler's step (the scan
 * above); lam_t = 1/2 is the trapezoid rule, the default (lam = NULL); a data-
 * dependent lam, like dt, makes the rule more expressive than either. The first
 * step's previous input is B_prev x_prev (NULL: zero, a sequence with no input
 * before it); a caller resuming a sequence passes the last step of the previous
 * part. y_t is as in the Euler scan. Order of operations:
 *     dA = exp(dt * A[d][n]);  wc = dt * lam;  wp = dt * (1 - lam);
 *     h[n] = (dA * h[n]) + ((wp * (dA * (Bp[n] * xp))) + (wc * (B[n] * x)));
 *     acc = acc + C[n] * h[n]  (n ascending);  y = acc + D[d] * x;  then the gate.
 * Layouts as above; lam [batch][L][Dn] like dt (NULL: 1/2 everywhere); x_prev
 * [batch][Dn], B_prev [batch][N].
 */
int oracle_scan_trap_f64(int64_t batch, int64_t L, int64_t Dn, int64_t N,
                         const double *x, const double *dt, const double *A,
                         const double *B, const double *C, const double *Dv,
                         const double *z, const double *h0,
                         const double *x_prev, const double *B_prev, const double *lam,
                         double *y, double *h_final)
{
    if (batch < 0 || L < 0 || Dn < 0 || N <= 0) return -1;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    if (!h) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
            /* the input before step 0 */
            const int has_prev = x_prev && B_prev;
            double xp = has_prev ? x_prev[b * Dn + d] : 0.0;
            const double *Bp = has_prev ? B_prev + b * N : NULL;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * Dn + d;
                const int64_t s = (b * L + t) * N;
                const double xv = x[i], dv = dt[i];
                const double lv = lam ? lam[i] : 0.5;
                const double wc = dv * lv, wp = dv * (1.0 - lv);
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * A[d * N + n]);
                    const double prev = Bp ? Bp[n] * xp : 0.0;
                    h[n] = dA * h[n] + (wp * (dA * prev) + wc * (B[s + n] * xv));
                    acc = acc + C[s + n] * h[n];
                }
                double yv = acc + Dv[d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
                xp = xv;
                Bp = B + s;
            }
            if (h_final)
                for (int64_t n = 0; n < N; ++n) h_final[(b * Dn + d) * N + n] = h[n];
        }
    }
    free(h);
    return 0;
}

/* One decode token of the exponential-trapezoidal recurrence; h updated in place.
 * x_prev [n_layers][n_seq][Dn] and B_prev [n_layers][n_seq][N] are the previous
 * token's x and B (NULL: no previous input); lam [n_layers][n_seq][Dn] is the token's
 * weight (NULL: 1/2). */
int oracle_step_trap_f64(int64_t n_layers, int64_t n_seq, int64_t Dn, int64_t N,
                         double *h, const double *x_prev, const double *B_prev,
                         const double *x, const double *dt, const double *lam,
                         const double *A, const double *B, const double *C,
                         const double *Dv, const double *z, double *y)
{
    if (n_layers < 0 || n_seq < 0 || Dn < 0 || N <= 0) return -1;
    const int has_prev = x_prev && B_prev;
    for (int64_t l = 0; l < n_layers; ++l) {
        for (int64_t q = 0; q < n_seq; ++q) {
            const int64_t s = (l * n_seq + q) * N;
            for (int64_t d = 0; d < Dn; ++d) {
                const int64_t i = (l * n_seq + q) * Dn + d;
                double *hs = h + i * N;
                const double *Ad = A + (l * Dn + d) * N;
                const double xv = x[i], dv = dt[i];
                const double lv = lam ? lam[i] : 0.5;
                const double wc = dv * lv, wp = dv * (1.0 - lv);
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * Ad[n]);
                    const double prev = has_prev ? B_prev[s + n] * x_prev[i] : 0.0;
                    hs[n] = dA * hs[n] + (wp * (dA * prev) + wc * (B[s + n] * xv));
                    acc = acc + C[s + n] * hs[n];
                }
                double yv = acc + Dv[l * Dn + d] * xv;
                if (z) yv = yv * silu(z[i]);
                y[i] = yv;
            }
        }
    }
    return 0;
}

/*
 * Multi-input multi-output (MIMO) projections, real diagonal state.
 *
 * "Jamba — SSM-Transformer Híbrido", section "Mamba-3: a linha de base de SSM puro
 * em 2026", item 3 (and the glossary entry "MIMO" of the zh and hi lesson pages):
 * Mamba-3 replaces the scalar per-feature projections with matrix-valued ones, for
 * more modelling power and better use of the hardware at inference without a longer
 * decode. The pages give no formula. The reading taken here: a channel's input and
 * output become R-vectors instead of scalars, and B_t, C_t become N x R matrices
 * (the projections into and out of the N-wide state), so
 *
 *     h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + dt_t sum_r B_t[n][r] x_t[r]
 *     y_t[r] = (sum_n C_t[n][r] h_t[n] + D x_t[r]) * silu(z_t[r])
 *
 * The state per channel keeps its size N, so the decode step moves the same state
 * bytes while doing R times the multiply-adds. R = 1 is the scan above, term for
 * term: the order of operations below reduces to it.
 *     dA = exp(dt * A[d][n]);  u = sum over r ascending of ((dt * B[n][r]) * x[r]);
 *     h[n] = (dA * h[n]) + u;  acc[r] = acc[r] + C[n][r] * h[n]   (n ascending)
 *     y[r] = acc[r] + D[d] * x[r];  if gated: y[r] = y[r] * silu(z[r])
 * Layouts: x, z, y [batch][L][Dn][R]; dt [batch][L][Dn]; B, C [batch][L][N][R];
 * A [Dn][N]; Dv [Dn]; h0, h_final [batch][Dn][N].
 */
int oracle_scan_mimo_f64(int64_t batch, int64_t L, int64_t Dn, int64_t N, int64_t R,
                         const double *x, const double *dt, const double *A,
                         const double *B, const double *C, const double *Dv,
                         const double *z, const double *h0,
                         double *y, double *h_final)
{
    if (batch < 0 || L < 0 || Dn < 0 || N <= 0 || R <= 0) return -1;
    double *h = (double *)malloc((size_t)(N + R) * sizeof(double));
    if (!h) return -1;
    double *acc = h + N;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < Dn; ++d) {
            for (int64_t n = 0; n < N; ++n)
                h[n] = h0 ? h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * Dn + d;        /* (b, t, d) of dt */
                const double *xv = x + i * R;                 /* (b, t, d, 0) */
                const double *Bt = B + (b * L + t) * N * R;   /* (b, t, 0, 0) */
                const double *Ct = C + (b * L + t) * N * R;
                const double dv = dt[i];
                for (int64_t r = 0; r < R; ++r) acc[r] = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * A[d * N + n]);
                    double u = 0.0;
                    for (int64_t r = 0; r < R; ++r) u = u + (dv * Bt[n * R + r]) * xv[r];
                    h[n] = dA * h[n] + u;
                    for (int64_t r = 0; r < R; ++r) acc[r] = acc[r] + Ct[n * R + r] * h[n];
                }
                for (int64_t r = 0; r < R; ++r) {
                    double yv = acc[r] + Dv[d] * xv[r];
                    if (z) yv = yv * silu(z[i * R + r]);
                    y[i * R + r] = yv;
                }
            }
            if (h_final)
                for (int64_t n = 0; n < N; ++n) h_final[(b * Dn + d) * N + n] = h[n];
        }
    }
    free(h);
    return 0;
}

/* One MIMO decode token for every (layer, sequence, channel); h updated in place.
 * h [n_layers][n_seq][Dn][N]; x, z, y [n_layers][n_seq][Dn][R]; dt [n_layers][n_seq][Dn];
 * B, C [n_layers][n_seq][N][R]; A [n_layers][Dn][N]; Dv [n_layers][Dn]. */
int oracle_step_mimo_f64(int64_t n_layers, int64_t n_seq, int64_t Dn, int64_t N, int64_t R,
                         double *h, const double *x, const double *dt, const double *A,
                         const double *B, const double *C, const double *Dv,
                         const double *z, double *y)
{
    if (n_layers < 0 || n_seq < 0 || Dn < 0 || N <= 0 || R <= 0) return -1;
    double *acc = (double *)malloc((size_t)R * sizeof(double));
    if (!acc) return -1;
    for (int64_t l = 0; l < n_layers; ++l) {
        for (int64_t q = 0; q < n_seq; ++q) {
            const double *Bt = B + (l * n_seq + q) * N * R;
            const double *Ct = C + (l * n_seq + q) * N * R;
            for (int64_t d = 0; d < Dn; ++d) {
                const int64_t i = (l * n_seq + q) * Dn + d;
                double *hs = h + i * N;
                const double *Ad = A + (l * Dn + d) * N;
                const double *xv = x + i * R;
                const double dv = dt[i];
                for (int64_t r = 0; r < R; ++r) acc[r] = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA = exp(dv * Ad[n]);
                    double u = 0.0;
                    for (int64_t r = 0; r < R; ++r) u = u + (dv * Bt[n * R + r]) * xv[r];
                    hs[n] = dA * hs[n] + u;
                    for (int64_t r = 0; r < R; ++r) acc[r] = acc[r] + Ct[n * R + r] * hs[n];
                }
                for (int64_t r = 0; r < R; ++r) {
                    double yv = acc[r] + Dv[l * Dn + d] * xv[r];
                    if (z) yv = yv * silu(z[i * R + r]);
                    y[i * R + r] = yv;
                }
            }
        }
    }
    free(acc);
    return 0;
}
