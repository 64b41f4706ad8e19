/*
 * Plain fp64 CPU oracle for packed variable-length conv1d + selective scan.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no
 * code, header, table or helper with the HIP library, and it never runs on
 * the product path.
 *
 * Sources (pages, by address):
 *   [P5] Shanghai AI Lab HPC/NDS article on packed variable-length Mamba-1
 *        training, https://gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html
 *   [P1] practitioner article on variable-length Mamba-1 training,
 *        https://lpnh.cn/news/2780078
 *
 * What is computed is the plain definition the packed method is meant to
 * reach: every packed sequence behaves exactly as if it were run alone with
 * zero initial conv and SSM state ([P5] "Mamba block中的步骤": only the
 * sequence-wise steps see neighbouring tokens; [P5] "基本原理": reset the SSM
 * state at every sequence boundary; [P1] section 3.2: zero states at each
 * document start). Every loop below walks tokens in packed order and applies
 * that reset at the head tokens, so packed and per-sequence runs execute the
 * same floating-point operations in the same order.
 *
 * Inputs are fp64 arrays (the caller widens the stored bf16/fp32 bits
 * exactly). Layouts are token-major: a (T, D) array has element (t, d) at
 * t*D + d; B and C are (T, N); A is (D, N); the conv weight is (D, W) with
 * w[d*W + W-1] multiplying the current token (PyTorch depthwise conv1d
 * cross-correlation order). Channel ranges [d0, d1) let a caller split the
 * channels over threads; channels never interact except through the sums
 * dB and dC, which each call accumulates into the buffers it is given.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_CU_SEQLENS 3
#define ORACLE_ERR_ALLOC 6

/*
 * Error-scale mode of the backward functions. With it on, every sum they
 * form (over tokens, channels, states, taps, and the recursions over time)
 * adds the absolute value of each term instead of the term, and products
 * take the absolute value of their signed factors; the nonlinear factors
 * (sigmoid, the SiLU derivative, exp) keep their values. Each output is then
 * the sum of the magnitudes of the terms that make it up: the scale of the
 * rounding error of any evaluation of that sum, which a comparison of a sum
 * that cancels needs in place of the size of its result. Off, term() is the
 * identity and every expression rounds exactly as written. Process-wide; set
 * it only while no oracle call runs.
 */
static int g_abs_terms = 0;
void oracle_set_abs_terms(int on) { g_abs_terms = on != 0; }
static double term(double v) { return g_abs_terms ? fabs(v) : v; }

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
/* softplus(v) = log(1 + exp(v)), in a form that neither overflows nor loses
 * the tail: max(v, 0) + log1p(exp(-|v|)) */
static double softplus(double v) { return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v))); }

/* Step size as the scan uses it: delta_eff = softplus(delta + bias[d]) when
 * softplus is set, else delta + bias[d] (bias may be NULL). Its derivative
 * with respect to the stored delta is sigmoid(delta + bias[d]), or 1. */
static double delta_eff(double raw, const double *bias, int32_t d, int sp)
{
    const double v = raw + (bias ? bias[d] : 0.0);
    return sp ? softplus(v) : v;
}
static double delta_grad(double raw, const double *bias, int32_t d, int sp)
{
    return sp ? sigmoid(raw + (bias ? bias[d] : 0.0)) : 1.0;
}

/*
 * position_indices from cu_seqlens. [P5] "conv1d_pack 算子": pack() emits, for
 * every packed token, its position inside its own sequence; lengths
 * [4,2,3,7] give 0,1,2,3,0,1,0,1,2,0,1,2,3,4,5,6. cu_seqlens follows the
 * FlashAttention varlen convention ([P5] "基本原理"): cu[0] = 0, cu[nseq] = T,
 * non-decreasing (zero-length sequences allowed).
 * head[t] = 1 marks the first token of a sequence (pos 0).
 */
int oracle_pack_indices(const int32_t *cu, int32_t nseq, int64_t T, int32_t *pos, uint8_t *head)
{
    if (nseq < 0 || T < 0) return ORACLE_ERR_CU_SEQLENS;
    if (cu[0] != 0 || (int64_t)cu[nseq] != T) return ORACLE_ERR_CU_SEQLENS;
    for (int32_t s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return ORACLE_ERR_CU_SEQLENS;
    for (int32_t s = 0; s < nseq; ++s) {
        for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
            pos[t] = (int32_t)(t - cu[s]);
            if (head) head[t] = (t == cu[s]) ? 1 : 0;
        }
    }
    return ORACLE_OK;
}

/*
 * conv1d_pack forward. [P5] "conv1d_pack 算子": the causal depthwise conv looks
 * back W-1 tokens and must stop at its sequence's head token. Tap k (k tokens
 * back) contributes iff k <= pos[t], i.e. iff token t-k lies in the same
 * sequence. Result: the zero-left-padded causal conv of each sequence alone.
 *   v[t,d] = b[d] + sum_{k=0}^{W-1} [k <= pos[t]] * w[d, W-1-k] * x[t-k, d]
 *   u[t,d] = silu ? v * sigmoid(v) : v
 * b may be NULL (no bias). v may be NULL.
 */
void oracle_conv_fwd(int64_t T, int32_t D, int32_t W, const int32_t *pos,
                     const double *x, const double *w, const double *b, int silu,
                     int32_t d0, int32_t d1, double *v, double *u)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t d = d0; d < d1; ++d) {
            double acc = b ? b[d] : 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (k <= pos[t]) acc += w[(int64_t)d * W + (W - 1 - k)] * x[(t - k) * D + d];
            if (v) v[t * D + d] = acc;
            u[t * D + d] = silu ? acc * sigmoid(acc) : acc;
        }
    }
}

/*
 * Selective scan forward with resets. [P5] "SSM_pack算子" and "基本原理": state
 * flows across packed sequences only through the recurrence, so the state is
 * reset at every head token. The recurrence is Mamba-1's discretised form
 * (exp(delta*A) decay, delta*B*u input), per channel d and state n:
 *   h_t = head(t) ? delta_t B_t u_t : exp(delta_t A) h_{t-1} + delta_t B_t u_t
 *   y_t = sum_n C_t[n] h_t[n] + Dp[d] u_t
 *   out_t = y_t * (silu(z_t) + gate_floor)        (no gate when z is NULL)
 * The gate floor is [P4] "修法" GateFloor: a positive offset on the gate so
 * it stays above zero at zero input (0 = the plain SiLU gate). delta_t is the
 * step as stored, or softplus(stored + bias) (delta_eff above).
 * At a head the previous state is not read at all (a select, not a multiply
 * by zero), so a non-finite state can never cross a boundary.
 * Dp may be NULL (no skip). y and hs may be NULL; hs receives every state,
 * (T, D, N) at ((t*D)+d)*N + n, for small inspection cases.
 */
int oracle_scan_fwd_ex(int64_t T, int32_t D, int32_t N, const int32_t *pos,
                       const double *u, const double *delta, const double *A,
                       const double *B, const double *C, const double *Dp, const double *z,
                       const double *dbias, int32_t sp, double gate_floor,
                       int32_t d0, int32_t d1, double *y, double *out, double *hs)
{
    double *h = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    if (!h) return ORACLE_ERR_ALLOC;
    for (int32_t d = d0; d < d1; ++d) {
        for (int64_t t = 0; t < T; ++t) {
            const int head = pos[t] == 0;
            const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
            const double uu = u[t * D + d];
            double acc = 0.0;
            for (int32_t n = 0; n < N; ++n) {
                const double bu = dt * B[t * N + n] * uu;
                if (head) {
                    h[n] = bu;
                } else {
                    const double a = exp(dt * A[(int64_t)d * N + n]);
                    h[n] = a * h[n] + bu;
                }
                acc += C[t * N + n] * h[n];
                if (hs) hs[(t * D + d) * N + n] = h[n];
            }
            if (Dp) acc += Dp[d] * uu;
            if (y) y[t * D + d] = acc;
            out[t * D + d] = z ? acc * (z[t * D + d] * sigmoid(z[t * D + d]) + gate_floor) : acc;
        }
    }
    free(h);
    return ORACLE_OK;
}

int oracle_scan_fwd(int64_t T, int32_t D, int32_t N, const int32_t *pos,
                    const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *Dp, const double *z,
                    int32_t d0, int32_t d1, double *y, double *out, double *hs)
{
    return oracle_scan_fwd_ex(T, D, N, pos, u, delta, A, B, C, Dp, z, NULL, 0, 0.0, d0, d1, y, out, hs);
}

/*
 * Selective scan backward: the chain rule of oracle_scan_fwd, written out.
 * Given dout = dL/dout (T, D):
 *   g = dout * (silu(z) + gate_floor)       (dL/dy)
 *   dz = dout * y * s * (1 + z (1 - s)),  s = sigmoid(z)
 *   dDp[d] = sum_t g u,   du starts at g * Dp[d]
 * then per state n, t descending, with carry c (dL/dh_t through h_{t+1}):
 *   dh = g C_t[n] + c
 *   dC[t,n] += g h_t[n]
 *   dB[t,n] += dh delta_t u_t
 *   du[t]   += dh delta_t B_t[n]
 *   ddelta[t] += dh (B_t[n] u_t + [not head] A a_t h_{t-1})
 *   dA[d,n] += [not head] dh delta_t a_t h_{t-1}
 *   c = [not head] a_t dh        ([P5] "基本原理": no gradient crosses a head)
 * with a_t = exp(delta_t A[d,n]). ddelta is returned with respect to the
 * stored delta (times sigmoid(delta + bias) under softplus), and ddbias[d] is
 * its sum over t. dB and dC (T, N) are ACCUMULATED into (the caller zeroes
 * them, and sums per-thread buffers); all other outputs are overwritten for
 * channels [d0, d1). Dp, z, dbias may be NULL; dz, ddbias may be NULL.
 */
int oracle_scan_bwd_ex(int64_t T, int32_t D, int32_t N, const int32_t *pos,
                       const double *u, const double *delta, const double *A,
                       const double *B, const double *C, const double *Dp, const double *z,
                       const double *dbias, int32_t sp, double gate_floor,
                       const double *dout, int32_t d0, int32_t d1,
                       double *du, double *ddelta, double *dA, double *dB, double *dC,
                       double *dDp, double *dz, double *ddbias)
{
    double *hs = (double *)malloc((size_t)(T > 0 ? T : 1) * (size_t)(N > 0 ? N : 1) * sizeof(double));
    double *ys = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    double *c = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    if (!hs || !ys || !c) { free(hs); free(ys); free(c); return ORACLE_ERR_ALLOC; }
    for (int32_t d = d0; d < d1; ++d) {
        /* forward, keeping every state of this channel */
        for (int64_t t = 0; t < T; ++t) {
            const int head = pos[t] == 0;
            const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
            const double uu = u[t * D + d];
            double acc = 0.0;
            for (int32_t n = 0; n < N; ++n) {
                const double bu = dt * B[t * N + n] * uu;
                double hn;
                if (head) {
                    hn = term(bu);
                } else {
                    const double a = exp(dt * A[(int64_t)d * N + n]);
                    hn = a * hs[(t - 1) * N + n] + term(bu);
                }
                hs[t * N + n] = hn;
                acc += term(C[t * N + n] * hn);
            }
            if (Dp) acc += term(Dp[d] * uu);
            ys[t] = acc;
        }
        /* reverse */
        for (int32_t n = 0; n < N; ++n) c[n] = 0.0;
        double dDp_acc = 0.0;
        double *dA_d = dA + (int64_t)d * N;
        for (int32_t n = 0; n < N; ++n) dA_d[n] = 0.0;
        double ddb_acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const int head = pos[t] == 0;
            const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
            const double uu = u[t * D + d];
            const double go = dout[t * D + d];
            double g = go;
            if (z) {
                const double zz = z[t * D + d];
                const double s = sigmoid(zz);
                g = term(go) * (term(zz * s) + gate_floor);
                if (dz) dz[t * D + d] = term(go * ys[t] * s * (1.0 + zz * (1.0 - s)));
            } else if (dz) {
                dz[t * D + d] = 0.0;
            }
            double du_acc = Dp ? term(g * Dp[d]) : 0.0;
            double ddt = 0.0;
            dDp_acc += term(g * uu);
            for (int32_t n = 0; n < N; ++n) {
                const double Bn = B[t * N + n];
                const double dh = term(g * C[t * N + n]) + c[n];
                dC[t * N + n] += term(g * hs[t * N + n]);
                dB[t * N + n] += term(dh * dt * uu);
                du_acc += term(dh * dt * Bn);
                if (head) {
                    ddt += term(dh * (Bn * uu));
                    c[n] = 0.0;
                } else {
                    const double An = A[(int64_t)d * N + n];
                    const double a = exp(dt * An);
                    const double hp = hs[(t - 1) * N + n];
                    ddt += term(dh) * (term(Bn * uu) + term(An * a * hp));
                    dA_d[n] += term(dh * dt * a * hp);
                    c[n] = a * dh;
                }
            }
            du[t * D + d] = du_acc;
            /* through the step map: d delta_eff / d delta */
            const double ddraw = ddt * delta_grad(delta[t * D + d], dbias, d, sp);
            ddelta[t * D + d] = ddraw;
            ddb_acc += term(ddraw);
        }
        if (dDp) dDp[d] = dDp_acc;
        if (ddbias) ddbias[d] = ddb_acc;
    }
    free(hs); free(ys); free(c);
    return ORACLE_OK;
}

int oracle_scan_bwd(int64_t T, int32_t D, int32_t N, const int32_t *pos,
                    const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *Dp, const double *z,
                    const double *dout, int32_t d0, int32_t d1,
                    double *du, double *ddelta, double *dA, double *dB, double *dC,
                    double *dDp, double *dz)
{
    return oracle_scan_bwd_ex(T, D, N, pos, u, delta, A, B, C, Dp, z, NULL, 0, 0.0, dout, d0, d1,
                              du, ddelta, dA, dB, dC, dDp, dz, NULL);
}

/*
 * conv1d_pack backward: the chain rule of oracle_conv_fwd. [P5]
 * "conv1d_pack 算子": dx and dweight need the same early stop, and the
 * backward needs the position W-1 tokens ahead: token s receives from token
 * s+k only if pos[s+k] >= k (s+k is in the same sequence as s).
 *   gv[t] = silu ? du[t] * s(v) * (1 + v (1 - s(v))) : du[t],  s = sigmoid
 *   db[d]        = sum_t gv[t]
 *   dw[d, W-1-k] = sum_t [k <= pos[t]] gv[t] x[t-k]
 *   dx[s]        = sum_k [s+k < T and k <= pos[s+k]] w[d, W-1-k] gv[s+k]
 * b may be NULL; db may be NULL. Overwrites outputs for channels [d0, d1).
 */
int oracle_conv_bwd(int64_t T, int32_t D, int32_t W, const int32_t *pos,
                    const double *x, const double *w, const double *b, int silu,
                    const double *du, int32_t d0, int32_t d1,
                    double *dx, double *dw, double *db)
{
    double *gv = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    if (!gv) return ORACLE_ERR_ALLOC;
    for (int32_t d = d0; d < d1; ++d) {
        for (int64_t t = 0; t < T; ++t) {
            double v = b ? b[d] : 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (k <= pos[t]) v += w[(int64_t)d * W + (W - 1 - k)] * x[(t - k) * D + d];
            const double g = du[t * D + d];
            if (silu) {
                const double s = sigmoid(v);
                gv[t] = term(g * s * (1.0 + v * (1.0 - s)));
            } else {
                gv[t] = term(g);
            }
        }
        double dbd = 0.0;
        for (int64_t t = 0; t < T; ++t) dbd += gv[t];
        if (db) db[d] = dbd;
        for (int32_t k = 0; k < W; ++k) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t)
                if (k <= pos[t]) acc += term(gv[t] * x[(t - k) * D + d]);
            dw[(int64_t)d * W + (W - 1 - k)] = acc;
        }
        for (int64_t s = 0; s < T; ++s) {
            double acc = 0.0;
            for (int32_t k = 0; k < W; ++k)
                if (s + k < T && k <= pos[s + k]) acc += term(w[(int64_t)d * W + (W - 1 - k)] * gv[s + k]);
            dx[s * D + d] = acc;
        }
    }
    free(gv);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Sequences that continue across packs.
 *
 * [P5] "结论与讨论" proposes cutting a sequence that overruns a pack into two
 * pieces that keep passing state, so that packs need no padding; [P1]
 * section 3.2 describes segment-wise runs that reset, or hand on, the conv
 * and SSM states at segment starts. The plain definition: sequence s runs
 * alone, but starting from a given SSM state h0[s] (instead of zero) and with
 * the W-1 inputs that precede it, xc0[s], visible to the causal conv
 * (instead of zeros); it hands on its final SSM state hT[s] and its last W-1
 * conv inputs xcT[s]. A piece that continues a sequence, given the previous
 * piece's hT and xcT, then computes exactly what the uncut sequence would.
 *
 * These functions walk each sequence's tokens [cu[s], cu[s+1]) directly.
 * State layouts: h0, hT, dhT, dh0 are (nseq, D, N) at (s*D + d)*N + n;
 * xc0, xcT, dxcT, dxc0 are (nseq, W-1, D) at (s*(W-1) + j)*D + d, j = 0 the
 * oldest input, j = W-2 the one just before the sequence's first token.
 * Every state pointer may be NULL: a NULL initial state is zero, a NULL
 * final-state gradient is zero, a NULL output is not written.
 * ------------------------------------------------------------------------ */

/* Input i of sequence s's extended input [xc0[s]; x[cu[s]:cu[s+1]]]:
 * x itself for i >= cu[s], the conv context for cu[s]-(W-1) <= i < cu[s]. */
static double conv_input(const double *x, const double *xc0, const int32_t *cu, int32_t s,
                         int64_t i, int32_t D, int32_t W, int32_t d)
{
    if (i >= cu[s]) return x[i * D + d];
    if (!xc0) return 0.0;
    const int64_t j = i - ((int64_t)cu[s] - (W - 1));
    return xc0[((int64_t)s * (W - 1) + j) * D + d];
}

/*
 * conv1d_pack forward with conv context per sequence:
 *   v[t,d] = b[d] + sum_{k=0}^{W-1} w[d, W-1-k] * X_s(t-k)
 * where X_s is the extended input above (taps that reach before the
 * context's start do not exist: k <= W-1 never does). xcT[s][j] = X_s(cu[s+1]
 * - (W-1) + j): the last W-1 inputs of the extended sequence.
 * With xc0 NULL this is oracle_conv_fwd term for term.
 */
int oracle_conv_fwd_state(int64_t T, int32_t D, int32_t W, const int32_t *cu, int32_t nseq,
                          const double *x, const double *w, const double *b, int silu,
                          const double *xc0, int32_t d0, int32_t d1, double *v, double *u, double *xcT)
{
    if (cu[0] != 0 || (int64_t)cu[nseq] != T) return ORACLE_ERR_CU_SEQLENS;
    for (int32_t s = 0; s < nseq; ++s) {
        if (cu[s + 1] < cu[s]) return ORACLE_ERR_CU_SEQLENS;
        for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
            for (int32_t d = d0; d < d1; ++d) {
                double acc = b ? b[d] : 0.0;
                for (int32_t k = 0; k < W; ++k) {
                    if (t - k < cu[s] && !xc0) continue;  /* zero context: no term */
                    acc += w[(int64_t)d * W + (W - 1 - k)] * conv_input(x, xc0, cu, s, t - k, D, W, d);
                }
                if (v) v[t * D + d] = acc;
                u[t * D + d] = silu ? acc * sigmoid(acc) : acc;
            }
        }
        if (xcT) {
            for (int32_t j = 0; j < W - 1; ++j)
                for (int32_t d = d0; d < d1; ++d)
                    xcT[((int64_t)s * (W - 1) + j) * D + d] =
                        conv_input(x, xc0, cu, s, (int64_t)cu[s + 1] - (W - 1) + j, D, W, d);
        }
    }
    return ORACLE_OK;
}

/*
 * conv1d_pack backward with conv context: the chain rule of
 * oracle_conv_fwd_state for the loss sum(du * u) + sum(dxcT * xcT).
 *   gv[t]         = du[t] * silu'(v[t])   (du[t] when silu is off)
 *   db[d]         = sum_t gv[t]
 *   dw[d, W-1-k]  = sum_t gv[t] X_s(t-k)
 *   dX_s(i)       = sum_{k : cu[s] <= i+k < cu[s+1]} w[d, W-1-k] gv[i+k]
 *                   + dxcT[s][i - (cu[s+1] - (W-1))]  when that index is in 0..W-2
 * and dX_s(i) lands in dx[i] (i >= cu[s]) or dxc0[s][i - (cu[s] - (W-1))].
 * dxcT, xc0 may be NULL; dxc0, db may be NULL. Overwrites its outputs for
 * channels [d0, d1).
 */
int oracle_conv_bwd_state(int64_t T, int32_t D, int32_t W, const int32_t *cu, int32_t nseq,
                          const double *x, const double *w, const double *b, int silu,
                          const double *xc0, const double *du, const double *dxcT,
                          int32_t d0, int32_t d1, double *dx, double *dw, double *db, double *dxc0)
{
    if (cu[0] != 0 || (int64_t)cu[nseq] != T) return ORACLE_ERR_CU_SEQLENS;
    double *gv = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    if (!gv) return ORACLE_ERR_ALLOC;
    for (int32_t d = d0; d < d1; ++d) {
        double dbd = 0.0;
        for (int32_t s = 0; s < nseq; ++s) {
            for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
                double vv = b ? b[d] : 0.0;
                for (int32_t k = 0; k < W; ++k) {
                    if (t - k < cu[s] && !xc0) continue;
                    vv += w[(int64_t)d * W + (W - 1 - k)] * conv_input(x, xc0, cu, s, t - k, D, W, d);
                }
                const double g = du[t * D + d];
                if (silu) {
                    const double sg = sigmoid(vv);
                    gv[t] = term(g * sg * (1.0 + vv * (1.0 - sg)));
                } else {
                    gv[t] = term(g);
                }
            }
        }
        for (int64_t t = 0; t < T; ++t) dbd += gv[t];
        for (int32_t k = 0; k < W; ++k) {
            double acc = 0.0;
            for (int32_t s = 0; s < nseq; ++s)
                for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
                    if (t - k < cu[s] && !xc0) continue;
                    acc += term(gv[t] * conv_input(x, xc0, cu, s, t - k, D, W, d));
                }
            dw[(int64_t)d * W + (W - 1 - k)] = acc;
        }
        /* gradient of every extended input, context first */
        for (int32_t s = 0; s < nseq; ++s) {
            const int64_t a = cu[s], e = cu[s + 1];
            for (int64_t i = a - (W - 1); i < e; ++i) {
                double acc = 0.0;
                for (int32_t k = 0; k < W; ++k)
                    if (i + k >= a && i + k < e) acc += term(w[(int64_t)d * W + (W - 1 - k)] * gv[i + k]);
                const int64_t jt = i - (e - (W - 1));
                if (dxcT && jt >= 0 && jt < W - 1) acc += term(dxcT[((int64_t)s * (W - 1) + jt) * D + d]);
                if (i >= a) {
                    dx[i * D + d] = acc;
                } else if (dxc0) {
                    dxc0[((int64_t)s * (W - 1) + (i - (a - (W - 1)))) * D + d] = acc;
                }
            }
        }
        if (db) db[d] = dbd;
    }
    free(gv);
    return ORACLE_OK;
}

/*
 * Selective scan forward with an initial SSM state per sequence: the
 * recurrence of oracle_scan_fwd_ex started from h_{cu[s]-1} = h0[s]:
 *   h_t = exp(delta_t A) h_{t-1} + delta_t B_t u_t   for t in [cu[s], cu[s+1])
 * and hT[s] = the state after the sequence's last token (h0[s], or zero, for
 * an empty sequence). Outputs as oracle_scan_fwd_ex.
 */
int oracle_scan_fwd_state(int64_t T, int32_t D, int32_t N, const int32_t *cu, int32_t nseq,
                          const double *u, const double *delta, const double *A,
                          const double *B, const double *C, const double *Dp, const double *z,
                          const double *dbias, int32_t sp, double gate_floor, const double *h0,
                          int32_t d0, int32_t d1, double *y, double *out, double *hT)
{
    if (cu[0] != 0 || (int64_t)cu[nseq] != T) return ORACLE_ERR_CU_SEQLENS;
    for (int32_t s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return ORACLE_ERR_CU_SEQLENS;
    double *h = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    if (!h) return ORACLE_ERR_ALLOC;
    for (int32_t d = d0; d < d1; ++d) {
        for (int32_t s = 0; s < nseq; ++s) {
            for (int32_t n = 0; n < N; ++n) h[n] = h0 ? h0[((int64_t)s * D + d) * N + n] : 0.0;
            for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
                const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
                const double uu = u[t * D + d];
                double acc = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    const double a = exp(dt * A[(int64_t)d * N + n]);
                    h[n] = a * h[n] + dt * B[t * N + n] * uu;
                    acc += C[t * N + n] * h[n];
                }
                if (Dp) acc += Dp[d] * uu;
                if (y) y[t * D + d] = acc;
                out[t * D + d] = z ? acc * (z[t * D + d] * sigmoid(z[t * D + d]) + gate_floor) : acc;
            }
            if (hT)
                for (int32_t n = 0; n < N; ++n) hT[((int64_t)s * D + d) * N + n] = h[n];
        }
    }
    free(h);
    return ORACLE_OK;
}

/*
 * Selective scan backward with states: the chain rule of
 * oracle_scan_fwd_state for the loss sum(dout * out) + sum(dhT * hT). Per
 * sequence the reverse carry starts from dhT[s] (zero when NULL) at its last
 * token; at the first token the previous state is h0[s]; what the carry holds
 * after the first token is dL/dh0[s] (dhT[s] for an empty sequence).
 * Sequences are walked last to first and tokens last to first, so the sums
 * dA, dDp, ddbias are formed in the order oracle_scan_bwd_ex forms them.
 * Other conventions as oracle_scan_bwd_ex; dh0 may be NULL.
 */
int oracle_scan_bwd_state(int64_t T, int32_t D, int32_t N, const int32_t *cu, int32_t nseq,
                          const double *u, const double *delta, const double *A,
                          const double *B, const double *C, const double *Dp, const double *z,
                          const double *dbias, int32_t sp, double gate_floor, const double *h0,
                          const double *dout, const double *dhT, int32_t d0, int32_t d1,
                          double *du, double *ddelta, double *dA, double *dB, double *dC,
                          double *dDp, double *dz, double *ddbias, double *dh0)
{
    if (cu[0] != 0 || (int64_t)cu[nseq] != T) return ORACLE_ERR_CU_SEQLENS;
    for (int32_t s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return ORACLE_ERR_CU_SEQLENS;
    double *hs = (double *)malloc((size_t)(T > 0 ? T : 1) * (size_t)(N > 0 ? N : 1) * sizeof(double));
    double *ys = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    double *c = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    double *hinit = (double *)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
    if (!hs || !ys || !c || !hinit) { free(hs); free(ys); free(c); free(hinit); return ORACLE_ERR_ALLOC; }
    for (int32_t d = d0; d < d1; ++d) {
        /* forward, keeping every state of this channel */
        for (int32_t s = 0; s < nseq; ++s) {
            for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
                const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
                const double uu = u[t * D + d];
                double acc = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    const double hp = (t == cu[s]) ? (h0 ? term(h0[((int64_t)s * D + d) * N + n]) : 0.0)
                                                   : hs[(t - 1) * N + n];
                    const double hn = exp(dt * A[(int64_t)d * N + n]) * hp + term(dt * B[t * N + n] * uu);
                    hs[t * N + n] = hn;
                    acc += term(C[t * N + n] * hn);
                }
                if (Dp) acc += term(Dp[d] * uu);
                ys[t] = acc;
            }
        }
        /* reverse, sequence by sequence */
        double dDp_acc = 0.0, ddb_acc = 0.0;
        double *dA_d = dA + (int64_t)d * N;
        for (int32_t n = 0; n < N; ++n) dA_d[n] = 0.0;
        for (int32_t s = nseq - 1; s >= 0; --s) {
            for (int32_t n = 0; n < N; ++n) {
                c[n] = dhT ? term(dhT[((int64_t)s * D + d) * N + n]) : 0.0;
                hinit[n] = h0 ? term(h0[((int64_t)s * D + d) * N + n]) : 0.0;
            }
            for (int64_t t = (int64_t)cu[s + 1] - 1; t >= cu[s]; --t) {
                const double dt = delta_eff(delta[t * D + d], dbias, d, sp);
                const double uu = u[t * D + d];
                const double go = dout[t * D + d];
                double g = go;
                if (z) {
                    const double zz = z[t * D + d];
                    const double sg = sigmoid(zz);
                    g = term(go) * (term(zz * sg) + gate_floor);
                    if (dz) dz[t * D + d] = term(go * ys[t] * sg * (1.0 + zz * (1.0 - sg)));
                } else if (dz) {
                    dz[t * D + d] = 0.0;
                }
                double du_acc = Dp ? term(g * Dp[d]) : 0.0;
                double ddt = 0.0;
                dDp_acc += term(g * uu);
                for (int32_t n = 0; n < N; ++n) {
                    const double Bn = B[t * N + n], An = A[(int64_t)d * N + n];
                    const double dh = term(g * C[t * N + n]) + c[n];
                    const double a = exp(dt * An);
                    const double hp = (t == cu[s]) ? hinit[n] : hs[(t - 1) * N + n];
                    dC[t * N + n] += term(g * hs[t * N + n]);
                    dB[t * N + n] += term(dh * dt * uu);
                    du_acc += term(dh * dt * Bn);
                    ddt += term(dh) * (term(Bn * uu) + term(An * a * hp));
                    dA_d[n] += term(dh * dt * a * hp);
                    c[n] = a * dh;
                }
                du[t * D + d] = du_acc;
                const double ddraw = ddt * delta_grad(delta[t * D + d], dbias, d, sp);
                ddelta[t * D + d] = ddraw;
                ddb_acc += term(ddraw);
            }
            if (dh0)
                for (int32_t n = 0; n < N; ++n) dh0[((int64_t)s * D + d) * N + n] = c[n];
        }
        if (dDp) dDp[d] = dDp_acc;
        if (ddbias) ddbias[d] = ddb_acc;
    }
    free(hs); free(ys); free(c); free(hinit);
    return ORACLE_OK;
}
