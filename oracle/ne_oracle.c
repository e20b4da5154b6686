/*
 * ne_oracle.c -- double-precision CPU oracle for causal grouped-query attention
 * with rotary position embeddings (RoPE), forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where the pages state it:
 *   - RoPE applied to queries and keys: "NanoEuler: 使用 C 和 CUDA 从零开始构建的
 *     GPT-2 规模 LLM" (agentlenshq), section "技术规格" (technical specs).
 *   - Grouped-query attention: a smaller set of key/value heads is shared by
 *     groups of query heads -- same page, "技术规格" and the table "模型配置"
 *     (12 q / 4 kv heads on the GPU model, 4 / 2 on the CPU model).
 *   - Decoder-only transformer, hence a causal mask -- same page, "核心架构与设计".
 *   - The tiled online-softmax kernel computes exactly softmax attention without
 *     storing the T x T matrix -- same page, "内核实现"; and "用 100KB C/CUDA 单文件
 *     复刻 GPT-2:NanoEuler 116M 单卡可跑的全流程拆解" (cnblogs), section 3.4
 *     "FlashAttention 是性能关键".  The oracle is the plain definition that the
 *     tiled kernel reaches: it DOES store the full masked T x T matrix.
 *   - Hand-written backward checked in double precision -- agentlenshq page,
 *     "验证与稳定性"; cnblogs page, section 2.1 "编译 + gradient check".
 *   - QK norm (the *_x entry points): same guide, section 模型架构速览, the feature list entry
 *     on QK norm (q and k normalised, then scaled up by 1.2); see qk_norm_rows below.
 *   - Sliding-window attention (the *_w entry points): "nanochat 全栈 LLM 训练实践指南"
 *     (the nanochat guide), section "模型架构速览" (architecture overview), the feature
 *     list entry on window_pattern: "S" layers see a quarter of the context, "L" layers
 *     the full context.
 *
 * Readings taken where the pages are silent:
 *   RoPE pairs adjacent elements (2i, 2i+1) and rotates them by +t*theta_i with
 *   theta_i = base^(-2i/D), positions t = 0..T-1, over the whole head dimension;
 *   base <= 0 disables RoPE.  Softmax scale 1/sqrt(D) applied after RoPE.  Key j
 *   is visible to query i iff j <= i.  Query head h reads KV head h / (Hq/Hkv).
 *   LSE is the natural-log log-sum-exp of the scaled scores.  Gradients are
 *   returned with respect to the un-rotated q and k (inverse rotation R^T).
 *   A window of W > 0 keys means query i sees keys i - W + 1 .. i (its own position
 *   and the W - 1 before it); W <= 0 is the full causal prefix.
 *   The *_x entry points and ne_oracle_rope also take the other common pairing, the
 *   "half-split" one: element i is rotated with element i + D/2 by t*theta_i (same
 *   frequencies, same positions), i = 0..D/2-1.
 *
 * Layouts: q, o, dO, dq are [B][T][Hq][D]; k, v, dk, dv are [B][T][Hkv][D];
 * lse is [B][Hq][T].  All arrays are dense row-major doubles owned by the caller.
 *
 * Determinism: every output element is produced by exactly one thread in a fixed
 * summation order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(b, t, h, d, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (d))

static int check_shape(int B, int T, int Hq, int Hkv, int D, double base) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1) return 1;
    if (Hq % Hkv != 0) return 1;
    if (base > 0.0 && (D % 2) != 0) return 1;
    return 0;
}

/* First key visible to query i (window as in the header). */
static int first_key(int i, int window) {
    return (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
}

/* Last query row that sees key j. */
static int last_row(int j, int T, int window) {
    return (window > 0 && j + window - 1 < T - 1) ? j + window - 1 : T - 1;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Rotate one head's rows: y[t][:] = R_t x[t][:] (sign = +1) or R_t^T x[t][:]
 * (sign = -1).  x and y are [T][D] with row stride `stride` doubles.  With
 * base <= 0 the rotation is the identity.  cos/sin come from libm in double.
 * Rotary pair i is (2i, 2i+1), or (i, i + D/2) when half != 0. */
static void rope_rows(const double* x, size_t xstride, double* y, size_t ystride,
                      int T, int D, double base, int sign, int half) {
    for (int t = 0; t < T; ++t) {
        const double* xr = x + (size_t)t * xstride;
        double* yr = y + (size_t)t * ystride;
        if (base <= 0.0) {
            for (int d = 0; d < D; ++d) yr[d] = xr[d];
            continue;
        }
        for (int i = 0; i < D / 2; ++i) {
            double theta = pow(base, -2.0 * (double)i / (double)D);
            double phi = (double)t * theta;
            double c = cos(phi), s = sin(phi) * (double)sign;
            const int i0 = half ? i : 2 * i, i1 = half ? i + D / 2 : 2 * i + 1;
            double a = xr[i0], b = xr[i1];
            yr[i0] = a * c - b * s;
            yr[i1] = a * s + b * c;
        }
    }
}

/* Public helper so the tests can check the rotation on its own:
 * y = R x (inverse = 0) or y = R^T x (inverse = 1), x and y [B][T][H][D];
 * half_split selects the pairing (i, i + D/2). */
int ne_oracle_rope(const double* x, double* y, int B, int T, int H, int D,
                   double base, int inverse, int half_split) {
    if (B < 1 || T < 1 || H < 1 || D < 1 || (base > 0.0 && D % 2)) return 1;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            rope_rows(x + IDX4(b, 0, h, 0, T, H, D), (size_t)H * D,
                      y + IDX4(b, 0, h, 0, T, H, D), (size_t)H * D, T, D, base,
                      inverse ? -1 : 1, half_split);
    return 0;
}

/* Probabilities of one (batch, query head): P[i][j] = softmax_j(S[i][j]) over
 * the visible keys lo <= j <= i (lo = first_key(i, window)), S = q' k'^T / sqrt(D).
 * qr, kr are the rotated [T][D] rows.  Invisible entries are set to 0 and never
 * dotted.  lse_row[i] gets m_i + log(sum_j exp(S_ij - m_i)). */
static void softmax_probs(const double* qr, const double* kr, double* P,
                          double* lse_row, int T, int D, int window) {
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(dynamic, 8)
    for (int i = 0; i < T; ++i) {
        double* Pi = P + (size_t)i * T;
        const int lo = first_key(i, window);
        double m = -INFINITY;
        for (int j = 0; j < lo; ++j) Pi[j] = 0.0;
        for (int j = lo; j <= i; ++j) {
            double s = 0.0;
            for (int d = 0; d < D; ++d) s += qr[(size_t)i * D + d] * kr[(size_t)j * D + d];
            s *= scale;
            Pi[j] = s;
            if (s > m) m = s;
        }
        double l = 0.0;
        for (int j = lo; j <= i; ++j) {
            Pi[j] = exp(Pi[j] - m);
            l += Pi[j];
        }
        for (int j = lo; j <= i; ++j) Pi[j] /= l;
        for (int j = i + 1; j < T; ++j) Pi[j] = 0.0;
        lse_row[i] = m + log(l);
    }
}

/* Forward: o = softmax(mask(q' k'^T / sqrt(D))) v, lse as above; window W as in
 * the header (W <= 0: full causal prefix). */
static int fwd_impl(const double* q, const double* k, const double* v, double* o,
                    double* lse, int B, int T, int Hq, int Hkv, int D, double base,
                    int window, int half, int nthreads) {
    if (check_shape(B, T, Hq, Hkv, D, base)) return 1;
    set_threads(nthreads);
    const int G = Hq / Hkv;
    double* qr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* P = (double*)malloc(sizeof(double) * (size_t)T * T);
    if (!qr || !kr || !P) { free(qr); free(kr); free(P); return 2; }
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;  /* GQA: KV head shared by G consecutive query heads */
            rope_rows(q + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, qr, (size_t)D, T, D, base, 1, half);
            rope_rows(k + IDX4(b, 0, g, 0, T, Hkv, D), (size_t)Hkv * D, kr, (size_t)D, T, D, base, 1, half);
            softmax_probs(qr, kr, P, lse + ((size_t)b * Hq + h) * T, T, D, window);
#pragma omp parallel for schedule(static)
            for (int i = 0; i < T; ++i) {
                double* orow = o + IDX4(b, i, h, 0, T, Hq, D);
                for (int d = 0; d < D; ++d) orow[d] = 0.0;
                for (int j = first_key(i, window); j <= i; ++j) {
                    const double p = P[(size_t)i * T + j];
                    const double* vrow = v + IDX4(b, j, g, 0, T, Hkv, D);
                    for (int d = 0; d < D; ++d) orow[d] += p * vrow[d];
                }
            }
        }
    }
    free(qr); free(kr); free(P);
    return 0;
}

int ne_oracle_fwd_w(const double* q, const double* k, const double* v, double* o,
                    double* lse, int B, int T, int Hq, int Hkv, int D, double base,
                    int window, int nthreads) {
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, D, base, window, 0, nthreads);
}

int ne_oracle_fwd(const double* q, const double* k, const double* v, double* o,
                  double* lse, int B, int T, int Hq, int Hkv, int D, double base,
                  int nthreads) {
    return ne_oracle_fwd_w(q, k, v, o, lse, B, T, Hq, Hkv, D, base, 0, nthreads);
}

/* Backward, given dO: exact gradients of sum(o * dO) with respect to q, k, v.
 *   dP_ij = dO_i . v_j,   Delta_i = dO_i . o_i,   dS_ij = P_ij (dP_ij - Delta_i)
 *   dq'_i = sum_j dS_ij k'_j / sqrt(D)
 *   dk'_j = sum over heads h of the group, sum_i dS_ij q'_i / sqrt(D)
 *   dv_j  = sum over heads h of the group, sum_i P_ij dO_i
 *   dq = R^T dq',  dk = R^T dk'.
 * The heads of a group are accumulated in ascending order. */
static int bwd_impl(const double* q, const double* k, const double* v, const double* dO,
                    const double* o_given, double* dq, double* dk, double* dv, int B, int T,
                    int Hq, int Hkv, int D, double base, int window, int half, int nthreads);

int ne_oracle_bwd(const double* q, const double* k, const double* v, const double* dO,
                  double* dq, double* dk, double* dv, int B, int T, int Hq, int Hkv,
                  int D, double base, int nthreads) {
    return bwd_impl(q, k, v, dO, NULL, dq, dk, dv, B, T, Hq, Hkv, D, base, 0, 0, nthreads);
}

int ne_oracle_bwd_w(const double* q, const double* k, const double* v, const double* dO,
                    double* dq, double* dk, double* dv, int B, int T, int Hq, int Hkv,
                    int D, double base, int window, int nthreads) {
    return bwd_impl(q, k, v, dO, NULL, dq, dk, dv, B, T, Hq, Hkv, D, base, window, 0, nthreads);
}

/* The same backward with Delta_i = dO_i . o_i taken from a caller-supplied o ([B][T][Hq][D])
 * instead of the exact forward output: the function the library's backward computes when it
 * is handed an o stored in a narrower format.  Everything else is exact. */
int ne_oracle_bwd_given_o(const double* q, const double* k, const double* v, const double* o,
                          const double* dO, double* dq, double* dk, double* dv, int B, int T,
                          int Hq, int Hkv, int D, double base, int nthreads) {
    if (!o) return 1;
    return bwd_impl(q, k, v, dO, o, dq, dk, dv, B, T, Hq, Hkv, D, base, 0, 0, nthreads);
}

int ne_oracle_bwd_given_o_w(const double* q, const double* k, const double* v, const double* o,
                            const double* dO, double* dq, double* dk, double* dv, int B, int T,
                            int Hq, int Hkv, int D, double base, int window, int nthreads) {
    if (!o) return 1;
    return bwd_impl(q, k, v, dO, o, dq, dk, dv, B, T, Hq, Hkv, D, base, window, 0, nthreads);
}

static int bwd_impl(const double* q, const double* k, const double* v, const double* dO,
                    const double* o_given, double* dq, double* dk, double* dv, int B, int T,
                    int Hq, int Hkv, int D, double base, int window, int half, int nthreads) {
    if (check_shape(B, T, Hq, Hkv, D, base)) return 1;
    set_threads(nthreads);
    const int G = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)D);
    double* qr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* kr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* orow = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* delta = (double*)malloc(sizeof(double) * (size_t)T);
    double* lse_row = (double*)malloc(sizeof(double) * (size_t)T);
    double* P = (double*)malloc(sizeof(double) * (size_t)T * T);
    double* dS = (double*)malloc(sizeof(double) * (size_t)T * T);
    double* dqr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* dkr = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* dvg = (double*)malloc(sizeof(double) * (size_t)T * D);
    if (!qr || !kr || !orow || !delta || !lse_row || !P || !dS || !dqr || !dkr || !dvg) {
        free(qr); free(kr); free(orow); free(delta); free(lse_row); free(P); free(dS);
        free(dqr); free(dkr); free(dvg);
        return 2;
    }
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            rope_rows(k + IDX4(b, 0, g, 0, T, Hkv, D), (size_t)Hkv * D, kr, (size_t)D, T, D, base, 1, half);
            memset(dkr, 0, sizeof(double) * (size_t)T * D);
            memset(dvg, 0, sizeof(double) * (size_t)T * D);
            for (int h = g * G; h < (g + 1) * G; ++h) {
                rope_rows(q + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, qr, (size_t)D, T, D, base, 1, half);
                softmax_probs(qr, kr, P, lse_row, T, D, window);
#pragma omp parallel for schedule(dynamic, 8)
                for (int i = 0; i < T; ++i) {
                    /* o_i, Delta_i and the row of dS */
                    const int lo = first_key(i, window);
                    double* oi = orow + (size_t)i * D;
                    const double* dOi = dO + IDX4(b, i, h, 0, T, Hq, D);
                    for (int d = 0; d < D; ++d) oi[d] = 0.0;
                    for (int j = lo; j <= i; ++j) {
                        const double p = P[(size_t)i * T + j];
                        const double* vj = v + IDX4(b, j, g, 0, T, Hkv, D);
                        for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
                    }
                    const double* od = o_given ? o_given + IDX4(b, i, h, 0, T, Hq, D) : oi;
                    double di = 0.0;
                    for (int d = 0; d < D; ++d) di += dOi[d] * od[d];
                    delta[i] = di;
                    for (int j = 0; j < lo; ++j) dS[(size_t)i * T + j] = 0.0;
                    for (int j = lo; j <= i; ++j) {
                        const double* vj = v + IDX4(b, j, g, 0, T, Hkv, D);
                        double dp = 0.0;
                        for (int d = 0; d < D; ++d) dp += dOi[d] * vj[d];
                        dS[(size_t)i * T + j] = P[(size_t)i * T + j] * (dp - di);
                    }
                    for (int j = i + 1; j < T; ++j) dS[(size_t)i * T + j] = 0.0;
                    /* dq'_i */
                    double* dqi = dqr + (size_t)i * D;
                    for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                    for (int j = lo; j <= i; ++j) {
                        const double s = dS[(size_t)i * T + j];
                        for (int d = 0; d < D; ++d) dqi[d] += s * kr[(size_t)j * D + d];
                    }
                    for (int d = 0; d < D; ++d) dqi[d] *= scale;
                }
                /* dq = R^T dq' for this head */
                rope_rows(dqr, (size_t)D, dq + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, T, D, base, -1, half);
                /* column sums over the query rows that see key j, one thread per key row j */
#pragma omp parallel for schedule(dynamic, 8)
                for (int j = 0; j < T; ++j) {
                    double* dkj = dkr + (size_t)j * D;
                    double* dvj = dvg + (size_t)j * D;
                    const int hi = last_row(j, T, window);
                    for (int i = j; i <= hi; ++i) {
                        const double s = dS[(size_t)i * T + j] * scale;
                        const double p = P[(size_t)i * T + j];
                        const double* qi = qr + (size_t)i * D;
                        const double* dOi = dO + IDX4(b, i, h, 0, T, Hq, D);
                        for (int d = 0; d < D; ++d) {
                            dkj[d] += s * qi[d];
                            dvj[d] += p * dOi[d];
                        }
                    }
                }
            }
            rope_rows(dkr, (size_t)D, dk + IDX4(b, 0, g, 0, T, Hkv, D), (size_t)Hkv * D, T, D, base, -1, half);
            for (int t = 0; t < T; ++t)
                memcpy(dv + IDX4(b, t, g, 0, T, Hkv, D), dvg + (size_t)t * D, sizeof(double) * D);
        }
    }
    free(qr); free(kr); free(orow); free(delta); free(lse_row); free(P); free(dS);
    free(dqr); free(dkr); free(dvg);
    return 0;
}

/* ---- QK norm ------------------------------------------------------------------------------
 * Every (b, t, head) row x of q and of k is replaced, before RoPE, by
 *   x_hat = gain * x / sqrt(mean_d(x_d^2) + eps)
 * (nanochat guide, section 模型架构速览: q and k are normalised and scaled up by 1.2).  Attention
 * then runs on (q_hat, k_hat, v) exactly as above, and the gradients flow back through the
 * normalisation: with rho = 1 / sqrt(mean(x^2) + eps) and dy the gradient with respect to
 * x_hat, dx = gain * rho * (dy - x * rho^2 * (dy . x) / D).  (RoPE preserves the sum of squares
 * of each row, so normalising before or after the rotation gives the same x_hat.) */
static void qk_norm_rows(const double* x, double* y, size_t nrows, int D, double gain, double eps) {
    for (size_t r = 0; r < nrows; ++r) {
        const double* xr = x + r * D;
        double ss = 0.0;
        for (int d = 0; d < D; ++d) ss += xr[d] * xr[d];
        const double rho = 1.0 / sqrt(ss / (double)D + eps);
        for (int d = 0; d < D; ++d) y[r * D + d] = gain * xr[d] * rho;
    }
}

static void qk_norm_rows_bwd(const double* x, double* dxy, size_t nrows, int D, double gain, double eps) {
    /* dxy holds dy on entry and dx on return */
    for (size_t r = 0; r < nrows; ++r) {
        const double* xr = x + r * D;
        double* g = dxy + r * D;
        double ss = 0.0, dot = 0.0;
        for (int d = 0; d < D; ++d) {
            ss += xr[d] * xr[d];
            dot += g[d] * xr[d];
        }
        const double rho = 1.0 / sqrt(ss / (double)D + eps);
        for (int d = 0; d < D; ++d) g[d] = gain * rho * (g[d] - xr[d] * rho * rho * dot / (double)D);
    }
}

static int qk_norm_copies(const double* q, const double* k, double** qh, double** kh, int B, int T,
                          int Hq, int Hkv, int D, double gain, double eps) {
    const size_t nq = (size_t)B * T * Hq, nk = (size_t)B * T * Hkv;
    *qh = (double*)malloc(sizeof(double) * nq * D);
    *kh = (double*)malloc(sizeof(double) * nk * D);
    if (!*qh || !*kh) { free(*qh); free(*kh); return 2; }
    qk_norm_rows(q, *qh, nq, D, gain, eps);
    qk_norm_rows(k, *kh, nk, D, gain, eps);
    return 0;
}

/* Forward with every option: window as in the header, qk_norm != 0 applies the QK norm,
 * half_split != 0 pairs element i with element i + D/2 in the rotation. */
int ne_oracle_fwd_x(const double* q, const double* k, const double* v, double* o, double* lse,
                    int B, int T, int Hq, int Hkv, int D, double base, int window, int qk_norm,
                    double gain, double eps, int half_split, int nthreads) {
    if (check_shape(B, T, Hq, Hkv, D, base) || (qk_norm && !(eps >= 0.0))) return 1;
    if (!qk_norm) return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, D, base, window, half_split, nthreads);
    double *qh, *kh;
    if (qk_norm_copies(q, k, &qh, &kh, B, T, Hq, Hkv, D, gain, eps)) return 2;
    const int rc = fwd_impl(qh, kh, v, o, lse, B, T, Hq, Hkv, D, base, window, half_split, nthreads);
    free(qh); free(kh);
    return rc;
}

/* Backward with every option; o may be NULL (exact Delta) or the o to take Delta from;
 * half_split as in ne_oracle_fwd_x. */
int ne_oracle_bwd_x(const double* q, const double* k, const double* v, const double* o,
                    const double* dO, double* dq, double* dk, double* dv, int B, int T, int Hq,
                    int Hkv, int D, double base, int window, int qk_norm, double gain, double eps,
                    int half_split, int nthreads) {
    if (check_shape(B, T, Hq, Hkv, D, base) || (qk_norm && !(eps >= 0.0))) return 1;
    if (!qk_norm)
        return bwd_impl(q, k, v, dO, o, dq, dk, dv, B, T, Hq, Hkv, D, base, window, half_split, nthreads);
    double *qh, *kh;
    if (qk_norm_copies(q, k, &qh, &kh, B, T, Hq, Hkv, D, gain, eps)) return 2;
    const int rc = bwd_impl(qh, kh, v, dO, o, dq, dk, dv, B, T, Hq, Hkv, D, base, window, half_split, nthreads);
    free(qh); free(kh);
    if (rc) return rc;
    qk_norm_rows_bwd(q, dq, (size_t)B * T * Hq, D, gain, eps);
    qk_norm_rows_bwd(k, dk, (size_t)B * T * Hkv, D, gain, eps);
    return 0;
}

/* Threads the oracle will use (for the benchmark's report). */
int ne_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
