/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the fused gated-delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes: FlashInfer, "flashinfer.gdn_fused_decode_step" page -- one
 * decode token per batch entry: the b/a projection GEMV, the causal conv1d
 * update, the q/k/v split and the gated delta-rule decode with qk-L2-norm,
 * over paged conv and ssm pools indexed by state_indices (negative = padding:
 * no pool access, zero output).  The page names the steps and shapes but not
 * their formulas; the readings taken (each listed with its reason in the
 * design notes) are, per batch entry b with pool slot s:
 *   ba      = hidden[b] @ w_ba                      (columns [:HV] -> b, [HV:] -> a)
 *   beta    = sigmoid(b_h),  g_h = -exp(A_log_h) * softplus(a_h + dt_bias_h),
 *   alpha_h = exp(g_h)
 *   window  = [conv_state[s, c, 0 .. W-2], mixed_qkv[b, c]]   (oldest first)
 *   y_c     = silu(sum_j window[j] * conv_weight[c, j] + conv_bias[c])
 *   conv_state[s, c, :] = window[1 ..]               (the last W-1 raw inputs)
 *   q, k    = y channels [0, Hq D), [Hq D, 2 Hq D) as [Hq, D]; v = the rest as [HV, D]
 *   q, k    = x / sqrt(sum x^2 + 1e-6) per head when use_qk_l2norm; q *= scale
 *   value head h reads q/k head h / (HV / Hq)
 *   S       = ssm_state[s, h]  ([V, K], V-major, K-last)
 *   S      *= alpha_h;  S[v][:] += beta_h * (vv[v] - S[v][:] . k) * k
 *   out[b, 0, h, v] = S[v][:] . q
 * All arithmetic in fp64, one element at a time; -ffp-contract=off.
 *
 * Parity pins: tests/test_oracle_gdn_pins.py (closed forms, the delta rule's
 * write-at-key property, conv shift, padding) and brute force against the
 * pure-Python oracle/ref_tiny.py.
 *
 * Parity unpinned as to the page: it prints no formula and no worked value for
 * this step, so the pins above fix the oracle to the readings listed here (the
 * gate parameterisation, the norm eps, the conv tap order, the q/k/v split and
 * the head map), not to anything the page states.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double g_softplus(double v)
{
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

static double g_sigmoid(double v)
{
    return 1.0 / (1.0 + exp(-v));
}

static double g_silu(double v)
{
    return v / (1.0 + exp(-v));
}

/* conv_state strides (elements) select the physical layout: slot, channel, tap. */
void oracle_gdn_decode(int32_t batch, int32_t hidden, int32_t hq, int32_t hv, int32_t dhead,
                       int32_t width, const double *hidden_states, const double *w_ba,
                       const double *mixed_qkv, const double *conv_weight,
                       const double *conv_bias, double *conv_state, int64_t cs_slot,
                       int64_t cs_chan, int64_t cs_tap, const double *A_log,
                       const double *dt_bias, double scale, double *ssm_state,
                       int64_t ssm_row_stride, const int32_t *state_indices,
                       int32_t use_qk_l2norm, double *out)
{
    const int64_t qkv_dim = (int64_t)(2 * hq + hv) * dhead;
    const int64_t tile = (int64_t)dhead * dhead;
    const int per_group = hv / hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int64_t s = state_indices[b];
        if (s < 0) {
            for (int64_t i = 0; i < (int64_t)hv * dhead; ++i)
                out[(int64_t)b * hv * dhead + i] = 0.0;
            continue;
        }
        /* b/a projection */
        double *ba = (double *)malloc(sizeof(double) * 2 * hv);
        for (int j = 0; j < 2 * hv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < hidden; ++i)
                acc += hidden_states[(int64_t)b * hidden + i] * w_ba[(int64_t)i * 2 * hv + j];
            ba[j] = acc;
        }
        /* causal conv1d update over every channel */
        double *y = (double *)malloc(sizeof(double) * qkv_dim);
        double *win = (double *)malloc(sizeof(double) * width);
        for (int64_t c = 0; c < qkv_dim; ++c) {
            double *cs = conv_state + s * cs_slot + c * cs_chan;
            for (int j = 0; j < width - 1; ++j)
                win[j] = cs[j * cs_tap];
            win[width - 1] = mixed_qkv[(int64_t)b * qkv_dim + c];
            double acc = conv_bias[c];
            for (int j = 0; j < width; ++j)
                acc += win[j] * conv_weight[c * width + j];
            y[c] = g_silu(acc);
            for (int j = 0; j < width - 1; ++j)
                cs[j * cs_tap] = win[j + 1];
        }
        /* q, k normalisation per q/k head */
        for (int part = 0; part < 2; ++part) {
            for (int h = 0; h < hq; ++h) {
                double *x = y + (int64_t)part * hq * dhead + (int64_t)h * dhead;
                if (use_qk_l2norm) {
                    double ss = 0.0;
                    for (int d = 0; d < dhead; ++d)
                        ss += x[d] * x[d];
                    const double inv = 1.0 / sqrt(ss + 1e-6);
                    for (int d = 0; d < dhead; ++d)
                        x[d] *= inv;
                }
                if (part == 0)
                    for (int d = 0; d < dhead; ++d)
                        x[d] *= scale;
            }
        }
        /* gated delta rule per value head */
        for (int h = 0; h < hv; ++h) {
            const int qh = h / per_group;
            const double *q = y + (int64_t)qh * dhead;
            const double *k = y + (int64_t)hq * dhead + (int64_t)qh * dhead;
            const double *vv = y + (int64_t)2 * hq * dhead + (int64_t)h * dhead;
            const double beta = g_sigmoid(ba[h]);
            const double g = -exp(A_log[h]) * g_softplus(ba[hv + h] + dt_bias[h]);
            const double alpha = exp(g);
            double *S = ssm_state + s * ssm_row_stride + (int64_t)h * tile;
            for (int v = 0; v < dhead; ++v) {
                double *row = S + (int64_t)v * dhead;
                double pred = 0.0;
                for (int kk = 0; kk < dhead; ++kk) {
                    row[kk] *= alpha;
                    pred += row[kk] * k[kk];
                }
                const double delta = beta * (vv[v] - pred);
                double o = 0.0;
                for (int kk = 0; kk < dhead; ++kk) {
                    row[kk] += delta * k[kk];
                    o += row[kk] * q[kk];
                }
                out[((int64_t)b * hv + h) * dhead + v] = o;
            }
        }
        free(win);
        free(y);
        free(ba);
    }
}
