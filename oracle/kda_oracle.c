/*
 * CPU oracle for the fused causal-conv1d + Kimi-Delta-Attention (KDA) multi-token
 * verify-decode step.
 *
 * TEST INFRASTRUCTURE ONLY. This file is a plain, slow, sequential float64
 * statement of what the step computes. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it. The GPU library never links, calls or
 * includes it, and it shares no code with the GPU library.
 *
 * Source page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull
 * request), cited below as PR#107 with the part of the page:
 *   - "description": the PR description (what the fused op computes, verify
 *     semantics, the rolled conv_state, GVA, gate forms);
 *   - "commit 1": the first commit message (width-4 conv with SiLU, any T >= 1,
 *     HV >= H);
 *   - "review": the bot code review (the softplus threshold must be a real branch).
 * Where the page leaves a formula open, the reading taken is named at the function.
 *
 * All arithmetic is float64 on inputs that were exactly upcast from their stored
 * dtype (bf16 or fp32). Layouts are dense row-major:
 *   mixed_qkv [N,T,C], C = 2*H*K + HV*V, channels q | k | v, head-major
 *   conv_weight [C,4], conv_state [N,C,3], gate [N,T,HV,K], A_log [HV],
 *   dt_bias [HV*K], beta [N,T,HV], state [N,HV,K,V],
 *   o [N,T,HV,V], inter_ssm [N,T,HV,K,V], conv_window [N,T,C,3].
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_W 4 /* conv width; the cache holds W-1 = 3 raw tokens */

/* Extended raw sequence of one channel (PR#107 description: conv_state holds the
 * three most recent raw inputs, then the T new tokens):
 *   e[tau] = conv_state[n,c,tau] for tau < 3, mixed_qkv[n,tau-3,c] otherwise. */
static double ext_raw(const double* mixed_qkv, const double* conv_state, int T, int C,
                      int n, int c, int tau) {
  if (tau < ORACLE_W - 1) return conv_state[((size_t)n * C + c) * (ORACLE_W - 1) + tau];
  return mixed_qkv[((size_t)n * T + (tau - (ORACLE_W - 1))) * C + c];
}

/* SiLU(y) = y * sigmoid(y). */
double oracle_silu(double y) { return y / (1.0 + exp(-y)); }

/* sigmoid(x) = 1 / (1 + e^-x); used for beta (PR#107 description: gate/beta). */
double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Width-4 depthwise causal conv1d followed by SiLU, every channel and token
 * (PR#107 commit 1 and description). Tap j = 3 multiplies the current token,
 * taps 0..2 the three before it; there is no bias.
 *   act[n,t,c] = SiLU( sum_j w[c,j] * e[t+j] ). */
void oracle_conv_silu(int N, int T, int C, const double* mixed_qkv, const double* conv_weight,
                      const double* conv_state, double* act) {
  for (int n = 0; n < N; ++n)
    for (int t = 0; t < T; ++t)
      for (int c = 0; c < C; ++c) {
        double y = 0.0;
        for (int j = 0; j < ORACLE_W; ++j)
          y += conv_weight[(size_t)c * ORACLE_W + j] *
               ext_raw(mixed_qkv, conv_state, T, C, n, c, t + j);
        act[((size_t)n * T + t) * C + c] = oracle_silu(y);
      }
}

/* Rollback snapshots of the raw conv window and the rolled conv cache (PR#107
 * description: per-token convolution-window snapshots; conv_state rolled to the
 * three most recent raw tokens). These are copies of raw inputs, no arithmetic:
 *   conv_window[n,t,c,j] = e[t+1+j]   (the cache to restore if tokens 0..t are kept)
 *   conv_state_out[n,c,j] = e[T+j]. */
void oracle_conv_roll(int N, int T, int C, const double* mixed_qkv, const double* conv_state,
                      double* conv_window, double* conv_state_out) {
  for (int n = 0; n < N; ++n)
    for (int c = 0; c < C; ++c) {
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < ORACLE_W - 1; ++j)
          conv_window[(((size_t)n * T + t) * C + c) * (ORACLE_W - 1) + j] =
              ext_raw(mixed_qkv, conv_state, T, C, n, c, t + 1 + j);
      for (int j = 0; j < ORACLE_W - 1; ++j)
        conv_state_out[((size_t)n * C + c) * (ORACLE_W - 1) + j] =
            ext_raw(mixed_qkv, conv_state, T, C, n, c, T + j);
    }
}

/* q/k L2 normalisation (PR#107 description). Reading: out = scale * x / sqrt(sum x^2 + eps). */
void oracle_l2norm(int K, const double* x, double eps, double scale, double* out) {
  double s = 0.0;
  for (int i = 0; i < K; ++i) s += x[i] * x[i];
  double r = 1.0 / sqrt(s + eps);
  for (int i = 0; i < K; ++i) out[i] = scale * x[i] * r;
}

/* softplus with a linear tail: (1/b) log(1 + e^{b x}) when b*x <= threshold, x above
 * it. A real branch, so the exponential is never formed on the linear side (PR#107
 * review: evaluating it there overflows and 0*inf gives NaN). */
double oracle_softplus(double x, double b, double threshold) {
  if (b * x <= threshold) return log1p(exp(b * x)) / b;
  return x;
}

/* Per-channel log-decay (PR#107 description: softplus gate and safe gate with a
 * lower bound). The page names the two forms but prints neither formula; the
 * reading taken (the public KDA gate) is, with gamma = g + dt_bias:
 *   mode 0 (softplus): -exp(A_log) * softplus(gamma)
 *   mode 1 (safe):     lower_bound * sigmoid(exp(A_log) * gamma)
 * The decay itself is alpha = exp(log-decay). */
double oracle_log_decay(int mode, double g, double dt_bias, double A_log, double lower_bound,
                        double softplus_beta, double softplus_threshold) {
  double gamma = g + dt_bias;
  if (mode == 0) return -exp(A_log) * oracle_softplus(gamma, softplus_beta, softplus_threshold);
  return lower_bound * oracle_sigmoid(exp(A_log) * gamma);
}

/* One token of the gated delta rule on a K x V state, in the order the rule states
 * (PR#107 description: the gated delta-rule recurrence):
 *   S <- Diag(alpha) S
 *   u_j = sum_i k_i S_ij                      (what the state predicts for key k)
 *   S_ij <- S_ij + k_i * beta * (v_j - u_j)   (write beta-weighted correction)
 *   o_j = sum_i q_i S_ij                      (read with the query after the write)
 * which is S' = (I - beta k k^T) Diag(alpha) S + beta k v^T, o = S'^T q. */
void oracle_delta_step(int K, int V, double* S, const double* alpha, const double* k,
                       const double* v, double beta, const double* q, double* o) {
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= alpha[i];
  for (int j = 0; j < V; ++j) {
    double u = 0.0;
    for (int i = 0; i < K; ++i) u += k[i] * S[(size_t)i * V + j];
    double d = beta * (v[j] - u);
    for (int i = 0; i < K; ++i) S[(size_t)i * V + j] += k[i] * d;
  }
  for (int j = 0; j < V; ++j) {
    double acc = 0.0;
    for (int i = 0; i < K; ++i) acc += q[i] * S[(size_t)i * V + j];
    o[j] = acc;
  }
}

/* The whole verify step (PR#107 description, verify semantics): the persistent
 * state is only read; every token's state is written to inter_ssm, its output to o;
 * the raw conv window of every token and the rolled conv cache are written.
 * Value head hv reads q/k head h = hv / (HV/H) (HV >= H, PR#107 commit 1).
 * Returns 0, or -1 for an invalid shape. */
int oracle_verify(int N, int T, int H, int HV, int K, int V, int gate_mode, double lower_bound,
                  double softplus_beta, double softplus_threshold, double scale, double eps,
                  const double* mixed_qkv, const double* conv_weight, const double* conv_state,
                  const double* gate, const double* A_log, const double* dt_bias,
                  const double* beta, const double* state, double* o, double* inter_ssm,
                  double* conv_window, double* conv_state_out) {
  if (N < 0 || T < 1 || H < 1 || HV < H || HV % H != 0 || K < 1 || V < 1) return -1;
  if (gate_mode != 0 && gate_mode != 1) return -1;
  const int C = 2 * H * K + HV * V;
  const int g = HV / H;
  const size_t KV = (size_t)K * V;

  double* act = (double*)malloc(sizeof(double) * (size_t)T * C);
  double* S = (double*)malloc(sizeof(double) * KV);
  double* qn = (double*)malloc(sizeof(double) * K);
  double* kn = (double*)malloc(sizeof(double) * K);
  double* alpha = (double*)malloc(sizeof(double) * K);
  if (!act || !S || !qn || !kn || !alpha) {
    free(act); free(S); free(qn); free(kn); free(alpha);
    return -2;
  }

  oracle_conv_roll(N, T, C, mixed_qkv, conv_state, conv_window, conv_state_out);
  for (int n = 0; n < N; ++n) {
    /* conv + SiLU of sequence n, all tokens and channels */
    oracle_conv_silu(1, T, C, mixed_qkv + (size_t)n * T * C, conv_weight,
                     conv_state + (size_t)n * C * (ORACLE_W - 1), act);
    for (int hv = 0; hv < HV; ++hv) {
      const int h = hv / g;
      memcpy(S, state + ((size_t)n * HV + hv) * KV, sizeof(double) * KV);
      for (int t = 0; t < T; ++t) {
        const double* a = act + (size_t)t * C;
        oracle_l2norm(K, a + (size_t)h * K, eps, scale, qn);
        oracle_l2norm(K, a + (size_t)H * K + (size_t)h * K, eps, 1.0, kn);
        const double* vv = a + 2 * (size_t)H * K + (size_t)hv * V;
        const size_t nth = ((size_t)n * T + t) * HV + hv;
        for (int i = 0; i < K; ++i)
          alpha[i] = exp(oracle_log_decay(gate_mode, gate[nth * K + i], dt_bias[(size_t)hv * K + i],
                                          A_log[hv], lower_bound, softplus_beta,
                                          softplus_threshold));
        const double b = oracle_sigmoid(beta[nth]);
        oracle_delta_step(K, V, S, alpha, kn, vv, b, qn, o + nth * V);
        memcpy(inter_ssm + nth * KV, S, sizeof(double) * KV);
      }
    }
  }
  free(act); free(S); free(qn); free(kn); free(alpha);
  return 0;
}
