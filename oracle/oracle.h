/*
 * oracle.h -- plain, slow CPU reference for one flow-matching action-expert
 * decision, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library; the two agree only on the documented input formats.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [PhyAI]   "PhyAI" paper, section 4.2 (Kernel fusion; Graph replay;
 *             Profiled operator selection).
 *   [Blog]    "Introducing PhyAI: Real-Time Physical AI at the Edge, Scalable
 *             Rollouts in the Cloud", section "How we optimize PI0.5 and GR00T".
 *   [FlashRT] "FlashRT-PAI: Fast Kernels Are Not Fast Pipelines for Physical
 *             AI Inference", section 2.1 (Figure 1a), section 3.2 (fusion),
 *             Figure 3 caption (37 modulation projections), Appendix A.1.
 *
 * Weight blob (all float32, values as the caller stored them; every matrix is
 * [in][out] row-major, so a projection is y = x . W):
 *   W_in   [A][D]
 *   per layer l = 0..NL-1:
 *     W_qkv  [D][(H + 2*KVH)*Dh]   output columns: q heads, then k heads, then v heads
 *     W_o    [H*Dh][D]
 *     W_gu   [D][2F]               first F columns are the gate g, last F the up u
 *     W_down [F][D]
 *   W_out  [D][A]
 *   W_mod  [2*NL+1][E][2D]         norm n: first D outputs scale, last D shift;
 *                                  norm 2l before attention, 2l+1 before the MLP,
 *                                  2*NL the final norm.
 * Prefix K/V (float32): [B][NL][C][KVH*Dh]; request b uses rows t < len[b].
 * Noise / actions: [B][M][A].
 */
#ifndef PHX_ORACLE_H
#define PHX_ORACLE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct orc_config {
  int layers;       /* NL */
  int width;        /* D  */
  int n_heads;      /* H  */
  int head_dim;     /* Dh (even) */
  int n_kv_heads;   /* KVH, divides H */
  int mlp_hidden;   /* F  */
  int state_dim;    /* A  */
  int rows;         /* M: action rows per request */
  int batch;        /* B  */
  int capacity;     /* C: prefix rows stored per request and layer */
  int steps;        /* S  */
  int time_emb_dim; /* E (even) */
  double tau0;      /* flow time of the first step */
  double dt;        /* Euler step (negative: tau runs from 1 towards 0) */
  double rms_eps;
  double rope_base;
} orc_config;

/* Number of float32 values in the weight blob for cfg. */
size_t orc_weight_count(const orc_config* cfg);

/* e[j] = sin(tau*w_j), e[E/2+j] = cos(tau*w_j), w_j = 10000^(-j/(E/2)). */
void orc_time_embedding(int E, double tau, double* e);

/* mod[c] = sum_j e[j] * Wmod_n[j][c] for c < 2D (scale | shift). */
void orc_modulation(int E, int D, const float* Wmod_n, const double* e, double* mod);

/* out[m][d] = h[m][d] / sqrt(mean_d h[m][.]^2 + eps) * (1 + scale[d]) + shift[d]. */
void orc_ada_rmsnorm(int M, int D, const double* h, const double* mod, double eps, double* out);

/* y[m][n] = sum_k x[m][k] * W[k][n], k summed in increasing order. */
void orc_matmul(int M, int K, int N, const double* x, const float* W, double* y);

/* Rotate-half RoPE in place on x[M][nh*Dh]; row m sits at position pos[m]. */
void orc_rope(int M, int nh, int Dh, const int* pos, double base, double* x);

/* tanh-form GELU. */
double orc_gelu_tanh(double z);

/*
 * Attention of one request: M query rows, H query heads sharing KVH key/value
 * heads.  Keys are the L prefix rows (Kp/Vp [L][KVH*Dh], stride kv_stride
 * floats between rows) followed by the M action rows ka/va [M][KVH*Dh]; every
 * query row sees all L+M keys.  o [M][H*Dh].  Returns the largest
 * |sum(p) - 1| over all softmax rows.
 */
double orc_attention(int M, int H, int KVH, int Dh, int L, const double* q, const double* ka, const double* va,
                     const float* Kp, const float* Vp, size_t kv_stride, double* o);

/*
 * One decision.  actions [B][M][A] receives the integrated state.  If
 * trace is non-NULL it receives the residual stream h after the input
 * projection and after every layer of every step:
 * [S][NL+1][B*M][D] doubles.  If velocity is non-NULL it receives v of every
 * step: [S][B*M][A].  Returns 0, or -1 on a bad argument.
 */
int orc_decide(const orc_config* cfg, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
               const float* noise, double* actions, double* trace, double* velocity);

/* orc_decide with the rows of request b at positions pos0[b] + lens[b] + i
   (the window of a history cache that has dropped its oldest rows keeps
   absolute positions); pos0 NULL is orc_decide. */
int orc_decide_at(const orc_config* cfg, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
                  const int* pos0, const float* noise, double* actions, double* trace, double* velocity);

/*
 * Commit of a decided chunk into a history cache: one pass of the layer
 * stack over x [B][M][A] at flow time tau, the rows at positions pos0[b] +
 * lens[b] + i, attending to the lens[b] cached rows and the chunk.  kout and
 * vout receive every layer's keys (after RoPE) and values of the chunk rows,
 * [B][NL][M][KVH*Dh]; trace (optional) the residual stream as for
 * orc_decide with one step.  Returns 0, or -1 on a bad argument.
 */
int orc_commit(const orc_config* cfg, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
               const int* pos0, const float* x, double tau, double* kout, double* vout, double* trace);

/* Largest |sum(p) - 1| seen by any softmax row of the last orc_decide or
   orc_dit call. */
double orc_last_softmax_dev(void);

/*
 * Adaptive LayerNorm without a learned affine (the DiT-style block):
 * out[m][d] = (h[m][d] - mean) / sqrt(var + eps) * (1 + scale[d]) + shift[d],
 * mean and (biased) variance over the row's D entries.
 */
void orc_ada_layernorm(int M, int D, const double* h, const double* scale, const double* shift, double eps,
                       double* out);

/*
 * One DiT-style denoise step over T = cfg->rows tokens (the large-token
 * workload; cfg->n_kv_heads must equal cfg->n_heads).  Weight blob (float32):
 *   for each block b < NL: W_qkv [D][3*H*Dh] (q heads, k heads, v heads),
 *                          W_o [H*Dh][D], W_up [D][F], W_down [F][D];
 *   W_mod [NL][E][6D]: block b's modulation, in the order shift, scale, gate
 *                      of the attention branch, then shift, scale, gate of
 *                      the MLP branch (D outputs each).
 * Per block, with e the sinusoid of tau0 and m_b = e . W_mod[b]:
 *   n = AdaLN(x; scale_a, shift_a);  o = Attention(n W_qkv) over all T tokens
 *   (no mask, no rotary positions);  x += gate_a * (o W_o)
 *   n = AdaLN(x; scale_m, shift_m);  x += gate_m * (GELU_tanh(n W_up) W_down)
 * x_in [T][D] float; out [T][D] receives x after the last block.  If trace is
 * non-NULL it receives x after every block: [NL][T][D].  Returns 0, or -1 on
 * a bad argument.
 */
int orc_dit(const orc_config* cfg, const float* weights, const float* x_in, double* out, double* trace);

/* Number of float32 values in the DiT-style weight blob for cfg. */
size_t orc_dit_weight_count(const orc_config* cfg);

/*
 * Prefix prefill over the first T tokens of x_in [T][D] (float32): the
 * decoder stack that writes the key/value cache the expert reads.  Weight
 * blob (float32):
 *   for each layer l < NL: W_qkv [D][(H+2*KVH)*Dh] (q, k, v heads), W_o
 *                          [H*Dh][D], W_gu [D][2F] (gate, then up), W_down
 *                          [F][D];
 *   G [2*NL][D]: RMSNorm gains, row 2l before attention, 2l+1 before the MLP.
 * Per layer: n = RMSNorm(x) * (1 + g); q, k, v = n W_qkv with RoPE on q and
 * k at positions 0..T-1; kout[l] = k, vout[l] = v; o = causal attention
 * (token i sees 0..i, scale 1/sqrt(Dh)); x += o W_o; n = RMSNorm(x) * (1 + g');
 * x += (GELU_tanh(n W_g) * (n W_u)) W_down.  The last layer stops after its
 * cache.  kout and vout: [NL][T][KVH*Dh]; trace (optional): x after every
 * layer but the last, [NL-1][T][D].  Returns 0, or -1 on a bad argument.
 */
int orc_prefill(const orc_config* cfg, const float* weights, const float* x_in, int T, double* kout, double* vout,
                double* trace);

/* Number of float32 values in the prefill weight blob for cfg. */
size_t orc_prefill_weight_count(const orc_config* cfg);

/*
 * 8-bit weight tier (round-to-nearest, weight-only): per output channel n of
 * W [K][N] (float32), s[n] = max_k |W[k][n]| / 127 and q[k][n] =
 * clamp(rint(W[k][n] / s[n]), -127, 127), both divisions in float32, ties to
 * even; a zero column gives s = 0 and q = 0.  q [K][N], s [N].
 */
void orc_quantize_i8(int K, int N, const float* W, signed char* q, float* s);

#ifdef __cplusplus
}
#endif
#endif
