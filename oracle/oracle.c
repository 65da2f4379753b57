/*
 * oracle.c -- plain double-precision CPU reference for one decision of a
 * pi0.5-style flow-matching action expert.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): the HIP library never links or
 * calls this file, and this file includes nothing from the library.
 *
 * The steps follow the pages in their order:
 *   - a prefix key/value cache written once and read by every denoising step,
 *     an action expert of NL layers over M action rows, integrated over S
 *     flow-matching Euler steps ("FlashRT-PAI", section 2.1, Figure 1a;
 *     "PhyAI", section 4.2 Graph replay);
 *   - the sinusoidal timestep table and each norm's adaptive-RMSNorm
 *     modulation built once per step index, 2*NL+1 projections
 *     ("Introducing PhyAI", How we optimize PI0.5 and GR00T; "FlashRT-PAI",
 *     Figure 3 caption);
 *   - per layer: adaptive RMSNorm, one Q/K/V projection, RoPE on Q and K,
 *     attention of the action rows to the prefix and to themselves
 *     (head_dim 256 in the pages' shape), output projection + residual,
 *     adaptive RMSNorm, merged gate/up projection, GeGLU, down projection +
 *     residual ("PhyAI", section 4.2 Kernel fusion and Profiled operator
 *     selection; "FlashRT-PAI", section 3.2);
 *   - a final adaptive RMSNorm, the velocity projection and x += dt * v.
 *
 * Where the pages are silent the readings are: no biases; modulation gives
 * (scale, shift) with y*(1+scale)+shift; eps inside the square root;
 * rotate-half RoPE pairing j with j+Dh/2, theta_j = base^(-2j/Dh), action row
 * i at position L+i, prefix keys stored already rotated; the softmax scale is
 * 1/sqrt(Dh); GELU in its tanh form; the time embedding is [sin | cos] with
 * frequencies 10000^(-j/(E/2)).
 *
 * Everything is double precision.  Loops run in a fixed order; OpenMP only
 * splits independent outputs, so results do not depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double g_last_softmax_dev = 0.0;

double orc_last_softmax_dev(void) { return g_last_softmax_dev; }

size_t orc_weight_count(const orc_config* c) {
  size_t D = (size_t)c->width, A = (size_t)c->state_dim, F = (size_t)c->mlp_hidden;
  size_t qkv = (size_t)(c->n_heads + 2 * c->n_kv_heads) * (size_t)c->head_dim;
  size_t hd = (size_t)c->n_heads * (size_t)c->head_dim;
  size_t per_layer = D * qkv + hd * D + D * 2 * F + F * D;
  size_t norms = 2 * (size_t)c->layers + 1;
  return A * D + (size_t)c->layers * per_layer + D * A + norms * (size_t)c->time_emb_dim * 2 * D;
}

void orc_time_embedding(int E, double tau, double* e) {
  int half = E / 2;
  for (int j = 0; j < half; ++j) {
    double w = pow(10000.0, -(double)j / (double)half);
    e[j] = sin(tau * w);
    e[half + j] = cos(tau * w);
  }
}

void orc_modulation(int E, int D, const float* Wmod_n, const double* e, double* mod) {
  int n2 = 2 * D;
#pragma omp parallel for schedule(static)
  for (int c = 0; c < n2; ++c) {
    double s = 0.0;
    for (int j = 0; j < E; ++j) s += e[j] * (double)Wmod_n[(size_t)j * n2 + c];
    mod[c] = s;
  }
}

void orc_ada_rmsnorm(int M, int D, const double* h, const double* mod, double eps, double* out) {
  const double* scale = mod;
  const double* shift = mod + D;
  for (int m = 0; m < M; ++m) {
    const double* y = h + (size_t)m * D;
    double ss = 0.0;
    for (int d = 0; d < D; ++d) ss += y[d] * y[d];
    double r = 1.0 / sqrt(ss / (double)D + eps);
    for (int d = 0; d < D; ++d) out[(size_t)m * D + d] = y[d] * r * (1.0 + scale[d]) + shift[d];
  }
}

void orc_matmul(int M, int K, int N, const double* x, const float* W, double* y) {
  /* Independent output columns are split into blocks across threads; each
   * output still sums k = 0..K-1 in order. */
  const int blk = 64;
  int nblk = (N + blk - 1) / blk;
#pragma omp parallel for schedule(static)
  for (int b = 0; b < nblk; ++b) {
    int n0 = b * blk, n1 = n0 + blk < N ? n0 + blk : N;
    for (int m = 0; m < M; ++m) {
      double* yr = y + (size_t)m * N;
      for (int n = n0; n < n1; ++n) yr[n] = 0.0;
      for (int k = 0; k < K; ++k) {
        double xv = x[(size_t)m * K + k];
        const float* wr = W + (size_t)k * N;
        for (int n = n0; n < n1; ++n) yr[n] += xv * (double)wr[n];
      }
    }
  }
}

void orc_rope(int M, int nh, int Dh, const int* pos, double base, double* x) {
  int half = Dh / 2;
  for (int m = 0; m < M; ++m) {
    for (int j = 0; j < half; ++j) {
      double theta = pow(base, -2.0 * (double)j / (double)Dh);
      double ang = (double)pos[m] * theta;
      double c = cos(ang), s = sin(ang);
      for (int hh = 0; hh < nh; ++hh) {
        double* v = x + (size_t)m * nh * Dh + (size_t)hh * Dh;
        double a = v[j], b = v[j + half];
        v[j] = a * c - b * s;
        v[j + half] = b * c + a * s;
      }
    }
  }
}

double orc_gelu_tanh(double z) {
  const double k = sqrt(2.0 / M_PI);
  return 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z)));
}

double orc_attention(int M, int H, int KVH, int Dh, int L, const double* q, const double* ka, const double* va,
                     const float* Kp, const float* Vp, size_t kv_stride, double* o) {
  int T = L + M;
  int group = H / KVH;
  int kvd = KVH * Dh;
  double scale = 1.0 / sqrt((double)Dh);
  double worst = 0.0;
#pragma omp parallel for schedule(static) reduction(max : worst)
  for (int mh = 0; mh < M * H; ++mh) {
    int m = mh / H, hh = mh % H, g = hh / group;
    const double* qv = q + (size_t)m * H * Dh + (size_t)hh * Dh;
    double* logit = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    /* logits q.k / sqrt(Dh) over prefix keys then action keys */
    for (int t = 0; t < T; ++t) {
      double s = 0.0;
      if (t < L) {
        const float* kr = Kp + (size_t)t * kv_stride + (size_t)g * Dh;
        for (int d = 0; d < Dh; ++d) s += qv[d] * (double)kr[d];
      } else {
        const double* kr = ka + (size_t)(t - L) * kvd + (size_t)g * Dh;
        for (int d = 0; d < Dh; ++d) s += qv[d] * kr[d];
      }
      logit[t] = s * scale;
    }
    /* softmax (max subtracted) */
    double mx = -INFINITY;
    for (int t = 0; t < T; ++t) if (logit[t] > mx) mx = logit[t];
    double den = 0.0;
    for (int t = 0; t < T; ++t) { logit[t] = exp(logit[t] - mx); den += logit[t]; }
    double psum = 0.0;
    for (int t = 0; t < T; ++t) { logit[t] /= den; psum += logit[t]; }
    double dev = fabs(psum - 1.0);
    if (dev > worst) worst = dev;
    /* o = sum_t p_t v_t */
    double* ov = o + (size_t)m * H * Dh + (size_t)hh * Dh;
    for (int d = 0; d < Dh; ++d) ov[d] = 0.0;
    for (int t = 0; t < T; ++t) {
      double p = logit[t];
      if (t < L) {
        const float* vr = Vp + (size_t)t * kv_stride + (size_t)g * Dh;
        for (int d = 0; d < Dh; ++d) ov[d] += p * (double)vr[d];
      } else {
        const double* vr = va + (size_t)(t - L) * kvd + (size_t)g * Dh;
        for (int d = 0; d < Dh; ++d) ov[d] += p * vr[d];
      }
    }
    free(logit);
  }
  return worst;
}

static int check_cfg(const orc_config* c) {
  if (!c) return -1;
  if (c->layers < 0 || c->width <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || (c->head_dim & 1)) return -1;
  if (c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads) return -1;
  if (c->mlp_hidden <= 0 || c->state_dim <= 0 || c->rows <= 0 || c->batch <= 0 || c->capacity < 0) return -1;
  if (c->steps < 0 || c->time_emb_dim <= 0 || (c->time_emb_dim & 1)) return -1;
  return 0;
}

/* The decision, with the row positions of request b starting at pos0[b] + lens[b]
   (pos0 NULL: at lens[b]) and, when kout/vout are given, every layer's keys
   (after RoPE) and values of the rows captured as [B][NL][M][KVH*Dh]. */
static int decide_impl(const orc_config* c, const float* weights, const float* kv_k, const float* kv_v,
                       const int* lens, const int* pos0, const float* noise, double* actions, double* trace,
                       double* velocity, double* kout, double* vout) {
  if (check_cfg(c) || !weights || !noise || !actions || !lens) return -1;
  const int NL = c->layers, D = c->width, H = c->n_heads, Dh = c->head_dim, KVH = c->n_kv_heads;
  const int F = c->mlp_hidden, A = c->state_dim, M = c->rows, B = c->batch, C = c->capacity, S = c->steps;
  const int E = c->time_emb_dim;
  const int BM = B * M;
  const int hd = H * Dh, kvd = KVH * Dh, nqkv = hd + 2 * kvd;
  for (int b = 0; b < B; ++b)
    if (lens[b] < 0 || lens[b] > C) return -1;
  if (C > 0 && (!kv_k || !kv_v)) return -1;

  /* weight offsets, in the documented blob order */
  const float* W_in = weights;
  size_t off = (size_t)A * D;
  size_t per_layer = (size_t)D * nqkv + (size_t)hd * D + (size_t)D * 2 * F + (size_t)F * D;
  const float* layer0 = weights + off;
  off += (size_t)NL * per_layer;
  const float* W_out = weights + off;
  off += (size_t)D * A;
  const float* W_mod = weights + off;
  const int n_norm = 2 * NL + 1;

  double* x = (double*)malloc(sizeof(double) * (size_t)BM * A);
  double* h = (double*)malloc(sizeof(double) * (size_t)BM * D);
  double* n = (double*)malloc(sizeof(double) * (size_t)BM * D);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)BM * nqkv);
  double* q = (double*)malloc(sizeof(double) * (size_t)M * hd);
  double* ka = (double*)malloc(sizeof(double) * (size_t)M * kvd);
  double* va = (double*)malloc(sizeof(double) * (size_t)M * kvd);
  double* o = (double*)malloc(sizeof(double) * (size_t)BM * hd);
  double* proj = (double*)malloc(sizeof(double) * (size_t)BM * (D > A ? D : A));
  double* gu = (double*)malloc(sizeof(double) * (size_t)BM * 2 * F);
  double* act = (double*)malloc(sizeof(double) * (size_t)BM * F);
  double* e = (double*)malloc(sizeof(double) * (size_t)E);
  double* mod = (double*)malloc(sizeof(double) * (size_t)n_norm * 2 * D);
  int* pos = (int*)malloc(sizeof(int) * (size_t)M);
  double worst = 0.0;

  for (int i = 0; i < BM * A; ++i) x[i] = (double)noise[i];

  for (int k = 0; k < S; ++k) {
    /* step conditioning: depends only on the step index */
    double tau = c->tau0 + (double)k * c->dt;
    orc_time_embedding(E, tau, e);
    for (int nn = 0; nn < n_norm; ++nn)
      orc_modulation(E, D, W_mod + (size_t)nn * E * 2 * D, e, mod + (size_t)nn * 2 * D);

    /* input projection */
    orc_matmul(BM, A, D, x, W_in, h);
    if (trace) memcpy(trace + ((size_t)k * (NL + 1)) * BM * D, h, sizeof(double) * (size_t)BM * D);

    for (int l = 0; l < NL; ++l) {
      const float* W_qkv = layer0 + (size_t)l * per_layer;
      const float* W_o = W_qkv + (size_t)D * nqkv;
      const float* W_gu = W_o + (size_t)hd * D;
      const float* W_down = W_gu + (size_t)D * 2 * F;

      /* attention block */
      orc_ada_rmsnorm(BM, D, h, mod + (size_t)(2 * l) * 2 * D, c->rms_eps, n);
      orc_matmul(BM, D, nqkv, n, W_qkv, qkv);
      for (int b = 0; b < B; ++b) {
        int L = lens[b];
        const int base = pos0 ? pos0[b] : 0;
        for (int m = 0; m < M; ++m) {
          const double* src = qkv + (size_t)(b * M + m) * nqkv;
          memcpy(q + (size_t)m * hd, src, sizeof(double) * hd);
          memcpy(ka + (size_t)m * kvd, src + hd, sizeof(double) * kvd);
          memcpy(va + (size_t)m * kvd, src + hd + kvd, sizeof(double) * kvd);
          pos[m] = base + L + m;
        }
        orc_rope(M, H, Dh, pos, c->rope_base, q);
        orc_rope(M, KVH, Dh, pos, c->rope_base, ka);
        if (kout && vout) {
          memcpy(kout + (((size_t)b * NL + l) * M) * kvd, ka, sizeof(double) * (size_t)M * kvd);
          memcpy(vout + (((size_t)b * NL + l) * M) * kvd, va, sizeof(double) * (size_t)M * kvd);
        }
        const float* Kp = kv_k ? kv_k + ((size_t)b * NL + l) * (size_t)C * kvd : NULL;
        const float* Vp = kv_v ? kv_v + ((size_t)b * NL + l) * (size_t)C * kvd : NULL;
        double dev = orc_attention(M, H, KVH, Dh, L, q, ka, va, Kp, Vp, (size_t)kvd, o + (size_t)b * M * hd);
        if (dev > worst) worst = dev;
      }
      orc_matmul(BM, hd, D, o, W_o, proj);
      for (int i = 0; i < BM * D; ++i) h[i] += proj[i];

      /* MLP block */
      orc_ada_rmsnorm(BM, D, h, mod + (size_t)(2 * l + 1) * 2 * D, c->rms_eps, n);
      orc_matmul(BM, D, 2 * F, n, W_gu, gu);
      for (int r = 0; r < BM; ++r)
        for (int f = 0; f < F; ++f) {
          double g = gu[(size_t)r * 2 * F + f], u = gu[(size_t)r * 2 * F + F + f];
          act[(size_t)r * F + f] = orc_gelu_tanh(g) * u;
        }
      orc_matmul(BM, F, D, act, W_down, proj);
      for (int i = 0; i < BM * D; ++i) h[i] += proj[i];
      if (trace) memcpy(trace + ((size_t)k * (NL + 1) + l + 1) * BM * D, h, sizeof(double) * (size_t)BM * D);
    }

    /* velocity head and Euler update */
    orc_ada_rmsnorm(BM, D, h, mod + (size_t)(2 * NL) * 2 * D, c->rms_eps, n);
    orc_matmul(BM, D, A, n, W_out, proj);
    if (velocity) memcpy(velocity + (size_t)k * BM * A, proj, sizeof(double) * (size_t)BM * A);
    for (int i = 0; i < BM * A; ++i) x[i] += c->dt * proj[i];
  }

  for (int i = 0; i < BM * A; ++i) actions[i] = x[i];
  g_last_softmax_dev = worst;
  free(x); free(h); free(n); free(qkv); free(q); free(ka); free(va); free(o); free(proj);
  free(gu); free(act); free(e); free(mod); free(pos);
  return 0;
}

int orc_decide(const orc_config* c, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
               const float* noise, double* actions, double* trace, double* velocity) {
  return decide_impl(c, weights, kv_k, kv_v, lens, NULL, noise, actions, trace, velocity, NULL, NULL);
}

int orc_decide_at(const orc_config* c, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
                  const int* pos0, const float* noise, double* actions, double* trace, double* velocity) {
  return decide_impl(c, weights, kv_k, kv_v, lens, pos0, noise, actions, trace, velocity, NULL, NULL);
}

/* The history update of an autoregressive chunk policy ("FlashRT-PAI" section
 * 2.1, Figure 1b: the cache over earlier chunks persists from one decision to
 * the next): one pass of the layer stack over the decided chunk x at flow
 * time tau -- the same pass a decision step makes, attending to the L cached
 * rows and the chunk itself -- whose per-layer keys and values of the chunk
 * rows are what the cache gains. */
int orc_commit(const orc_config* c, const float* weights, const float* kv_k, const float* kv_v, const int* lens,
               const int* pos0, const float* x, double tau, double* kout, double* vout, double* trace) {
  if (!c || !x || !kout || !vout) return -1;
  orc_config one = *c;
  one.steps = 1;
  one.tau0 = tau;
  double* scratch = (double*)malloc(sizeof(double) * (size_t)c->batch * c->rows * c->state_dim);
  if (!scratch) return -1;
  int rc = decide_impl(&one, weights, kv_k, kv_v, lens, pos0, x, scratch, trace, NULL, kout, vout);
  free(scratch);
  return rc;
}

/* ------------------------------------------------------------------------
 * DiT-style block (adaLN-Zero): "Scalable Diffusion Models with
 * Transformers" block structure as the large-token step uses it -- a
 * LayerNorm without affine whose output is modulated by (1 + scale) and
 * shift, a residual branch multiplied by a gate, for attention and MLP.
 * ------------------------------------------------------------------------ */

void orc_ada_layernorm(int M, int D, const double* h, const double* scale, const double* shift, double eps,
                       double* out) {
  for (int m = 0; m < M; ++m) {
    const double* r = h + (size_t)m * D;
    double mean = 0.0;
    for (int d = 0; d < D; ++d) mean += r[d];
    mean /= (double)D;
    double var = 0.0;
    for (int d = 0; d < D; ++d) var += (r[d] - mean) * (r[d] - mean);
    var /= (double)D;
    double inv = 1.0 / sqrt(var + eps);
    for (int d = 0; d < D; ++d) out[(size_t)m * D + d] = shift[d] + (1.0 + scale[d]) * ((r[d] - mean) * inv);
  }
}

size_t orc_dit_weight_count(const orc_config* c) {
  size_t D = (size_t)c->width, F = (size_t)c->mlp_hidden, hd = (size_t)c->n_heads * c->head_dim;
  size_t per_block = D * 3 * hd + hd * D + D * F + F * D;
  return (size_t)c->layers * per_block + (size_t)c->layers * (size_t)c->time_emb_dim * 6 * D;
}

int orc_dit(const orc_config* c, const float* weights, const float* x_in, double* out, double* trace) {
  if (check_cfg(c) || !weights || !x_in || !out || c->n_kv_heads != c->n_heads) return -1;
  const int NL = c->layers, D = c->width, H = c->n_heads, Dh = c->head_dim, F = c->mlp_hidden;
  const int T = c->rows, E = c->time_emb_dim;
  const int hd = H * Dh;
  const size_t per_block = (size_t)D * 3 * hd + (size_t)hd * D + (size_t)D * F + (size_t)F * D;
  const float* W_mod = weights + (size_t)NL * per_block;

  double* x = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* n = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)T * 3 * hd);
  double* q = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* k = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* v = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* o = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* proj = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* up = (double*)malloc(sizeof(double) * (size_t)T * F);
  double* e = (double*)malloc(sizeof(double) * (size_t)E);
  double* mod = (double*)malloc(sizeof(double) * (size_t)6 * D);
  double worst = 0.0;

  for (size_t i = 0; i < (size_t)T * D; ++i) x[i] = (double)x_in[i];
  orc_time_embedding(E, c->tau0, e);
  for (int b = 0; b < NL; ++b) {
    const float* W_qkv = weights + (size_t)b * per_block;
    const float* W_o = W_qkv + (size_t)D * 3 * hd;
    const float* W_up = W_o + (size_t)hd * D;
    const float* W_down = W_up + (size_t)D * F;
    /* modulation: m[c] = sum_j e[j] * W_mod[b][j][c], c < 6D */
    const float* Wm = W_mod + (size_t)b * E * 6 * D;
    for (int cc = 0; cc < 6 * D; ++cc) {
      double s = 0.0;
      for (int j = 0; j < E; ++j) s += e[j] * (double)Wm[(size_t)j * 6 * D + cc];
      mod[cc] = s;
    }
    const double *shift_a = mod, *scale_a = mod + D, *gate_a = mod + 2 * D;
    const double *shift_m = mod + 3 * D, *scale_m = mod + 4 * D, *gate_m = mod + 5 * D;

    /* attention branch */
    orc_ada_layernorm(T, D, x, scale_a, shift_a, c->rms_eps, n);
    orc_matmul(T, D, 3 * hd, n, W_qkv, qkv);
    for (int t = 0; t < T; ++t) {
      const double* src = qkv + (size_t)t * 3 * hd;
      memcpy(q + (size_t)t * hd, src, sizeof(double) * hd);
      memcpy(k + (size_t)t * hd, src + hd, sizeof(double) * hd);
      memcpy(v + (size_t)t * hd, src + 2 * hd, sizeof(double) * hd);
    }
    double dev = orc_attention(T, H, H, Dh, 0, q, k, v, NULL, NULL, 0, o);
    if (dev > worst) worst = dev;
    orc_matmul(T, hd, D, o, W_o, proj);
    for (int t = 0; t < T; ++t)
      for (int d = 0; d < D; ++d) x[(size_t)t * D + d] += gate_a[d] * proj[(size_t)t * D + d];

    /* MLP branch */
    orc_ada_layernorm(T, D, x, scale_m, shift_m, c->rms_eps, n);
    orc_matmul(T, D, F, n, W_up, up);
    for (size_t i = 0; i < (size_t)T * F; ++i) up[i] = orc_gelu_tanh(up[i]);
    orc_matmul(T, F, D, up, W_down, proj);
    for (int t = 0; t < T; ++t)
      for (int d = 0; d < D; ++d) x[(size_t)t * D + d] += gate_m[d] * proj[(size_t)t * D + d];
    if (trace) memcpy(trace + (size_t)b * T * D, x, sizeof(double) * (size_t)T * D);
  }
  memcpy(out, x, sizeof(double) * (size_t)T * D);
  g_last_softmax_dev = worst;
  free(x); free(n); free(qkv); free(q); free(k); free(v); free(o); free(proj); free(up); free(e); free(mod);
  return 0;
}

/* ------------------------------------------------------------------------
 * Prefix prefill: the language model that reads the prefix tokens (image and
 * prompt) and writes the key/value cache the action expert attends to
 * ("FlashRT-PAI", section 2.1, Figure 1a: an 18-layer PaliGemma language
 * model over a prefix of about 500 to 800 tokens writes its cache).
 *
 * Readings where the pages are silent: a decoder layer of the same family
 * as the expert's (RMSNorm with a learned per-channel gain, y*(1+g); one QKV
 * projection; rotate-half RoPE on q and k at positions 0..T-1; attention;
 * output projection + residual; RMSNorm; GeGLU MLP + residual), no biases,
 * and a causal mask: token i sees tokens 0..i.  The cache of layer l is its
 * keys after RoPE and its values.
 * ------------------------------------------------------------------------ */

size_t orc_prefill_weight_count(const orc_config* c) {
  size_t D = (size_t)c->width, F = (size_t)c->mlp_hidden;
  size_t hd = (size_t)c->n_heads * c->head_dim, nqkv = (size_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  size_t per_layer = D * nqkv + hd * D + D * 2 * F + F * D;
  return (size_t)c->layers * per_layer + 2 * (size_t)c->layers * D;
}

/* Causal attention of T tokens over their own keys: token i sees t <= i.
   q [T][H*Dh], k and v [T][KVH*Dh], o [T][H*Dh].  Returns the largest
   |sum(p) - 1| of any softmax row. */
static double causal_attention(int T, int H, int KVH, int Dh, const double* q, const double* k, const double* v,
                               double* o) {
  const int group = H / KVH, kvd = KVH * Dh;
  const double scale = 1.0 / sqrt((double)Dh);
  double worst = 0.0;
#pragma omp parallel for schedule(static) reduction(max : worst)
  for (int ih = 0; ih < T * H; ++ih) {
    const int i = ih / H, hh = ih % H, g = hh / group;
    const double* qv = q + (size_t)i * H * Dh + (size_t)hh * Dh;
    double* p = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    double mx = -INFINITY;
    for (int t = 0; t <= i; ++t) {
      const double* kr = k + (size_t)t * kvd + (size_t)g * Dh;
      double s = 0.0;
      for (int d = 0; d < Dh; ++d) s += qv[d] * kr[d];
      p[t] = s * scale;
      if (p[t] > mx) mx = p[t];
    }
    double den = 0.0;
    for (int t = 0; t <= i; ++t) { p[t] = exp(p[t] - mx); den += p[t]; }
    double psum = 0.0;
    for (int t = 0; t <= i; ++t) { p[t] /= den; psum += p[t]; }
    if (fabs(psum - 1.0) > worst) worst = fabs(psum - 1.0);
    double* ov = o + (size_t)i * H * Dh + (size_t)hh * Dh;
    for (int d = 0; d < Dh; ++d) ov[d] = 0.0;
    for (int t = 0; t <= i; ++t) {
      const double* vr = v + (size_t)t * kvd + (size_t)g * Dh;
      for (int d = 0; d < Dh; ++d) ov[d] += p[t] * vr[d];
    }
    free(p);
  }
  return worst;
}

int orc_prefill(const orc_config* c, const float* weights, const float* x_in, int T, double* kout, double* vout,
                double* trace) {
  if (check_cfg(c) || !weights || !x_in || !kout || !vout || T < 1) return -1;
  const int NL = c->layers, D = c->width, H = c->n_heads, Dh = c->head_dim, KVH = c->n_kv_heads;
  const int F = c->mlp_hidden, hd = H * Dh, kvd = KVH * Dh, nqkv = hd + 2 * kvd;
  const size_t per_layer = (size_t)D * nqkv + (size_t)hd * D + (size_t)D * 2 * F + (size_t)F * D;
  const float* G = weights + (size_t)NL * per_layer; /* [2NL][D] norm gains */

  double* x = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* n = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)T * nqkv);
  double* q = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* k = (double*)malloc(sizeof(double) * (size_t)T * kvd);
  double* v = (double*)malloc(sizeof(double) * (size_t)T * kvd);
  double* o = (double*)malloc(sizeof(double) * (size_t)T * hd);
  double* proj = (double*)malloc(sizeof(double) * (size_t)T * D);
  double* gu = (double*)malloc(sizeof(double) * (size_t)T * 2 * F);
  double* a = (double*)malloc(sizeof(double) * (size_t)T * F);
  double* mod = (double*)malloc(sizeof(double) * (size_t)2 * D);
  int* pos = (int*)malloc(sizeof(int) * (size_t)T);
  double worst = 0.0;

  for (size_t i = 0; i < (size_t)T * D; ++i) x[i] = (double)x_in[i];
  for (int i = 0; i < T; ++i) pos[i] = i;
  for (int l = 0; l < NL; ++l) {
    const float* W_qkv = weights + (size_t)l * per_layer;
    const float* W_o = W_qkv + (size_t)D * nqkv;
    const float* W_gu = W_o + (size_t)hd * D;
    const float* W_down = W_gu + (size_t)D * 2 * F;

    /* RMSNorm with gain: the adaptive form with scale = g, shift = 0 */
    for (int d = 0; d < D; ++d) { mod[d] = (double)G[(size_t)(2 * l) * D + d]; mod[D + d] = 0.0; }
    orc_ada_rmsnorm(T, D, x, mod, c->rms_eps, n);
    orc_matmul(T, D, nqkv, n, W_qkv, qkv);
    for (int t = 0; t < T; ++t) {
      const double* src = qkv + (size_t)t * nqkv;
      memcpy(q + (size_t)t * hd, src, sizeof(double) * hd);
      memcpy(k + (size_t)t * kvd, src + hd, sizeof(double) * kvd);
      memcpy(v + (size_t)t * kvd, src + hd + kvd, sizeof(double) * kvd);
    }
    orc_rope(T, H, Dh, pos, c->rope_base, q);
    orc_rope(T, KVH, Dh, pos, c->rope_base, k);
    memcpy(kout + (size_t)l * T * kvd, k, sizeof(double) * (size_t)T * kvd);
    memcpy(vout + (size_t)l * T * kvd, v, sizeof(double) * (size_t)T * kvd);
    /* the rest of the last layer writes no cache */
    if (l + 1 == NL) break;

    double dev = causal_attention(T, H, KVH, Dh, q, k, v, o);
    if (dev > worst) worst = dev;
    orc_matmul(T, hd, D, o, W_o, proj);
    for (size_t i = 0; i < (size_t)T * D; ++i) x[i] += proj[i];

    for (int d = 0; d < D; ++d) mod[d] = (double)G[(size_t)(2 * l + 1) * D + d];
    orc_ada_rmsnorm(T, D, x, mod, c->rms_eps, n);
    orc_matmul(T, D, 2 * F, n, W_gu, gu);
    for (int t = 0; t < T; ++t)
      for (int f = 0; f < F; ++f)
        a[(size_t)t * F + f] = orc_gelu_tanh(gu[(size_t)t * 2 * F + f]) * gu[(size_t)t * 2 * F + F + f];
    orc_matmul(T, F, D, a, W_down, proj);
    for (size_t i = 0; i < (size_t)T * D; ++i) x[i] += proj[i];
    if (trace) memcpy(trace + (size_t)l * T * D, x, sizeof(double) * (size_t)T * D);
  }
  g_last_softmax_dev = worst;
  free(x); free(n); free(qkv); free(q); free(k); free(v); free(o); free(proj); free(gu); free(a); free(mod);
  free(pos);
  return 0;
}

/* ------------------------------------------------------------------------
 * 8-bit weight tier (W8A16): weights quantised offline by round-to-nearest,
 * activations kept in 16 bits ("PhyAI", section 4.2 Quantization; the
 * "FlashRT-PAI" precision tiers, Table 4).  Readings where the pages are
 * silent: symmetric int8 codes per output channel (column n of W [K][N]),
 * s[n] = max_k |W[k][n]| / 127 and q = W / s rounded to the nearest integer,
 * ties to even, clamped to [-127, 127]; both divisions in float32; a zero
 * column has s = 0 and q = 0.  The weight is then s[n] * q[k][n].
 * ------------------------------------------------------------------------ */

void orc_quantize_i8(int K, int N, const float* W, signed char* q, float* s) {
  for (int n = 0; n < N; ++n) {
    float m = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float a = fabsf(W[(size_t)k * N + n]);
      if (a > m) m = a;
    }
    const float sc = m / 127.0f;
    s[n] = sc;
    for (int k = 0; k < K; ++k) {
      float v = sc > 0.0f ? rintf(W[(size_t)k * N + n] / sc) : 0.0f;
      if (v > 127.0f) v = 127.0f;
      if (v < -127.0f) v = -127.0f;
      q[(size_t)k * N + n] = (signed char)v;
    }
  }
}
