/*
 * svoracle.c -- plain fp64 CPU oracle for the verify step of MTP speculative
 * decoding (target-model verify attention over a shared KV cache, the LM-head
 * select, and the longest-accepted-prefix rule).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never links,
 * includes or calls anything here, and nothing here is shared with it: this
 * file has its own bf16 rounding, its own RoPE, its own loops.
 *
 * Every function is a direct transcription of a definition into nested loops,
 * evaluated one output row at a time in a fixed loop order that does not
 * depend on how many rows a call processes.  Arithmetic is fp64 throughout.
 * Inputs arrive as fp32 arrays (for bf16 workloads their values are already
 * bf16-exact) or, for the large weight tables, as raw bf16 bit patterns.
 * OpenMP, where present, only splits independent output elements across
 * threads; each element is still computed by one sequential loop, so results
 * are identical for any thread count.
 *
 * Sources (cited by page title and section):
 *  [G4]  "Gemma 4 拆解 | 多模态怎么塞进端侧，MTP drafter 又是怎么自带投机采样的"
 *        (marsggbo.github.io): section 2 (p-RoPE p=0.25 and value reusing key on
 *        global layers), section 4.2 (drafter cross-attends the target's KV cache;
 *        speculative_step: draft, one verify forward, accept longest prefix).
 *  [AG4] "Accelerating Gemma 4: faster inference with multi-token prediction
 *        drafters" (Lighthouse summary): section 3 (the target verifies all
 *        drafts in parallel and emits one extra token of its own).
 *  [FH]  "Gemma 4 发布时未包含 MTP 数据——为什么这很重要" (flowhunt): section
 *        "什么是 Gemma 4？" (alternating local sliding-window and global
 *        attention, p-RoPE, key-equals-value); section "什么是多标记预测？"
 *        (drafts accepted until the first wrong one).
 *  [KC]  "Gemma 4 与 Gemini Nano：端侧智能的架构拆解" (kongchang): section
 *        "草稿模型：共享 KV 缓存带来的加速" (speculative decoding leaves the
 *        output distribution unchanged; the drafter reuses the target's cache).
 *  The rejection-sampling rule the pages only assert (output distribution
 *  unchanged) is the standard one of Leviathan, Kalman & Matias (ICML 2023)
 *  and Chen et al. (2023); sampling uses the Gumbel-max trick.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* threads the parallel loops use from now on (n >= 1); timing only, results do not
 * depend on it */
void svo_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int svo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* bf16 storage rounding: round-to-nearest-even to 8 significant bits.       */
/* ------------------------------------------------------------------------ */

/* Round an fp64 value to the nearest bf16 value (ties to even).  bf16 keeps 8
 * significant bits and the fp32 exponent range (normal minimum 2^-126,
 * subnormal spacing 2^-133, largest finite (2 - 2^-7) * 2^127). */
double svo_bf16_round(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(x, &e);                 /* |x| = m * 2^e, m in [0.5, 1) */
  int shift = e - 8;            /* spacing of 8-significant-bit values near x */
  if (shift < -133) shift = -133;
  double q = ldexp(x, -shift);  /* exact: scaling by a power of two */
  double r = nearbyint(q);      /* default rounding mode: to nearest, ties even */
  double y = ldexp(r, shift);
  const double maxbf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (fabs(y) > maxbf) return x > 0 ? INFINITY : -INFINITY;
  return y;
}

void svo_bf16_round_array(double* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = svo_bf16_round(x[i]);
}

static inline double bf16_bits_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* element i of a weight table stored either as fp32 or as raw bf16 bits */
static inline double load_w(const void* w, int w_bf16, int64_t i) {
  if (w_bf16) return bf16_bits_to_double(((const uint16_t*)w)[i]);
  return (double)((const float*)w)[i];
}

/* ------------------------------------------------------------------------ */
/* RoPE / p-RoPE                                                             */
/* ------------------------------------------------------------------------ */

/* Rotary position embedding on the first `rope_dims` entries of x, rotate-half
 * pairing: entry i is paired with entry i + rope_dims/2 (i < rope_dims/2) and
 * the pair is rotated by the angle pos * base^(-2i/rope_dims).  Entries at or
 * beyond rope_dims are left as they are, which is p-RoPE when rope_dims is a
 * fraction p of the head dimension ([G4] section 2: p = 0.25 on global layers).
 * rope_dims == 0 means no rotation. */
void svo_rope(double* x, int rope_dims, double base, double pos) {
  int half = rope_dims / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)rope_dims);
    double ang = pos * theta;
    double c = cos(ang), s = sin(ang);
    double a = x[i], b = x[i + half];
    x[i] = a * c - b * s;
    x[i + half] = b * c + a * s;
  }
}

/* ------------------------------------------------------------------------ */
/* Verify attention for one sequence and one KV head                         */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t n_q;          /* query rows of this sequence (k+1 in a verify step) */
  int32_t group;        /* query heads sharing this KV head (Hq / Hkv) */
  int32_t head_dim;
  int32_t window;       /* 0: global (causal over all keys); W>0: p-W < t <= p */
  int32_t rope_dims;    /* 0: none; head_dim: full RoPE; < head_dim: p-RoPE */
  int32_t k_is_v;       /* 1: values are the stored (rotated) keys */
  int32_t append;       /* 1: write the n_q new rows at [L, L+n_q) first */
  int32_t q_pos_offset; /* query row j sits at position L + q_pos_offset + j */
  int32_t round_bf16;   /* 1: cache stores are rounded to bf16 */
  int32_t pad_;
  double rope_base;
  double scale;         /* softmax temperature on q.k (1/sqrt(head_dim)) */
  int64_t cap;          /* rows available in the cache arrays */
  int64_t L;            /* committed cache length of this sequence */
  const float* q;       /* [n_q][group][head_dim], pre-RoPE */
  const float* k_new;   /* [n_q][head_dim], pre-RoPE (append only) */
  const float* v_new;   /* [n_q][head_dim] (append and !k_is_v only) */
  float* k_cache;       /* [cap][head_dim], rotated keys */
  float* v_cache;       /* [cap][head_dim] (unused if k_is_v) */
  double* out;          /* [n_q][group][head_dim] */
  const float* k_scale; /* [head_dim] or NULL: appended keys are stored as fp8 E4M3 codes */
  const float* v_scale; /* [head_dim] or NULL: the same for appended values */
} svo_attn_args;

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (the OCP 8-bit float "E4M3FN"): 1 sign bit, 4 exponent bits with */
/* bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9;  */
/* no infinities; S.1111.111 is NaN, so the largest finite value is 448.     */
/* ------------------------------------------------------------------------ */
double svo_e4m3_decode(int code) {
  const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest code to x (ties to the even code), values beyond +-448 saturating to
 * +-448.  Brute force over the 127 finite magnitudes, which are increasing in the
 * code, so an exact tie falls between two neighbours and "even" is the one whose
 * lowest bit is 0. */
int svo_e4m3_encode(float x) {
  if (x != x) return 0x7F;
  const int sign = signbit(x) ? 0x80 : 0;
  const double a = fabs((double)x);
  int best = 0;
  double bd = a;
  for (int c = 1; c <= 0x7E; ++c) {
    const double d = fabs(svo_e4m3_decode(c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
  }
  if (a > 448.0) best = 0x7E;
  return sign | best;
}

/* value stored by a quantized cache: s * decode(encode(x / s)), the quotient an
 * IEEE fp32 division */
static float svo_q8_store(double x, float s) {
  const float q = (float)x / s;
  return (float)((double)s * svo_e4m3_decode(svo_e4m3_encode(q)));
}

/* Multi-query verify attention, [G4] section 4.2 (one target forward scores
 * the k drafts plus the bonus position) and [AG4] section 3.  Steps:
 *  1. append: the new key of row j is rotated at position L+j, stored (bf16
 *     rounded in bf16 mode) in cache row L+j; the new value is stored next to
 *     it unless values are the keys ([G4] section 2; [FH] "什么是 Gemma 4？").
 *  2. each query row j, head h: rotate q at position p = L + q_pos_offset + j,
 *     visible keys t with t <= min(p, last stored row) and, on a sliding
 *     window layer, t > p - window; scores s_t = scale * q.k_t; softmax over
 *     the visible keys; output = sum_t softmax_t * v_t (v_t = k_t when keys
 *     are reused as values).  No visible key gives a zero output row.
 * Returns 0, or -1 if the appended rows do not fit in the cache. */
int svo_attn_group(const svo_attn_args* a) {
  const int D = a->head_dim;
  const int64_t L = a->L;
  const int64_t n_new = a->append ? a->n_q : 0;
  if (L < 0 || L + n_new > a->cap) return -1;
  float* vc = a->k_is_v ? a->k_cache : a->v_cache;

  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  for (int64_t j = 0; j < n_new; ++j) {
    for (int d = 0; d < D; ++d) tmp[d] = (double)a->k_new[j * D + d];
    svo_rope(tmp, a->rope_dims, a->rope_base, (double)(L + j));
    for (int d = 0; d < D; ++d) {
      double kv = a->round_bf16 ? svo_bf16_round(tmp[d]) : tmp[d];
      a->k_cache[(L + j) * D + d] = a->k_scale ? svo_q8_store(kv, a->k_scale[d]) : (float)kv;
    }
    if (!a->k_is_v) {
      for (int d = 0; d < D; ++d) {
        double vv = (double)a->v_new[j * D + d];
        if (a->round_bf16) vv = svo_bf16_round(vv);
        a->v_cache[(L + j) * D + d] = a->v_scale ? svo_q8_store(vv, a->v_scale[d]) : (float)vv;
      }
    }
  }
  free(tmp);

  const int64_t last = L + n_new - 1;  /* last stored key row */
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < (int64_t)a->n_q * a->group; ++row) {
    const int64_t j = row / a->group;
    const int64_t h = row % a->group;
    const int64_t p = L + a->q_pos_offset + j;
    double* qv = (double*)malloc(sizeof(double) * (size_t)D);
    double* ov = a->out + (j * a->group + h) * D;
    for (int d = 0; d < D; ++d) qv[d] = (double)a->q[(j * a->group + h) * D + d];
    svo_rope(qv, a->rope_dims, a->rope_base, (double)p);
    int64_t t_hi = p < last ? p : last;
    int64_t t_lo = 0;
    if (a->window > 0 && p - a->window + 1 > 0) t_lo = p - a->window + 1;
    for (int d = 0; d < D; ++d) ov[d] = 0.0;
    if (t_lo <= t_hi) {
      int64_t n = t_hi - t_lo + 1;
      double* s = (double*)malloc(sizeof(double) * (size_t)n);
      double m = -INFINITY;
      for (int64_t t = t_lo; t <= t_hi; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[d] * (double)a->k_cache[t * D + d];
        s[t - t_lo] = a->scale * dot;
        if (s[t - t_lo] > m) m = s[t - t_lo];
      }
      double z = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        s[i] = exp(s[i] - m);
        z += s[i];
      }
      for (int64_t t = t_lo; t <= t_hi; ++t) {
        double w = s[t - t_lo] / z;
        for (int d = 0; d < D; ++d) ov[d] += w * (double)vc[t * D + d];
      }
      free(s);
    }
    free(qv);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense pieces of a decoder layer (used only by the composed verify step)   */
/* ------------------------------------------------------------------------ */

/* y[r][n] = sum_k x[r][k] * W[n][k]  (W row-major [N][K]) */
void svo_linear(int64_t R, int64_t K, int64_t N, const double* x, const void* W, int w_bf16,
                double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t r = 0; r < R; ++r) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[r * K + k] * load_w(W, w_bf16, n * K + k);
      y[r * N + n] = acc;
    }
  }
}

/* RMSNorm with unit gain: y = x / sqrt(mean(x^2) + eps) */
void svo_rmsnorm(int64_t R, int64_t d, double eps, const double* x, double* y) {
  for (int64_t r = 0; r < R; ++r) {
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) ss += x[r * d + i] * x[r * d + i];
    double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int64_t i = 0; i < d; ++i) y[r * d + i] = x[r * d + i] * inv;
  }
}

/* GELU, tanh form (Hendrycks & Gimpel 2016):
 * 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
double svo_gelu_tanh(double x) {
  const double c = sqrt(2.0 / M_PI);
  return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* GeGLU gating: f = gelu_tanh(g) * u, elementwise */
void svo_geglu(int64_t n, const double* g, const double* u, double* f) {
  for (int64_t i = 0; i < n; ++i) f[i] = svo_gelu_tanh(g[i]) * u[i];
}

/* ------------------------------------------------------------------------ */
/* LM head and per-row statistics                                            */
/* ------------------------------------------------------------------------ */

/* Full logits of R rows: z[r][v] = sum_d h[r][d] * W[v][d]; [G4] section 4.3
 * (the unembed is a d x vocab product; every vocabulary entry is scored). */
void svo_lmhead(int64_t R, int64_t d, int64_t V, const double* h, const void* W, int w_bf16,
                double* z) {
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < V; ++v) {
    for (int64_t r = 0; r < R; ++r) {
      double acc = 0.0;
      for (int64_t i = 0; i < d; ++i) acc += h[r * d + i] * load_w(W, w_bf16, v * d + i);
      z[r * V + v] = acc;
    }
  }
}

typedef struct {
  int32_t top1_id, top2_id;
  double top1, top2;      /* largest and second-largest logit (lowest id wins ties) */
  double lse;             /* log sum_v exp(z_v) */
  double draft_logit;     /* z[draft_id], NaN if draft_id < 0 */
} svo_stats;

/* Greedy statistics of one row of logits: the argmax (ties to the lowest id,
 * the order of the pages' argmax is unspecified), the runner-up (used for the
 * top-2 margin), the log-partition function and the logit of the token that
 * the next draft proposed. */
void svo_row_stats(int64_t V, const double* z, int32_t draft_id, svo_stats* st) {
  int64_t b1 = -1, b2 = -1;
  for (int64_t v = 0; v < V; ++v) {
    if (b1 < 0 || z[v] > z[b1]) { b2 = b1; b1 = v; }
    else if (b2 < 0 || z[v] > z[b2]) { b2 = v; }
  }
  double m = z[b1];
  double acc = 0.0;
  for (int64_t v = 0; v < V; ++v) acc += exp(z[v] - m);
  st->top1_id = (int32_t)b1;
  st->top1 = z[b1];
  st->top2_id = (int32_t)b2;
  st->top2 = b2 >= 0 ? z[b2] : -INFINITY;
  st->lse = m + log(acc);
  st->draft_logit = (draft_id >= 0 && draft_id < V) ? z[draft_id] : NAN;
}

/* ------------------------------------------------------------------------ */
/* Acceptance                                                                */
/* ------------------------------------------------------------------------ */

/* Greedy longest-matching-prefix rule ([G4] section 4.2, accept_longest_prefix;
 * [FH] "什么是多标记预测？"; [AG4] section 3).  Rows 0..k score the positions
 * after [last committed token, d_1..d_k]; draft d_i is checked against the
 * argmax of row i-1.  n = number of leading drafts that match, 0..k; the
 * emitted tokens are d_1..d_n followed by the argmax of row n (the target's own
 * token: a correction when n < k, the bonus token when n == k).
 * tokens_out[0..n] receive them, the rest of tokens_out[0..k] is -1.
 * Returns n. */
int svo_accept_greedy(int k, const int32_t* drafts, const int32_t* top1, int32_t* tokens_out) {
  int n = 0;
  while (n < k && drafts[n] == top1[n]) ++n;
  for (int i = 0; i <= k; ++i) tokens_out[i] = -1;
  for (int i = 0; i < n; ++i) tokens_out[i] = drafts[i];
  tokens_out[n] = top1[n];
  return n;
}

/* Gumbel noise from a uniform in [0,1): G = -log(-log u).  u == 0 gives -inf. */
static inline double gumbel(double u) { return -log(-log(u)); }

/* Speculative rejection-sampling acceptance for one sequence (temperature 1).
 * The pages assert only the outcome (output distribution unchanged: [KC]
 * "草稿模型：共享 KV 缓存带来的加速"; [FH] "MTP 能快多少？"); the rule is the
 * standard one: draft d_i (drawn by the drafter from q_i) is accepted iff
 * u_i * q_i(d_i) < p_{i-1}(d_i), p_{i-1} = softmax of row i-1, i.e. with
 * probability min(1, p/q).  p_{i-1}(d_i) = exp(draft_logit[i-1] - lse[i-1]).
 * margin[i-1] = log p - log(u q) for every tested draft (its sign is the
 * decision).  Returns n = number of accepted drafts (stops at the first
 * rejection). */
int svo_accept_sample(int k, const double* lse, const double* draft_logit, const float* q_at_draft,
                      const float* u_accept, double* margin) {
  int n = 0;
  for (int i = 0; i < k; ++i) {
    double logp = draft_logit[i] - lse[i];
    double p = exp(logp);
    double uq = (double)u_accept[i] * (double)q_at_draft[i];
    margin[i] = logp - log(uq);
    if (uq < p) ++n;
    else break;
  }
  return n;
}

/* Draw from the residual distribution r_v ~ max(p_v - q_v, 0) after a
 * rejection, by Gumbel-max: argmax over {v : r_v > 0} of log r_v + G(u_v).
 * If every r_v is 0 the draw falls back to p itself: argmax z_v + G(u_v).
 * *margin = best score - second best score.  Ties go to the lowest id. */
int svo_sample_residual(int64_t V, const double* z, double lse, const float* q_row, const float* u,
                        double* margin) {
  int64_t b1 = -1, b2 = -1;
  double s1 = -INFINITY, s2 = -INFINITY;
  for (int64_t v = 0; v < V; ++v) {
    double r = exp(z[v] - lse) - (double)q_row[v];
    if (!(r > 0.0)) continue;
    double sc = log(r) + gumbel((double)u[v]);
    if (b1 < 0 || sc > s1) { b2 = b1; s2 = s1; b1 = v; s1 = sc; }
    else if (b2 < 0 || sc > s2) { b2 = v; s2 = sc; }
  }
  if (b1 < 0) {
    for (int64_t v = 0; v < V; ++v) {
      double sc = z[v] + gumbel((double)u[v]);
      if (b1 < 0 || sc > s1) { b2 = b1; s2 = s1; b1 = v; s1 = sc; }
      else if (b2 < 0 || sc > s2) { b2 = v; s2 = sc; }
    }
  }
  *margin = s1 - s2;
  return (int)b1;
}

/* Draw the bonus token from p = softmax(z) by Gumbel-max: argmax z_v + G(u_v).
 * *margin = best score - second best score. */
int svo_sample_bonus(int64_t V, const double* z, const float* u, double* margin) {
  int64_t b1 = -1, b2 = -1;
  double s1 = -INFINITY, s2 = -INFINITY;
  for (int64_t v = 0; v < V; ++v) {
    double sc = z[v] + gumbel((double)u[v]);
    if (b1 < 0 || sc > s1) { b2 = b1; s2 = s1; b1 = v; s1 = sc; }
    else if (b2 < 0 || sc > s2) { b2 = v; s2 = sc; }
  }
  *margin = s1 - s2;
  return (int)b1;
}

/* ------------------------------------------------------------------------ */
/* Single-pass sampling: candidates drawn from p in the first pass, the      */
/* residual reached by rejection                                             */
/* ------------------------------------------------------------------------ */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): ten rounds of two
 * 32 x 32 -> 64-bit products of the even counter words with the round
 * multipliers, the high halves xored with the odd words and the key, the key
 * bumped by the Weyl constants between rounds. */
void svo_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform r (0..3) of token v for draft row i of sequence b: word r of the
 * Philox4x32-10 block with counter (v, i, b, 0) and key (key0, key1).  Bits x
 * become the open-interval uniform ((x >> 9) + 1/2) 2^-23, exact in fp32. */
double svo_rs_uniform(uint32_t key0, uint32_t key1, int b, int i, int64_t v, int r) {
  const uint32_t ctr[4] = {(uint32_t)v, (uint32_t)i, (uint32_t)b, 0};
  const uint32_t key[2] = {key0, key1};
  uint32_t o[4];
  svo_philox4x32(ctr, key, o);
  return ((double)(o[r] >> 9) + 0.5) * ldexp(1.0, -23);
}

/* R independent draws from p = softmax(z) for draft row (b, i), each by
 * Gumbel-max with its own uniforms: cand[r] = argmax_v z_v + G(u_r(v)) (ties:
 * lowest id), margin[r] = best score - second best. */
void svo_rs_candidates(int64_t V, const double* z, uint32_t key0, uint32_t key1, int b, int i, int R,
                       int32_t* cand, double* margin) {
  for (int r = 0; r < R; ++r) {
    int64_t b1 = -1;
    double s1 = -INFINITY, s2 = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
      const double sc = z[v] + gumbel(svo_rs_uniform(key0, key1, b, i, v, r));
      if (b1 < 0 || sc > s1) { s2 = s1; b1 = v; s1 = sc; }
      else if (sc > s2) { s2 = sc; }
    }
    cand[r] = (int32_t)b1;
    margin[r] = s1 - s2;
  }
}

/* Residual draw by rejection from the candidates of the rejected row: candidate
 * x = cand[r] (a draw from p) is accepted iff u_rs[r] p(x) < p(x) - q(x), i.e.
 * with probability max(0, 1 - q(x) / p(x)); an accepted draw is distributed as
 * max(p - q, 0) normalised.  The first accepted candidate is returned, -1 if
 * none is (the caller then draws the residual directly).  p(x) = exp(z_x - lse);
 * margin[r] = (p - q - u p) for each tested candidate (its sign is the decision). */
int svo_rs_accept(int R, const int32_t* cand, const double* z, double lse, const float* q_row,
                  const float* u_rs, double* margin) {
  for (int r = 0; r < R; ++r) {
    const int32_t x = cand[r];
    const double p = exp(z[x] - lse), q = (double)q_row[x];
    margin[r] = (p - q) - (double)u_rs[r] * p;
    if ((double)u_rs[r] * p < p - q) return x;
  }
  return -1;
}

/* ------------------------------------------------------------------------ */
/* Trial driver for the statistical pins of the sampling rule               */
/* ------------------------------------------------------------------------ */

/* Runs T independent sampling-mode verify steps of a context-free toy target
 * (every row has the same logits z[V]) against a context-free toy drafter
 * (every draft drawn from the same q[V]), using only the functions above:
 * svo_accept_sample on the k drafts, then svo_sample_residual on the row of
 * the first rejection or svo_sample_bonus on row k.
 * drafts [T][k], u_acc [T][k], u_tok [T][V] are the trial's random inputs.
 * n_out[t] = accepted drafts, y_out[t] = the target's own emitted token. */
void svo_toy_spec_trials(int64_t T, int k, int64_t V, const double* z, const float* q,
                         const int32_t* drafts, const float* u_acc, const float* u_tok,
                         int32_t* n_out, int32_t* y_out) {
  double m = -INFINITY, acc = 0.0;
  for (int64_t v = 0; v < V; ++v) if (z[v] > m) m = z[v];
  for (int64_t v = 0; v < V; ++v) acc += exp(z[v] - m);
  const double lse = m + log(acc);
  double* lse_rows = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  double* dl = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  float* qd = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  double* mg = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < k; ++i) {
      int32_t d = drafts[t * k + i];
      lse_rows[i] = lse;
      dl[i] = z[d];
      qd[i] = q[d];
    }
    int n = svo_accept_sample(k, lse_rows, dl, qd, u_acc + t * k, mg);
    double margin;
    int y;
    if (n < k) y = svo_sample_residual(V, z, lse, q, u_tok + t * V, &margin);
    else y = svo_sample_bonus(V, z, u_tok + t * V, &margin);
    n_out[t] = n;
    y_out[t] = y;
  }
  free(lse_rows); free(dl); free(qd); free(mg);
}

/* The same toy with single-pass sampling: after a rejection at row n the
 * residual comes from R candidates of row n (svo_rs_candidates with key
 * (key0 + t, key1), sequence 0) by svo_rs_accept, and only if all are refused
 * from svo_sample_residual.  u_rs [T][R]; fb_out[t] = 1 when the fallback ran. */
void svo_toy_spec_trials_rs(int64_t T, int k, int64_t V, const double* z, const float* q,
                            const int32_t* drafts, const float* u_acc, const float* u_tok, uint32_t key0,
                            uint32_t key1, int R, const float* u_rs, int32_t* n_out, int32_t* y_out,
                            int32_t* fb_out) {
  double m = -INFINITY, acc = 0.0;
  for (int64_t v = 0; v < V; ++v) if (z[v] > m) m = z[v];
  for (int64_t v = 0; v < V; ++v) acc += exp(z[v] - m);
  const double lse = m + log(acc);
  double* lse_rows = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  double* dl = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  float* qd = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  double* mg = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
  double* cm = (double*)malloc(sizeof(double) * (size_t)R);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < k; ++i) {
      int32_t d = drafts[t * k + i];
      lse_rows[i] = lse;
      dl[i] = z[d];
      qd[i] = q[d];
    }
    int n = svo_accept_sample(k, lse_rows, dl, qd, u_acc + t * k, mg);
    double margin;
    int y, fb = 0;
    if (n < k) {
      svo_rs_candidates(V, z, key0 + (uint32_t)t, key1, 0, n, R, cand, cm);
      y = svo_rs_accept(R, cand, z, lse, q, u_rs + t * R, cm);
      if (y < 0) {
        fb = 1;
        y = svo_sample_residual(V, z, lse, q, u_tok + t * V, &margin);
      }
    } else {
      y = svo_sample_bonus(V, z, u_tok + t * V, &margin);
    }
    n_out[t] = n;
    y_out[t] = y;
    fb_out[t] = fb;
  }
  free(lse_rows); free(dl); free(qd); free(mg); free(cand); free(cm);
}
