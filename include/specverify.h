/*
 * specverify.h -- C ABI of libspecverify: the verify step of MTP speculative
 * decoding on one AMD Instinct MI355X (gfx950).
 *
 * The calls follow the pages' statement of the problem:
 *   verify(draft_tokens, main_kv) -> logits, then accept_longest_prefix(draft_tokens,
 *   logits): "Gemma 4 拆解 | 多模态怎么塞进端侧，MTP drafter 又是怎么自带投机采样的"
 *   (marsggbo.github.io), section 4.2 (speculative_step).  The k drafts and one
 *   bonus position are scored in ONE target pass ("Accelerating Gemma 4: faster
 *   inference with multi-token prediction drafters" (Lighthouse), section 3)
 *   against a KV cache the drafter also reads ("Gemma 4 拆解", section 4.2:
 *   the drafter cross-attends the target's last local / global layer cache).
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers; the caller allocates and owns
 *     all memory (inputs, outputs and the workspace).  Descriptor pointers are
 *     HOST pointers, read before the call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t, NULL = the null
 *     stream): no host<->device copy, no synchronisation, no allocation.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call launches nothing and returns a negative sv_status.  A failed
 *     launch returns SV_ERR_LAUNCH.
 *   - Data-dependent errors found on the device (a cache that would overflow,
 *     a token id outside the vocabulary) OR bits into *dev_status (a device
 *     int32; NULL disables reporting) and the affected sequence is skipped or
 *     handled as documented; read the word after synchronising.
 *   - Tensors are dense row-major with the last dimension contiguous.
 *     Positions: query row j of sequence b sits at absolute position
 *     cache_len[b] + q_pos_offset + j.
 *   - The library holds no mutable global state (the one exception is the
 *     static scratch of sv_verify_attn_noalloc): calls on different streams
 *     that touch disjoint memory may overlap.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_ARG = -1,          /* a null pointer, a bad size, an inconsistent descriptor */
  SV_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. a head_dim with no kernel) */
  SV_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace() query */
  SV_ERR_LAUNCH = -4,       /* the HIP runtime rejected a kernel launch */
  SV_ERR_DEVICE = -5,       /* no usable gfx950 device is current */
  SV_ERR_SCRATCH = -6       /* sv_verify_attn_noalloc: the call needs more scratch than
                               SV_NOALLOC_SCRATCH_BYTES */
} sv_status;

/* SV_BF16X2 (an output type of the norms): a bf16 pair, two planes [2, ...] holding
 * hi = bf16(v) and lo = bf16(v - hi) of an fp32 value v -- hi + lo is within 2^-16 |v|
 * of v, and a bf16 MFMA takes it as two operands. */
/* The input enumerations of the ABI are fixed-width integers with named values, so
 * any value a caller passes is well defined and an unknown one is rejected. */
typedef int32_t sv_dtype;
enum { SV_F32 = 0, SV_BF16 = 1, SV_BF16X2 = 2 };

/* device status bits */
#define SV_DEV_CACHE_OVERFLOW 0x1  /* cache_len[b] + appended rows > cache_capacity */
#define SV_DEV_BAD_TOKEN 0x2       /* a token id outside [0, vocab) */
#define SV_DEV_BAD_LENGTH 0x4      /* cache_len[b] < 0 */

const char* sv_status_string(int status);
/* "libspecverify <version> gfx950" */
const char* sv_version(void);

/* ------------------------------------------------------------------------ */
/* Verify attention                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t batch;         /* B sequences */
  int32_t n_q;           /* query rows per sequence: k+1 in a verify step */
  int32_t n_heads_q;     /* Hq, a multiple of n_heads_kv */
  int32_t n_heads_kv;    /* Hkv */
  int32_t head_dim;      /* D: 128, 256 or 512 in bf16 (512 only with k_is_v); <= 512 in fp32 */
  int32_t window;        /* 0: global layer; W > 0: sliding window, key t is visible
                            to the query at position p iff p - W < t <= p */
  int32_t rope_dims;     /* rotated leading dims: 0 (none), D (full RoPE) or a fraction
                            of D (p-RoPE; D/4 on global layers) -- even, <= D */
  int32_t k_is_v;        /* 1: the layer stores one tensor used as key AND value
                            (v_cache, v_new must be NULL) */
  int32_t append;        /* 1: verify call -- rotate and write the n_q new key (value)
                            rows at cache rows [L, L+n_q) first; 0: read-only call (the
                            drafter's cross-attention), k_new/v_new must be NULL */
  int32_t q_pos_offset;  /* must be 0 when append == 1 */
  sv_dtype dtype;        /* of q, k_new, v_new, caches and out */
  int32_t in_splits;     /* 0: q, k_new, v_new hold values in dtype.  S > 0 (bf16 only):
                            they hold fp32 K-split partial products as SV_EPI_SPLIT_F32
                            writes them -- S slices, slice s of q at q + s*B*n_q*q_row_stride
                            elements (of k_new / v_new with kv_row_stride) -- and the value
                            used is bf16(sum of the slices in slice order), exactly what
                            an SV_EPI_STORE projection with the same slices would store */
  double rope_base;      /* theta_i = rope_base^(-2i/rope_dims) */
  float softmax_scale;   /* multiplies q.k before the softmax (1/sqrt(D)) */
  float reserved_f;      /* must be 0 */
  int64_t cache_capacity;/* rows per (sequence, kv head) in the cache tensors */
  int64_t q_row_stride;  /* elements between query rows (b, j) and (b, j+1); 0 = Hq*D */
  int64_t kv_row_stride; /* same for k_new / v_new; 0 = Hkv*D.  Lets q, k_new, v_new be
                            column slices of one fused projection output */
  int32_t act_pair;      /* 0: as above.  1 (dtype SV_BF16): pair activations -- q, k_new and
                            v_new are fp32 (or, with in_splits, their fp32 slice sums are used
                            without the bf16 rounding), so q and the new keys are rotated from
                            their fp32 values and k, v are rounded to the cache type only when
                            stored; out is written as a bf16 pair [2, B, n_q, Hq, D]: plane 0
                            hi = bf16(o), plane 1 lo = bf16(o - hi), together within 2^-16 |o|
                            of the fp32 result (the input sv_linear takes with act_pair).  The
                            caches and the rotated queries the products read stay bf16 */
  int32_t reserved_i;    /* must be 0 */
} sv_attn_desc;

/* Bytes of workspace sv_verify_attn needs for this descriptor (0 on an invalid
 * descriptor).  The workspace holds the rotated queries, the split-KV partial
 * results and per-(sequence, KV head) arrival counters; its contents are scratch
 * (set by the call itself), nothing survives the call. */
size_t sv_verify_attn_workspace(const sv_attn_desc* desc);

/* Verify attention over a shared KV cache, local (sliding window) or global
 * (causal; p-RoPE and K = V on Gemma-4-style global layers: "Gemma 4 拆解",
 * section 2; "Gemma 4 发布时未包含 MTP 数据——为什么这很重要" (flowhunt),
 * section "什么是 Gemma 4？").
 *
 *   q        [B, n_q, Hq, D]   queries before RoPE (row stride q_row_stride)
 *   k_new    [B, n_q, Hkv, D]  new keys before RoPE (append), else NULL (row stride
 *                              kv_row_stride)
 *   v_new    [B, n_q, Hkv, D]  new values (append and !k_is_v), else NULL
 *   k_cache  [B, Hkv, cap, D]  rotated keys; rows [L, L+n_q) written when append
 *   v_cache  [B, Hkv, cap, D]  values (NULL when k_is_v)
 *   cache_len[B] int32         committed rows L_b (read only)
 *   out      [B, n_q, Hq, D]   attention output per query head
 *
 * Query row j, head h (KV head h / (Hq/Hkv)) is rotated at position
 * p = L + q_pos_offset + j and attends to the keys t <= min(p, last stored
 * row) (and t > p - W on a window layer) with softmax(scale * q.k_t) weights.
 * RoPE pairs dim i with dim i + rope_dims/2 (rotate-half).  A query with no
 * visible key gets a zero row.  If L + n_q > cache_capacity on an append call
 * the sequence is skipped (out rows untouched) and SV_DEV_CACHE_OVERFLOW set.
 * bf16: batch <= 256 and cache_capacity < 2^31 - 4096, else SV_ERR_UNSUPPORTED. */
int sv_verify_attn(const sv_attn_desc* desc, const void* q, const void* k_new,
                   const void* v_new, void* k_cache, void* v_cache,
                   const int32_t* cache_len, void* out, void* workspace,
                   size_t workspace_bytes, int32_t* dev_status, void* stream);

/* The same verify attention over an fp8 KV cache: KV-cache quantization with
 * static, per-channel scales, as in the mobile quantization set of "Gemma 4 与
 * Gemini Nano：端侧智能的架构拆解" (kongchang), section "量化：为移动硬件定制的激进
 * 路线" (the 8-bit format is this library's choice).  desc is as above with dtype SV_BF16 (q, k_new,
 * v_new, out stay bf16); the caches hold one byte per element, an fp8 E4M3 code
 * (OCP E4M3FN: bias 7, largest magnitude 448, no infinities), and represent
 *   key[b, h, t, d] = k_scale[h, d] * e4m3(k_cache[b, h, t, d])
 * (the same for values with v_scale).  An appended row is stored as the code of
 * bf16(row) / scale (fp32 division, round to nearest even, saturating at +-448).
 * The products use the codes exactly: the key scales are folded into the rotated
 * queries (one bf16 rounding) and the value scales multiply the output.
 *   k_scale [Hkv, D] fp32, 16-byte aligned (also the value scales when k_is_v)
 *   v_scale [Hkv, D] fp32, 16-byte aligned; NULL when k_is_v
 * Workspace: sv_verify_attn_workspace(desc).  Errors as sv_verify_attn, plus
 * SV_ERR_ARG for a dtype other than bf16 or a missing or misaligned scale array. */
int sv_verify_attn_fp8(const sv_attn_desc* desc, const void* q, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                       const int32_t* cache_len, void* out, void* workspace, size_t workspace_bytes,
                       int32_t* dev_status, void* stream);

/* For callers that cannot allocate device memory: code recorded under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc.  sv_verify_attn
 * with the workspace replaced by a static device array of
 * SV_NOALLOC_SCRATCH_BYTES bytes inside the library: one copy per GPU, taken when
 * the library's code is loaded on that GPU and held until the process ends.  The
 * call allocates nothing and frees nothing.  Results are those of sv_verify_attn
 * (the same kernels).
 *   Arguments, layouts and device-side errors: as sv_verify_attn.
 *   Every call on one GPU uses that GPU's single array, and each call sets what it
 *   reads there itself (counters, work split), so calls ordered on one stream are
 *   independent; calls that overlap in time on one GPU (several streams or host
 *   threads) race on the array and give wrong results.
 *   Returns SV_ERR_SCRATCH (nothing launched) when the descriptor needs more than
 *   SV_NOALLOC_SCRATCH_BYTES of scratch on the current device: roughly
 *   (compute units + B*Hkv) * (Hq/Hkv) * n_q * (head_dim + 2) * 4 bytes plus the
 *   rotated queries, about 25 MiB for B = 8, 32 q / 4 KV heads, head_dim 512, n_q 5. */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)
int sv_verify_attn_noalloc(const sv_attn_desc* desc, const void* q, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, const int32_t* cache_len, void* out,
                           int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------ */
/* LM head + select                                                          */
/* ------------------------------------------------------------------------ */

typedef int32_t sv_select_mode;
enum {
  SV_SELECT_GREEDY = 0,    /* per-row argmax statistics */
  SV_SELECT_SAMPLE = 1,    /* GREEDY + a Gumbel-max draw from softmax(z) on bonus rows */
  SV_SELECT_RESIDUAL = 2,  /* draw from max(p - q, 0) for sequences that rejected */
  SV_SELECT_SAMPLE_RS = 3  /* SAMPLE + first-pass candidates for single-pass sampling
                              (sv_lmhead_select_rs, sv_accept_rs) */
};

/* Per-row result of the LM head (logits themselves are never written). */
typedef struct {
  int32_t top1_id, top2_id;  /* argmax and runner-up of z (ties: lowest id) */
  float top1, top2;          /* their logits */
  float lse;                 /* log sum_v exp(z_v) */
  float draft_logit;         /* z[draft of this row], NaN when the row has none */
  int32_t sample_id;         /* SAMPLE, bonus rows: argmax_v z_v + G(u_v); else -1 */
  float sample_s1, sample_s2;/* winning and runner-up perturbed scores */
} sv_row_stats;

/* One first-pass candidate of single-pass sampling: a draw from p = softmax(z) of a
 * draft row by Gumbel-max over counter-based uniforms. */
typedef struct {
  int32_t id;            /* the drawn token */
  float z;               /* its logit (p(id) = exp(z - lse of the row)) */
  float s1, s2;          /* winning and runner-up perturbed scores */
  int32_t pad;
} sv_rs_cand;
#define SV_RS_CANDIDATES 4

/* Per-sequence result of the accept step. */
typedef struct {
  int32_t n_accepted;    /* n_b in [0, k]: leading drafts accepted */
  int32_t next_token;    /* the target's own token y_b (-1 while a RESIDUAL draw is pending) */
  int32_t new_len;       /* committed length after the step: L_b + n_b + 1 */
  int32_t keep_begin;    /* cache rows [keep_begin, keep_end) are kept: [L_b, L_b+n_b+1) */
  int32_t keep_end;
  int32_t drop_begin;    /* rows [drop_begin, drop_end) = [L_b+n_b+1, L_b+k+1) are rolled
                            back; no data moves, the next append overwrites them */
  int32_t drop_end;
  int32_t hidden_row;    /* b(k+1)+n_b: the verify row whose last-layer hidden state is the
                            drafter's next prev_hidden ("Gemma 4 拆解", section 4.2) */
  int32_t residual_row;  /* SAMPLE: the rejected row whose residual must be drawn, else -1 */
  float draw_margin;     /* winner minus runner-up score of the draw that gave next_token */
} sv_accept_out;

typedef struct {
  int32_t batch;         /* B */
  int32_t k;             /* drafts per sequence; rows = B*(k+1), row b*(k+1)+i */
  int32_t d_model;       /* d, a multiple of 32 in bf16 */
  int32_t vocab;         /* V, a multiple of 64 */
  sv_select_mode mode;
  sv_dtype dtype;        /* of hidden and w */
  int32_t out_stride;    /* GREEDY / SAMPLE: when out_tokens is not NULL, the argmax of
                            row r goes to out_tokens[r * out_stride] (0 means 1): how a
                            drafter writes its token for step i into drafts[b][i] */
} sv_lmhead_desc;

/* Workspace of sv_lmhead_select, 0 for an invalid descriptor.  bf16: arrival
 * counters, split partials and per-workgroup select partials.  The workspace must be
 * zero-filled before its first use; every call leaves its counters zero again, so
 * one fill serves any sequence of calls (of any descriptor) on the same workspace.
 * Calls that overlap in time must not share a workspace.  The counters occupy the
 * first 256 KiB in every layout (shared with sv_linear's). */
size_t sv_lmhead_workspace(const sv_lmhead_desc* desc);

/* LM-head skinny GEMM z = h W^T fused with a split-vocabulary select
 * ("Gemma 4 拆解", section 4.3: the d x vocab unembed; the per-position argmax
 * of accept_longest_prefix, section 4.2).
 *
 *   hidden     [B*(k+1), d]  final hidden states (RESIDUAL: row acc[b].hidden_row is used)
 *   w          [V, d]        unembedding (tied embedding) table
 *   drafts     [B, k] int32  d_{b,1..k}; row b*(k+1)+i reports z[drafts[b][i]] (i < k)
 *   u_tok      [B, V] fp32   SAMPLE / RESIDUAL: uniforms in [0,1) of the token draw
 *                            (Gumbel noise G = -log(-log u)); NULL in GREEDY
 *   q_rows     [B, k, V] fp32 RESIDUAL: the drafter's distributions q_i; else NULL
 *   stats      [B*(k+1)]     GREEDY/SAMPLE: written; RESIDUAL: read (lse of the row)
 *   acc        [B]           RESIDUAL: read (residual_row, hidden_row, n_accepted) and
 *                            next_token / draw_margin written; else NULL
 *   out_tokens [B, k+1]      RESIDUAL: out_tokens[b][n_b] = the drawn token; GREEDY /
 *                            SAMPLE: optional, top1_id of row r at r * out_stride
 *
 * RESIDUAL draws, for each sequence with residual_row >= 0,
 * argmax over {v : r_v > 0} of log r_v + G(u_v), r_v = exp(z_v - lse) - q_v,
 * falling back to argmax z_v + G(u_v) if every r_v is 0.  Ties: lowest id. */
int sv_lmhead_select(const sv_lmhead_desc* desc, const void* hidden, const void* w,
                     const int32_t* drafts, const float* u_tok, const float* q_rows,
                     sv_row_stats* stats, sv_accept_out* acc, int32_t* out_tokens,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Single-pass sampling, first pass (the rejection of speculative sampling reached
 * without a second pass over w in most steps).  desc->mode must be
 * SV_SELECT_SAMPLE_RS; hidden, w, drafts, u_tok, stats and out_tokens are as in
 * SAMPLE mode (the bonus rows' Gumbel-max draw included).  In the same pass every
 * draft row b(k+1)+i, i < k, draws SV_RS_CANDIDATES independent tokens from its p:
 *   cands[(b k + i) * SV_RS_CANDIDATES + c].id = argmax_v z_v + G(u_c(v))
 * (ties: lowest id), u_c(v) from Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3"): word c of the block with key (key0, key1) and
 * counter (v, i, b, 0), as the uniform ((x >> 9) + 1/2) 2^-23; G(u) = -ln(-ln u)
 * in fp32 (hardware base-2 logarithms).  The caller changes the key every step.  cands [B*k, SV_RS_CANDIDATES];
 * bf16 only; workspace
 * sv_lmhead_workspace(desc). */
int sv_lmhead_select_rs(const sv_lmhead_desc* desc, const void* hidden, const void* w, const int32_t* drafts,
                        const float* u_tok, uint32_t key0, uint32_t key1, sv_row_stats* stats, sv_rs_cand* cands,
                        int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Clustered unembedding (a drafter's cheap unembed)                         */
/* ------------------------------------------------------------------------ */

/* "Gemma 4 拆解" (marsggbo), section 4.3 (cheap_unembed): score the rows against
 * per-cluster centroids, keep the best clusters, and compute real logits only for
 * the tokens of those clusters (about 4096 instead of the whole vocabulary).  The
 * vocabulary is cut into n_clusters equal clusters; the unembedding rows are given
 * grouped by cluster (w_perm row j holds token perm[j]; cluster c is rows
 * [c * V / n_clusters, (c + 1) * V / n_clusters)). */
typedef struct {
  int32_t rows;          /* R hidden rows (<= 64) */
  int32_t d_model;       /* d, a multiple of 8, <= 8192 */
  int32_t vocab;         /* V, a multiple of n_clusters */
  int32_t n_clusters;    /* C <= 4096 */
  int32_t top_clusters;  /* clusters kept per row, 1 <= top_clusters <= min(C, 64) */
  sv_dtype dtype;        /* bf16 only */
} sv_cluster_desc;

/* Workspace of sv_cluster_unembed (cluster score slices, kept clusters, per-block
 * select partials, arrival counters); 0 for an invalid descriptor.  Scratch: nothing
 * needs to survive between calls and nothing needs zeroing; calls that share one
 * workspace must be ordered (one stream). */
size_t sv_cluster_unembed_workspace(const sv_cluster_desc* desc);

/*   hidden     [R, d] bf16
 *   centroids  [C, d] bf16
 *   w_perm     [V, d] bf16   unembedding rows grouped by cluster
 *   perm       [V] int32     token id of each w_perm row
 *   stats      [R]           over the candidate tokens only: top1_id / top2_id (token
 *                            ids), their logits, lse = log sum over the candidates;
 *                            draft_logit NaN, sample_id -1
 *   clusters   [R, top_clusters] int32 (optional): the kept clusters, best first
 *   out_tokens optional: top1_id of row r at out_tokens[r * out_stride] (0 means 1)
 * Cluster scores s_c = h . centroid_c are fp32; the kept clusters are the
 * top_clusters largest (ties: lowest cluster index; a NaN score ranks as -inf);
 * logits are fp32 dot products; ties between tokens go to the lowest token id.
 * hidden, centroids and w_perm must be 16-byte aligned.  The caller owns every
 * buffer; perm entries are copied to the result as they are (not range-checked).
 * Errors: SV_ERR_ARG (bad descriptor, null or misaligned pointer, negative
 * out_stride), SV_ERR_UNSUPPORTED (beyond the limits above), SV_ERR_WORKSPACE. */
int sv_cluster_unembed(const sv_cluster_desc* desc, const void* hidden, const void* centroids,
                       const void* w_perm, const int32_t* perm, sv_row_stats* stats, int32_t* clusters,
                       int32_t* out_tokens, int32_t out_stride, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Accept                                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t batch;
  int32_t k;
  int32_t vocab;
  sv_select_mode mode;   /* GREEDY or SAMPLE */
} sv_accept_desc;

/* Longest-accepted-prefix rule with KV append / rollback indices
 * ("Gemma 4 拆解", section 4.1 and 4.2 accept_longest_prefix; "Gemma 4 发布时
 * 未包含 MTP 数据", section "什么是多标记预测？": cut at the first wrong draft).
 *
 * GREEDY: n_b = the largest m <= k with drafts[b][i] == stats[b(k+1)+i].top1_id
 *   for all i < m; next_token = stats[b(k+1)+n_b].top1_id.
 * SAMPLE (standard speculative rejection sampling, temperature 1; the pages
 *   assert only that it leaves the output distribution unchanged, "Gemma 4 与
 *   Gemini Nano：端侧智能的架构拆解" (kongchang), section "草稿模型"): draft i
 *   (1-based) is accepted iff u_accept[b][i-1] * q_rows[b][i-1][d_i] <
 *   exp(stats[row i-1].draft_logit - stats[row i-1].lse), stopping at the first
 *   rejection; if all k pass, next_token = stats[b(k+1)+k].sample_id, else it is
 *   left -1 with residual_row = b(k+1)+n_b for sv_lmhead_select(RESIDUAL).
 *
 *   drafts     [B, k] int32
 *   stats      [B*(k+1)]
 *   q_rows     [B, k, V] fp32  SAMPLE only, else NULL
 *   u_accept   [B, k] fp32     SAMPLE only, else NULL
 *   cache_len  [B] int32       in: L_b, out: L_b + n_b + 1
 *   out_tokens [B, k+1] int32  d_1..d_n, y, then -1
 *   acc        [B]             per-sequence results (see sv_accept_out)
 * A draft id outside [0, V) counts as a mismatch and sets SV_DEV_BAD_TOKEN. */
int sv_accept(const sv_accept_desc* desc, const int32_t* drafts, const sv_row_stats* stats,
              const float* q_rows, const float* u_accept, int32_t* cache_len,
              int32_t* out_tokens, sv_accept_out* acc, int32_t* dev_status, void* stream);

/* Accept step of single-pass sampling (desc->mode SV_SELECT_SAMPLE_RS).  Drafts
 * are accepted as in SAMPLE.  After a rejection at row n = n_b, the candidates
 * x_c of row b k + n are tested in order: x_c is taken iff
 *   u_rs[b][c] * p(x_c) < p(x_c) - q_rows[b][n][x_c],   p(x) = exp(z_x - lse_n),
 * i.e. with probability max(0, 1 - q/p), which makes the taken token a draw from
 * max(p - q, 0) normalised (rejection sampling with p as the proposal).  A taken
 * candidate becomes next_token (draw_margin = its Gumbel margin s1 - s2); if every
 * candidate is refused, next_token stays -1 and residual_row is set, exactly as in
 * SAMPLE, for the sv_lmhead_select(RESIDUAL) fallback.
 *   cands [B*k, SV_RS_CANDIDATES] from sv_lmhead_select_rs; u_rs [B, SV_RS_CANDIDATES]
 *   fp32 uniforms; the other arguments as sv_accept (q_rows and u_accept required). */
int sv_accept_rs(const sv_accept_desc* desc, const int32_t* drafts, const sv_row_stats* stats,
                 const sv_rs_cand* cands, const float* q_rows, const float* u_accept, const float* u_rs,
                 int32_t* cache_len, int32_t* out_tokens, sv_accept_out* acc, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------ */
/* Decoder-stack support (embedding, RMSNorm, projections, GeGLU)            */
/* ------------------------------------------------------------------------ */

/* x[r] = scale * table[tokens[r]] as fp32; an id outside [0, vocab) gives a zero
 * row and sets SV_DEV_BAD_TOKEN.  table [vocab, d] in `dtype`, x [rows, d] fp32. */
int sv_embed(int32_t rows, int32_t d_model, int32_t vocab, sv_dtype dtype,
             const int32_t* tokens, const void* table, float scale, float* x,
             int32_t* dev_status, void* stream);

/* y = x / sqrt(mean(x^2) + eps) * gain (gain NULL = unit gain); x [rows, dim] fp32,
 * gain [dim] fp32, y [rows, dim] in `out_dtype` (SV_BF16X2: [2, rows, dim], the pair
 * input of sv_linear with act_pair). */
int sv_rmsnorm(int32_t rows, int32_t dim, float eps, const float* x, const float* gain,
               void* y, sv_dtype out_dtype, void* stream);

/* Input stage of a drafter step ("Gemma 4 拆解", section 4.2: the drafter takes the
 * target's last-layer activation and the embedding of the last token, concatenated,
 * and projects them down to its own width).  For each sequence b:
 *   h = hidden[hidden_row[b * row_stride]]           (bf16 [rows_h, d_main])
 *   e = emb_scale * emb[tokens[b * tok_stride]]       (bf16 [vocab, d_draft])
 *   cat[b] = [rmsnorm(h), rmsnorm(e)]                 ([batch, d_main + d_draft] in cat_dtype:
 *                                                     SV_BF16, or SV_BF16X2 for the pair
 *                                                     [2, batch, d_main + d_draft] that
 *                                                     sv_linear takes with act_pair)
 *   x[b] = 0                                          (fp32 [batch, d_draft]: the drafter's
 *                                                     residual stream, which the down
 *                                                     projection then adds into)
 * rmsnorm has unit gain.  An out-of-range row or token sets SV_DEV_BAD_TOKEN and
 * gives that part zeros; another cat_dtype is SV_ERR_ARG. */
int sv_draft_input(int32_t batch, int32_t d_main, int32_t d_draft, float eps, const void* hidden,
                   int32_t rows_h, const int32_t* hidden_row, int32_t row_stride, const void* emb,
                   int32_t vocab, const int32_t* tokens, int32_t tok_stride, float emb_scale, void* cat,
                   sv_dtype cat_dtype, float* x, int32_t* dev_status, void* stream);

/* Residual add and RMSNorm in one launch (a pre-norm block's "x = x + f(...);
 * y = rmsnorm(x)"): x (fp32 [rows, dim], updated in place) += the sum of the
 * `splits` slices of parts (fp32 [splits, rows, dim], as SV_EPI_SPLIT_F32 writes
 * them; added in slice order, the sum then added to x), then y = rmsnorm(x) as
 * sv_rmsnorm (out_dtype SV_F32, SV_BF16 or SV_BF16X2).  parts NULL or splits 0: no
 * add.  dim % 4 == 0, x / parts / gain / y 16-byte aligned. */
int sv_add_rmsnorm(int32_t rows, int32_t dim, float eps, float* x, const float* parts, int32_t splits,
                   const float* gain, void* y, sv_dtype out_dtype, void* stream);

typedef int32_t sv_epilogue;
enum {
  SV_EPI_STORE = 0,      /* y = x W^T stored in the descriptor dtype */
  SV_EPI_ADD_F32 = 1,    /* y (fp32) += x W^T: a residual add */
  SV_EPI_GEGLU = 2,      /* bf16 only: the GeGLU gate fused into the gate/up projection.
                            W holds the gate and up rows interleaved by 16: rows
                            [32j, 32j+16) are gate features 16j..16j+15 and rows
                            [32j+16, 32j+32) the up features of the same indices;
                            y [R, N/2] bf16 gets gelu_tanh(g) * u with g and u rounded
                            to bf16 first (the values sv_geglu would read).  N % 128 == 0. */
  SV_EPI_SPLIT_F32 = 3   /* bf16 only: the product split over the input dims.  The K dims
                            are cut into S = sv_linear_splits(desc) equal ranges of whole
                            64-dim chunks; y (fp32 [S, R, N]) slice s receives the partial
                            product over range s, written whole (no accumulation), and the
                            sum over s in slice order is x W^T.  For a consumer that adds
                            the slices itself (sv_add_rmsnorm); the call needs no workspace
                            and writes every element of y. */
};

typedef struct {
  int32_t rows;          /* R <= 64 */
  int32_t in_features;   /* K, a multiple of 32 in bf16 */
  int32_t out_features;  /* N, a multiple of 64 */
  sv_dtype dtype;        /* of x and w (and y for SV_EPI_STORE) */
  sv_epilogue epilogue;
  int32_t act_pair;      /* 0: as above.  1 (dtype SV_BF16, weights bf16): pair activations --
                            x is a bf16 pair [2, R, K] (plane 0 hi = bf16(v), plane 1
                            lo = bf16(v - hi) of an fp32 activation v, together within
                            2^-16 |v|), multiplied as hi W^T + lo W^T (two MFMAs, fp32
                            accumulation); SV_EPI_STORE writes y in fp32; SV_EPI_GEGLU writes
                            gelu_tanh(g) * u, from the fp32 g and u (no bf16 rounding), as a
                            bf16 pair [2, R, N/2]; ADD_F32 and SPLIT_F32 are unchanged.
                            2: as 1, but SV_EPI_STORE writes y in bf16 (the fp32 result
                            rounded once, to nearest even).  Other values: SV_ERR_ARG */
  int32_t w_layout;      /* SV_W_ROWMAJOR: w is [N, K] row-major.  SV_W_TILED (bf16 only):
                            w is the tiled copy sv_linear_tile_weights made for a descriptor
                            with the same in_features, out_features, dtype and epilogue
                            (16-byte aligned).  Other values: SV_ERR_ARG */
} sv_linear_desc;

enum {
  SV_W_ROWMAJOR = 0,
  SV_W_TILED = 1         /* the weight stream reads one contiguous KiB per DMA instruction
                            instead of 128 bytes from each of eight rows (whole DRAM pages;
                            a DMA probe with the pair-activation chunk staged beside the
                            weights streamed 12 % more per workgroup this way).  Results are
                            bit for bit those of the row-major layout. */
};

/* S of SV_EPI_SPLIT_F32 for this shape on the current device (1 <= S <= the
 * device's compute units / ceil(N / 128)); 0 if the descriptor is invalid, not
 * SV_EPI_SPLIT_F32, or N is too large for a split (more than one workgroup's worth
 * of output features per compute unit). */
int32_t sv_linear_splits(const sv_linear_desc* desc);

/* Workspace of sv_linear (0 in fp32 and for SV_EPI_SPLIT_F32): arrival counters and split partials.  Same
 * contract as sv_lmhead_workspace: zero-filled before first use, left zero by
 * every call, one call at a time. */
size_t sv_linear_workspace(const sv_linear_desc* desc);

/* Bytes of the tiled copy of a weight for this descriptor (bf16; rows is not used):
 * ceil(N / 64T) * ceil(K / 64) tiles of 64T x 64 weights, T = 1 or 2 as the library picks
 * for the shape and epilogue; 0 if the descriptor is invalid or not bf16. */
size_t sv_linear_tiled_bytes(const sv_linear_desc* desc);

/* Write the tiled copy of w (bf16 [N, K] row-major, 16-byte aligned) into w_tiled
 * (sv_linear_tiled_bytes(desc) bytes, 16-byte aligned, caller-owned): for each block of
 * 64T output features and each 64-dim chunk of K, the chunk's weights in the order the
 * projection's DMA places them in LDS, zero past N and K.  Asynchronous on stream; the
 * desc's w_layout is ignored.  SV_ERR_ARG: bad descriptor, not bf16, null or misaligned
 * pointers. */
int sv_linear_tile_weights(const sv_linear_desc* desc, const void* w, void* w_tiled, void* stream);

/* Skinny projection y = x W^T for the few verify rows: x [R, K], W [N, K] (or its tiled
 * copy, desc->w_layout).
 * bf16: one persistent workgroup per CU over (64T-feature block, 64-dim chunk)
 * units; a block split across workgroups is summed in a fixed order, so results
 * are deterministic for a given device. */
int sv_linear(const sv_linear_desc* desc, const void* x, const void* w, void* y,
              void* workspace, size_t workspace_bytes, void* stream);

/* GeGLU gate: out[r][i] = gelu_tanh(gu[r][i]) * gu[r][d_ff + i] where gu [rows, 2*d_ff]
 * holds the gate projection then the up projection; out [rows, d_ff]; both in dtype. */
int sv_geglu(int32_t rows, int32_t d_ff, sv_dtype dtype, const void* gate_up, void* out,
             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
