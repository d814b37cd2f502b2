// lmhead.hip -- skinny GEMM on MFMA for the few verify rows, with fused epilogues:
//   * LM head + select over the vocabulary ("Gemma 4 拆解" (marsggbo), section 4.3:
//     the d x vocab unembed; section 4.2: argmax per position for
//     accept_longest_prefix).  Logits are reduced in registers to per-row
//     statistics (top-2, online log-sum-exp, the draft's logit, Gumbel-max draws)
//     and never written to memory; each workgroup leaves one partial per row
//     and lmhead_merge combines them in a fixed order (deterministic).
//   * plain projections of a decoder layer (store bf16, or add into the fp32
//     residual stream), optionally split along K with an ordered reduction.
//
// Tiling (bf16): the vocabulary / output features are the MFMA M side (16 per
// tile), the <= 64 verify rows the N side.  Each wave streams T tiles of W
// straight from HBM into MFMA A operands (16 B per lane, one k-step of 32
// columns per load), the rows of x come from L2 as B operands, and the
// accumulators stay in registers for the whole K range.
#include "sv_device.h"
#include "sv_host.h"

namespace sv {

enum GemmMode : int { GM_GREEDY = 0, GM_SAMPLE = 1, GM_RESIDUAL = 2, GM_STORE_BF16 = 3, GM_ADD_F32 = 4, GM_PARTIAL = 5 };

struct SelPart {   // per (workgroup, row) partial of the select epilogue
  float t1v, t2v;  // top-2 logits (RESIDUAL: residual-draw scores)
  int t1i, t2i;
  float m, s;      // log-sum-exp state
  float dl;        // draft logit (NaN if not in this workgroup's range)
  float s1v, s2v;  // top-2 perturbed scores (SAMPLE bonus rows / RESIDUAL fallback)
  int s1i, s2i;
  int pad;
};

struct GemmParams {
  const uint16_t* x;     // [R, K] rows (RESIDUAL: the hidden states, gathered per slot)
  const uint16_t* w;     // [N, K]
  int R, K, N;
  int k0_stride;         // K per split (split-K)
  int nblk;              // N blocks of the workgroup tile
  // select
  int batch, kdr;        // sequences and drafts per sequence
  const int32_t* drafts; // [batch, kdr]
  const float* u_tok;    // [batch, N]
  const float* q_rows;   // [batch, kdr, N]
  const sv_row_stats* stats_in;
  sv_accept_out* acc;
  SelPart* sel;          // [gridDim.x][R]
  // projections
  void* y;               // [R, N] bf16 or fp32
  float* part;           // [splits][R][N]
};

// ---------------------------------------------------------------------------
// select epilogue state (per lane, per row tile)
// ---------------------------------------------------------------------------
struct RowCtx {
  int r;                 // row (GREEDY/SAMPLE) or sequence slot (RESIDUAL)
  bool valid;
  int draft;             // token whose logit the row reports, -1 none
  bool bonus;            // SAMPLE: draw a Gumbel-max sample on this row
  const float* u;        // uniforms of the token draw
  const float* qrow;     // RESIDUAL: q distribution of the rejected draft
  float lse;             // RESIDUAL: log-partition of the row
};

struct RowState {
  Top2 a;                // top-2 logits (RESIDUAL: residual scores)
  LSE l;
  float dl;
  Top2 s;                // SAMPLE: perturbed scores; RESIDUAL: fallback draw from p
  __device__ __forceinline__ void init() {
    a.init();
    l.init();
    dl = __builtin_nanf("");
    s.init();
  }
};

template <int MODE>
__device__ __forceinline__ RowCtx make_ctx(const GemmParams& p, int r) {
  RowCtx c;
  c.r = r;
  c.valid = false;
  c.draft = -1;
  c.bonus = false;
  c.u = nullptr;
  c.qrow = nullptr;
  c.lse = 0.f;
  if constexpr (MODE == GM_RESIDUAL) {
    if (r < p.batch) {
      const sv_accept_out a = p.acc[r];
      // indices come from device memory: anything out of range is ignored
      if (a.residual_row >= 0 && a.residual_row < p.R && a.hidden_row >= 0 && a.hidden_row < p.R &&
          a.n_accepted >= 0 && a.n_accepted < p.kdr) {
        c.valid = true;
        c.u = p.u_tok + (int64_t)r * p.N;
        c.qrow = p.q_rows + ((int64_t)r * p.kdr + a.n_accepted) * p.N;
        c.lse = p.stats_in[a.residual_row].lse;
      }
    }
  } else {
    if (r < p.R) {
      c.valid = true;
      const int b = r / (p.kdr + 1), i = r % (p.kdr + 1);
      if (i < p.kdr) c.draft = p.drafts[b * p.kdr + i];
      if (MODE == GM_SAMPLE && i == p.kdr) {
        c.bonus = true;
        c.u = p.u_tok + (int64_t)b * p.N;
      }
    }
  }
  return c;
}

// fold four consecutive logits z[v0..v0+3] of one row into its state
template <int MODE>
__device__ __forceinline__ void select_push4(RowState& st, const RowCtx& c, const float z[4], int v0) {
  if (!c.valid) return;
  if constexpr (MODE == GM_RESIDUAL) {
    const f32x4_t q = *(const f32x4_t*)(c.qrow + v0);
    const f32x4_t u = *(const f32x4_t*)(c.u + v0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = gumbel(u[i]);
      const float rr = expf(z[i] - c.lse) - q[i];
      if (rr > 0.f) st.a.push(logf(rr) + g, v0 + i);
      st.s.push(z[i] + g, v0 + i);
    }
  } else {
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.a.push(z[i], v0 + i);
      e += exp2f((z[i] - mx) * kLog2e);
      if (v0 + i == c.draft) st.dl = z[i];
    }
    st.l.merge(mx, e);
    if (MODE == GM_SAMPLE && c.bonus) {
      const f32x4_t u = *(const f32x4_t*)(c.u + v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.s.push(z[i] + gumbel(u[i]), v0 + i);
    }
  }
}

__device__ __forceinline__ void state_merge(RowState& a, const RowState& b) {
  a.a.merge(b.a.v1, b.a.i1, b.a.v2, b.a.i2);
  a.l.merge(b.l.m, b.l.s);
  if (__builtin_isnan(a.dl)) a.dl = b.dl;
  a.s.merge(b.s.v1, b.s.i1, b.s.v2, b.s.i2);
}

__device__ __forceinline__ void state_merge_xor(RowState& st, int m) {
  RowState o;
  o.a.v1 = shfl_xor_f(st.a.v1, m); o.a.v2 = shfl_xor_f(st.a.v2, m);
  o.a.i1 = shfl_xor_i(st.a.i1, m); o.a.i2 = shfl_xor_i(st.a.i2, m);
  o.l.m = shfl_xor_f(st.l.m, m); o.l.s = shfl_xor_f(st.l.s, m);
  o.dl = shfl_xor_f(st.dl, m);
  o.s.v1 = shfl_xor_f(st.s.v1, m); o.s.v2 = shfl_xor_f(st.s.v2, m);
  o.s.i1 = shfl_xor_i(st.s.i1, m); o.s.i2 = shfl_xor_i(st.s.i2, m);
  state_merge(st, o);
}

__device__ __forceinline__ SelPart to_part(const RowState& s) {
  SelPart p;
  p.t1v = s.a.v1; p.t2v = s.a.v2; p.t1i = s.a.i1; p.t2i = s.a.i2;
  p.m = s.l.m; p.s = s.l.s; p.dl = s.dl;
  p.s1v = s.s.v1; p.s2v = s.s.v2; p.s1i = s.s.i1; p.s2i = s.s.i2;
  p.pad = 0;
  return p;
}
__device__ __forceinline__ RowState from_part(const SelPart& p) {
  RowState s;
  s.a.v1 = p.t1v; s.a.v2 = p.t2v; s.a.i1 = p.t1i; s.a.i2 = p.t2i;
  s.l.m = p.m; s.l.s = p.s; s.dl = p.dl;
  s.s.v1 = p.s1v; s.s.v2 = p.s2v; s.s.i1 = p.s1i; s.s.i2 = p.s2i;
  return s;
}

// ---------------------------------------------------------------------------
// bf16 MFMA skinny GEMM with fused epilogue
// ---------------------------------------------------------------------------
template <int MT, int T, int MODE>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmParams p) {
  constexpr bool SELECT = MODE <= GM_RESIDUAL;
  constexpr int NB = 4 * T * 16;       // output features per workgroup block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K;
  const int split = blockIdx.y;
  const int kbeg = split * p.k0_stride;
  const int nks = min(p.k0_stride, K - kbeg) / 32;

  // B operands: rows of x (gathered per slot in RESIDUAL mode)
  const uint16_t* xrow[MT];
  RowCtx ctx[MT];
  RowState st[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + lr;
    xrow[mt] = nullptr;
    if constexpr (SELECT) {
      ctx[mt] = make_ctx<MODE>(p, r);
      st[mt].init();
      if (ctx[mt].valid) {
        const int hr = MODE == GM_RESIDUAL ? p.acc[r].hidden_row : r;
        xrow[mt] = p.x + (int64_t)hr * K + kbeg + lg * 8;
      }
    } else {
      if (r < p.R) xrow[mt] = p.x + (int64_t)r * K + kbeg + lg * 8;
    }
  }

  for (int blk = blockIdx.x; blk < p.nblk; blk += gridDim.x) {
    const int n0 = blk * NB + wave * T * 16;
    const uint16_t* wrow[T];
    bool tv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      tv[t] = n0 + t * 16 < p.N;
      wrow[t] = p.w + (int64_t)(tv[t] ? n0 + t * 16 + lr : 0) * K + kbeg + lg * 8;
    }
    f32x4_t acc[T][MT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    V16 wc[T], xc[MT];
#pragma unroll
    for (int t = 0; t < T; ++t) wc[t].u = tv[t] ? *(const uint4*)(wrow[t]) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xc[mt].u = xrow[mt] ? *(const uint4*)(xrow[mt]) : make_uint4(0, 0, 0, 0);

    for (int ks = 0; ks < nks; ++ks) {
      V16 wn[T], xn[MT];
      const bool more = ks + 1 < nks;
      if (more) {
        const int o = (ks + 1) * 32;
#pragma unroll
        for (int t = 0; t < T; ++t) wn[t].u = tv[t] ? *(const uint4*)(wrow[t] + o) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xn[mt].u = xrow[mt] ? *(const uint4*)(xrow[mt] + o) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(wc[t].b, xc[mt].b, acc[t][mt]);
      if (more) {
#pragma unroll
        for (int t = 0; t < T; ++t) wc[t] = wn[t];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xc[mt] = xn[mt];
      }
    }

    // accumulator lane: row (mt*16 + lr), features n0 + 16 t + 4 lg + {0..3}
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (!tv[t]) continue;
      const int v0 = n0 + t * 16 + lg * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        const float z[4] = {acc[t][mt][0], acc[t][mt][1], acc[t][mt][2], acc[t][mt][3]};
        if constexpr (SELECT) {
          select_push4<MODE>(st[mt], ctx[mt], z, v0);
        } else if constexpr (MODE == GM_STORE_BF16) {
          if (r < p.R)
            *(uint2*)((uint16_t*)p.y + (int64_t)r * p.N + v0) = make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
        } else if constexpr (MODE == GM_ADD_F32) {
          if (r < p.R) {
            f32x4_t* d = (f32x4_t*)((float*)p.y + (int64_t)r * p.N + v0);
            f32x4_t o = *d;
            o[0] += z[0]; o[1] += z[1]; o[2] += z[2]; o[3] += z[3];
            *d = o;
          }
        } else {  // GM_PARTIAL
          if (r < p.R)
            *(f32x4_t*)(p.part + ((int64_t)split * p.R + r) * p.N + v0) = f32x4_t{z[0], z[1], z[2], z[3]};
        }
      }
    }
  }

  if constexpr (SELECT) {
    // lanes lr, lr+16, lr+32, lr+48 hold the same row: combine, then the 4 waves
    __shared__ SelPart s_sel[4][MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      state_merge_xor(st[mt], 16);
      state_merge_xor(st[mt], 32);
      if (lg == 0) s_sel[wave][mt][lr] = to_part(st[mt]);
    }
    __syncthreads();
    if (wave == 0 && lg == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        RowState a = from_part(s_sel[0][mt][lr]);
        for (int w = 1; w < 4; ++w) state_merge(a, from_part(s_sel[w][mt][lr]));
        const int nrows = MODE == GM_RESIDUAL ? p.batch : p.R;
        if (r < nrows) p.sel[(int64_t)blockIdx.x * nrows + r] = to_part(a);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 LM head (small vocabularies): one thread per vocabulary entry
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void lmhead_f32_kernel(GemmParams p, const float* x, const float* w) {
  __shared__ SelPart s_red[256];
  const int tid = threadIdx.x;
  const int v = blockIdx.x * 256 + tid;
  const int nrows = MODE == GM_RESIDUAL ? p.batch : p.R;
  for (int r = 0; r < nrows; ++r) {
    RowCtx c = make_ctx<MODE>(p, r);
    if (!c.valid) continue;   // uniform across the block
    const int hr = MODE == GM_RESIDUAL ? p.acc[r].hidden_row : r;
    RowState st;
    st.init();
    if (v < p.N) {
      const float* xr = x + (int64_t)hr * p.K;
      const float* wr = w + (int64_t)v * p.K;
      float z = 0.f;
      for (int d = 0; d < p.K; ++d) z = fmaf(xr[d], wr[d], z);
      if constexpr (MODE == GM_RESIDUAL) {
        const float g = gumbel(c.u[v]);
        const float rr = expf(z - c.lse) - c.qrow[v];
        if (rr > 0.f) st.a.push(logf(rr) + g, v);
        st.s.push(z + g, v);
      } else {
        st.a.push(z, v);
        st.l.merge(z, 1.f);
        if (v == c.draft) st.dl = z;
        if (MODE == GM_SAMPLE && c.bonus) st.s.push(z + gumbel(c.u[v]), v);
      }
    }
    s_red[tid] = to_part(st);
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) {
        RowState a = from_part(s_red[tid]);
        state_merge(a, from_part(s_red[tid + s]));
        s_red[tid] = to_part(a);
      }
      __syncthreads();
    }
    if (tid == 0) p.sel[(int64_t)blockIdx.x * nrows + r] = s_red[0];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// ordered merge of the per-workgroup partials
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void lmhead_merge_kernel(GemmParams p, int nparts, sv_row_stats* stats,
                                                           int32_t* out_tokens) {
  __shared__ SelPart s_red[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int nrows = MODE == GM_RESIDUAL ? p.batch : p.R;
  RowState a;
  a.init();
  for (int i = tid; i < nparts; i += 256) state_merge(a, from_part(p.sel[(int64_t)i * nrows + r]));
  s_red[tid] = to_part(a);
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      RowState x = from_part(s_red[tid]);
      state_merge(x, from_part(s_red[tid + s]));
      s_red[tid] = to_part(x);
    }
    __syncthreads();
  }
  if (tid != 0) return;
  const RowState f = from_part(s_red[0]);
  if constexpr (MODE == GM_RESIDUAL) {
    sv_accept_out* ac = p.acc + r;
    if (ac->residual_row < 0 || ac->residual_row >= p.R || ac->n_accepted < 0 || ac->n_accepted >= p.kdr)
      return;
    int y;
    float margin;
    if (f.a.i1 >= 0) { y = f.a.i1; margin = f.a.v1 - f.a.v2; }
    else { y = f.s.i1; margin = f.s.v1 - f.s.v2; }
    ac->next_token = y;
    ac->draw_margin = margin;
    out_tokens[(int64_t)r * (p.kdr + 1) + ac->n_accepted] = y;
  } else {
    sv_row_stats o;
    o.top1_id = f.a.i1;
    o.top2_id = f.a.i2;
    o.top1 = f.a.v1;
    o.top2 = f.a.v2;
    o.lse = f.l.m + logf(f.l.s);
    o.draft_logit = f.dl;
    o.sample_id = MODE == GM_SAMPLE ? f.s.i1 : -1;
    o.sample_s1 = MODE == GM_SAMPLE ? f.s.v1 : 0.f;
    o.sample_s2 = MODE == GM_SAMPLE ? f.s.v2 : 0.f;
    stats[r] = o;
  }
}

// ---------------------------------------------------------------------------
// split-K reduction of the projections (fixed split order)
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int splits) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t n = (int64_t)p.R * p.N;
  if (i4 >= n) return;
  f32x4_t a = *(const f32x4_t*)(p.part + i4);
  for (int s = 1; s < splits; ++s) {
    const f32x4_t o = *(const f32x4_t*)(p.part + (int64_t)s * n + i4);
    a[0] += o[0]; a[1] += o[1]; a[2] += o[2]; a[3] += o[3];
  }
  if constexpr (MODE == GM_STORE_BF16) {
    *(uint2*)((uint16_t*)p.y + i4) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
  } else {
    f32x4_t* d = (f32x4_t*)((float*)p.y + i4);
    f32x4_t o = *d;
    o[0] += a[0]; o[1] += a[1]; o[2] += a[2]; o[3] += a[3];
    *d = o;
  }
}

// fp32 projection (small shapes): one thread per output element
__global__ __launch_bounds__(256) void linear_f32_kernel(const float* x, const float* w, float* y, int R, int K,
                                                         int N, int add) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)R * N) return;
  const int r = (int)(i / N), n = (int)(i % N);
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(x[(int64_t)r * K + k], w[(int64_t)n * K + k], acc);
  y[i] = add ? y[i] + acc : acc;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int kSelT = 8;          // W tiles per wave in the LM head
static constexpr int kSelNB = 4 * kSelT * 16;
static constexpr int kSelGridMax = 1024;

static int lm_rows(const sv_lmhead_desc& d) { return d.batch * (d.k + 1); }

static int sel_grid(const sv_lmhead_desc& d) {
  if (d.dtype == SV_F32) return (d.vocab + 255) / 256;
  const int nblk = (d.vocab + kSelNB - 1) / kSelNB;
  return nblk < kSelGridMax ? nblk : kSelGridMax;
}

static int validate_lmhead(const sv_lmhead_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->batch <= 0 || d->k < 0 || d->d_model <= 0 || d->vocab <= 0) return SV_ERR_ARG;
  if (d->mode != SV_SELECT_GREEDY && d->mode != SV_SELECT_SAMPLE && d->mode != SV_SELECT_RESIDUAL) return SV_ERR_ARG;
  if (d->mode == SV_SELECT_RESIDUAL && d->k == 0) return SV_ERR_ARG;
  if (d->vocab % 64) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->d_model % 32) return SV_ERR_ARG;
    if (lm_rows(*d) > 64) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if (lm_rows(*d) > 256) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  return SV_OK;
}

template <int MT, int MODE>
static void launch_sel(const GemmParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, kSelT, MODE>), dim3(grid, 1), dim3(256), 0, s, p);
}

template <int MODE>
static int dispatch_sel(const GemmParams& p, int rows, int grid, hipStream_t s) {
  switch ((rows + 15) / 16) {
    case 1: launch_sel<1, MODE>(p, grid, s); break;
    case 2: launch_sel<2, MODE>(p, grid, s); break;
    case 3: launch_sel<3, MODE>(p, grid, s); break;
    case 4: launch_sel<4, MODE>(p, grid, s); break;
    default: return SV_ERR_UNSUPPORTED;
  }
  return SV_OK;
}

// projections: tiles per wave and K splits chosen so the grid fills the chip
static constexpr int kLinT = 2;
static constexpr int kLinNB = 4 * kLinT * 16;

struct LinPlan {
  int nblk, splits, kstride;
  size_t part_bytes;
};

static LinPlan lin_plan(const sv_linear_desc& d) {
  LinPlan pl{};
  pl.nblk = (d.out_features + kLinNB - 1) / kLinNB;
  pl.splits = 1;
  pl.kstride = d.in_features;
  if (d.dtype == SV_BF16) {
    const int ksteps = d.in_features / 32;
    int want = (1024 + pl.nblk - 1) / pl.nblk;  // aim at ~1024 workgroups
    if (want > ksteps / 8) want = ksteps / 8;  // keep >= 8 k-steps per split
    if (want > 16) want = 16;
    if (want < 1) want = 1;
    const int per = (ksteps + want - 1) / want;
    pl.kstride = per * 32;
    pl.splits = (d.in_features + pl.kstride - 1) / pl.kstride;
    if (pl.splits > 1) pl.part_bytes = align_up((size_t)pl.splits * d.rows * d.out_features * 4, 256);
  }
  return pl;
}

static int validate_linear(const sv_linear_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->rows <= 0 || d->in_features <= 0 || d->out_features <= 0) return SV_ERR_ARG;
  if (d->epilogue != SV_EPI_STORE && d->epilogue != SV_EPI_ADD_F32) return SV_ERR_ARG;
  if (d->out_features % 64) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->in_features % 32) return SV_ERR_ARG;
    if (d->rows > 64) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if ((int64_t)d->rows * d->out_features > ((int64_t)1 << 28)) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  return SV_OK;
}

template <int MT, int MODE>
static void launch_lin(const GemmParams& p, int gx, int gy, hipStream_t s) {
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, kLinT, MODE>), dim3(gx, gy), dim3(256), 0, s, p);
}

template <int MODE>
static int dispatch_lin(const GemmParams& p, int gx, int gy, hipStream_t s) {
  switch ((p.R + 15) / 16) {
    case 1: launch_lin<1, MODE>(p, gx, gy, s); break;
    case 2: launch_lin<2, MODE>(p, gx, gy, s); break;
    case 3: launch_lin<3, MODE>(p, gx, gy, s); break;
    case 4: launch_lin<4, MODE>(p, gx, gy, s); break;
    default: return SV_ERR_UNSUPPORTED;
  }
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_lmhead_workspace(const sv_lmhead_desc* d) {
  if (validate_lmhead(d) != SV_OK) return 0;
  const int nrows = d->mode == SV_SELECT_RESIDUAL ? d->batch : lm_rows(*d);
  return align_up((size_t)sel_grid(*d) * nrows * sizeof(SelPart), 256);
}

extern "C" int sv_lmhead_select(const sv_lmhead_desc* d, const void* hidden, const void* w,
                                const int32_t* drafts, const float* u_tok, const float* q_rows,
                                sv_row_stats* stats, sv_accept_out* acc, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_lmhead(d);
  if (rc != SV_OK) return rc;
  if (!hidden || !w || !stats) return SV_ERR_ARG;
  if (d->k > 0 && !drafts && d->mode != SV_SELECT_RESIDUAL) return SV_ERR_ARG;
  if (d->mode != SV_SELECT_GREEDY && !u_tok) return SV_ERR_ARG;
  if (d->mode == SV_SELECT_RESIDUAL && (!q_rows || !acc || !out_tokens)) return SV_ERR_ARG;
  if (workspace_bytes < sv_lmhead_workspace(d) || !workspace) return SV_ERR_WORKSPACE;
  rc = check_device();
  if (rc != SV_OK) return rc;

  GemmParams p{};
  p.x = (const uint16_t*)hidden;
  p.w = (const uint16_t*)w;
  p.R = lm_rows(*d);
  p.K = d->d_model;
  p.N = d->vocab;
  p.k0_stride = d->d_model;
  p.batch = d->batch;
  p.kdr = d->k;
  p.drafts = drafts;
  p.u_tok = u_tok;
  p.q_rows = q_rows;
  p.stats_in = stats;
  p.acc = acc;
  p.sel = (SelPart*)workspace;
  const int grid = sel_grid(*d);
  const int nrows = d->mode == SV_SELECT_RESIDUAL ? d->batch : p.R;
  hipStream_t s = (hipStream_t)stream;

  if (d->dtype == SV_BF16) {
    p.nblk = (d->vocab + kSelNB - 1) / kSelNB;
    switch (d->mode) {
      case SV_SELECT_GREEDY: rc = dispatch_sel<GM_GREEDY>(p, p.R, grid, s); break;
      case SV_SELECT_SAMPLE: rc = dispatch_sel<GM_SAMPLE>(p, p.R, grid, s); break;
      default: rc = dispatch_sel<GM_RESIDUAL>(p, d->batch, grid, s); break;
    }
    if (rc != SV_OK) return rc;
  } else {
    const float* xf = (const float*)hidden;
    const float* wf = (const float*)w;
    switch (d->mode) {
      case SV_SELECT_GREEDY: hipLaunchKernelGGL(lmhead_f32_kernel<GM_GREEDY>, dim3(grid), dim3(256), 0, s, p, xf, wf); break;
      case SV_SELECT_SAMPLE: hipLaunchKernelGGL(lmhead_f32_kernel<GM_SAMPLE>, dim3(grid), dim3(256), 0, s, p, xf, wf); break;
      default: hipLaunchKernelGGL(lmhead_f32_kernel<GM_RESIDUAL>, dim3(grid), dim3(256), 0, s, p, xf, wf); break;
    }
  }
  switch (d->mode) {
    case SV_SELECT_GREEDY:
      hipLaunchKernelGGL(lmhead_merge_kernel<GM_GREEDY>, dim3(nrows), dim3(256), 0, s, p, grid, stats, out_tokens);
      break;
    case SV_SELECT_SAMPLE:
      hipLaunchKernelGGL(lmhead_merge_kernel<GM_SAMPLE>, dim3(nrows), dim3(256), 0, s, p, grid, stats, out_tokens);
      break;
    default:
      hipLaunchKernelGGL(lmhead_merge_kernel<GM_RESIDUAL>, dim3(nrows), dim3(256), 0, s, p, grid, stats, out_tokens);
      break;
  }
  return launch_status();
}

extern "C" size_t sv_linear_workspace(const sv_linear_desc* d) {
  if (validate_linear(d) != SV_OK) return 0;
  return lin_plan(*d).part_bytes;
}

extern "C" int sv_linear(const sv_linear_desc* d, const void* x, const void* w, void* y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_linear(d);
  if (rc != SV_OK) return rc;
  if (!x || !w || !y) return SV_ERR_ARG;
  const LinPlan pl = lin_plan(*d);
  if (pl.part_bytes && (!workspace || workspace_bytes < pl.part_bytes)) return SV_ERR_WORKSPACE;
  rc = check_device();
  if (rc != SV_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (d->dtype == SV_F32) {
    const int64_t n = (int64_t)d->rows * d->out_features;
    hipLaunchKernelGGL(linear_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)x,
                       (const float*)w, (float*)y, d->rows, d->in_features, d->out_features,
                       d->epilogue == SV_EPI_ADD_F32 ? 1 : 0);
    return launch_status();
  }
  GemmParams p{};
  p.x = (const uint16_t*)x;
  p.w = (const uint16_t*)w;
  p.R = d->rows;
  p.K = d->in_features;
  p.N = d->out_features;
  p.k0_stride = pl.kstride;
  p.nblk = pl.nblk;
  p.y = y;
  p.part = (float*)workspace;
  const int gx = pl.nblk;
  if (pl.splits == 1) {
    rc = d->epilogue == SV_EPI_STORE ? dispatch_lin<GM_STORE_BF16>(p, gx, 1, s)
                                     : dispatch_lin<GM_ADD_F32>(p, gx, 1, s);
    if (rc != SV_OK) return rc;
  } else {
    rc = dispatch_lin<GM_PARTIAL>(p, gx, pl.splits, s);
    if (rc != SV_OK) return rc;
    const int64_t n4 = (int64_t)d->rows * d->out_features / 4;
    const unsigned g = (unsigned)((n4 + 255) / 256);
    if (d->epilogue == SV_EPI_STORE)
      hipLaunchKernelGGL(splitk_reduce_kernel<GM_STORE_BF16>, dim3(g), dim3(256), 0, s, p, pl.splits);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<GM_ADD_F32>, dim3(g), dim3(256), 0, s, p, pl.splits);
  }
  return launch_status();
}
