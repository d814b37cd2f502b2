// lmhead.hip -- skinny GEMM on MFMA for the few verify rows, with fused epilogues:
//   * LM head + select over the vocabulary ("Gemma 4 拆解" (marsggbo), section 4.3:
//     the d x vocab unembed; section 4.2: argmax per position for
//     accept_longest_prefix).  Logits are reduced in registers to per-row
//     statistics (top-2, online log-sum-exp, the draft's logit, Gumbel-max draws)
//     and never written to memory; each workgroup leaves one partial per row
//     and lmhead_merge combines them in a fixed order (deterministic).
//   * plain projections of a decoder layer (store bf16, or add into the fp32
//     residual stream).
//
// Tiling (bf16): the vocabulary / output features are the MFMA M side (16 per
// tile), the <= 64 verify rows the N side.  One persistent workgroup per CU
// streams its share of W (and the rows of x) through an LDS ring fed by direct
// HBM -> LDS DMA; the accumulators stay in registers across the K range.
#include "sv_device.h"
#include "sv_host.h"

#include <type_traits>

namespace sv {

enum GemmMode : int { GM_GREEDY = 0, GM_SAMPLE = 1, GM_RESIDUAL = 2, GM_STORE_BF16 = 3, GM_ADD_F32 = 4, GM_GEGLU = 5,
                      GM_SPLIT = 6, GM_SAMPLE_RS = 7, GM_STORE_F32 = 8 };

struct SelPart {   // per (workgroup, row) partial of the select epilogue
  float t1v, t2v;  // top-2 logits (RESIDUAL: residual-draw scores)
  int t1i, t2i;
  float m, s;      // log-sum-exp state
  float dl;        // draft logit (NaN if not in this workgroup's range)
  float s1v, s2v;  // top-2 perturbed scores (SAMPLE bonus rows / RESIDUAL fallback)
  int s1i, s2i;
  int pad;
};

constexpr bool sample_mode(int m) { return m == GM_SAMPLE || m == GM_SAMPLE_RS; }
constexpr bool select_mode(int m) { return m <= GM_RESIDUAL || m == GM_SAMPLE_RS; }
constexpr int kRsCand = 4;  // first-pass candidates per draft row (single-pass sampling)

struct GemmParams {
  const void* x;         // [R, K] rows, bf16 (with the kernel's XF: two bf16 planes [2, R, K],
                         // hi then lo, of pair activations; RESIDUAL: the hidden states,
                         // gathered per slot)
  const uint16_t* w;     // [N, K], or (w_tiled) the tiled copy: per (block, chunk) the W part
                         // of a ring stage exactly as the DMA lays it out in LDS
  int w_tiled;
  int R, K, N;
  int nblk, kch;         // feature blocks, 64-wide K chunks
  // select
  int batch, kdr;        // sequences and drafts per sequence
  const int32_t* drafts; // [batch, kdr]
  const float* u_tok;    // [batch, N]
  const float* q_rows;   // [batch, kdr, N]
  const sv_row_stats* stats_in;
  sv_accept_out* acc;
  SelPart* sel;          // [grid][rows]
  // projections
  void* y;               // [R, N] bf16 or fp32
  // stream-K
  float* part;           // [grid][2][rows][NB] partial sums
  int splits;            // GM_SPLIT: K slices per block (grid = nblk * splits)
  int out_stride;        // GREEDY / SAMPLE: top-1 ids to out_tokens[r * out_stride]
  uint32_t rs_key0, rs_key1;  // SAMPLE_RS: Philox key of the candidate draws
  float* rs_part;        // SAMPLE_RS: [grid][rows][kRsCand][4] candidate partials
  sv_rs_cand* rs_out;    // SAMPLE_RS: [B*k][kRsCand] candidates of the draft rows
  int32_t* cnt;          // [nblk][4] arrival counters, zero between calls
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
  bool rs;               // SAMPLE_RS: a draft row, which draws candidates
  int rb, ri;            // SAMPLE_RS: its sequence and draft index
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
  c.rs = false;
  c.rb = 0;
  c.ri = 0;
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
      if (sample_mode(MODE) && i == p.kdr) {
        c.bonus = true;
        c.u = p.u_tok + (int64_t)b * p.N;
      }
      if (MODE == GM_SAMPLE_RS && i < p.kdr) {
        c.rs = true;
        c.rb = b;
        c.ri = i;
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
    if (sample_mode(MODE) && c.bonus) {
      const f32x4_t u = *(const f32x4_t*)(c.u + v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.s.push(z[i] + gumbel(u[i]), v0 + i);
    }
  }
}

// fold a wave tile's 4 T logits of one row, ids vbase + 16 t + i (t < T, i < 4),
// into its state (GREEDY / SAMPLE): one block maximum and one exponential per logit
// for the log-partition, the block's own top two merged into the running pair, all
// without divergent branches.
template <int MODE, int T>
__device__ __forceinline__ void select_fold(RowState& st, const RowCtx& c, const f32x4_t (&z)[T], int vbase) {
  if (!c.valid) return;
  float m = z[0][0];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, z[t][i]);
  const float mb = m * kLog2e;
  float e = 0.f;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) e += __builtin_amdgcn_exp2f(fmaf(z[t][i], kLog2e, -mb));
  st.l.merge(m, e);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (vbase + t * 16 + i == c.draft) st.dl = z[t][i];
  // the block's own best two (ids ascending, so a strictly larger value wins), then
  // one merge into the running pair
  float b1 = z[0][0], b2 = kNegInf;
  int j1 = vbase, j2 = -1;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = (t == 0 ? 1 : 0); i < 4; ++i) {
      const float v = z[t][i];
      const int id = vbase + t * 16 + i;
      const bool g1 = v > b1, g2 = v > b2;
      const float nb2 = g1 ? b1 : (g2 ? v : b2);
      const int nj2 = g1 ? j1 : (g2 ? id : j2);
      b1 = g1 ? v : b1;
      j1 = g1 ? id : j1;
      b2 = nb2;
      j2 = nj2;
    }
  st.a.merge(b1, j1, b2, j2);
  if (sample_mode(MODE) && c.bonus) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const f32x4_t u = *(const f32x4_t*)(c.u + vbase + t * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.s.push(z[t][i] + gumbel(u[i]), vbase + t * 16 + i);
    }
  }
}

// ---------------------------------------------------------------------------
// single-pass sampling: kRsCand independent Gumbel-max draws from p per draft row
// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011): ten rounds of 32 x 32 -> 64-bit products of counter words 0
// and 2 with the round multipliers; the key advances by the Weyl constants.  NL
// counters go through the rounds together: with one wave per SIMD nothing else
// hides a multiply's latency, so independent chains fill it; each product is one
// 64-bit multiply (high and low words at once).
template <int NL>
__device__ __forceinline__ void philox4x32(uint32_t (&c)[NL][4], uint32_t k0, uint32_t k1) {
#pragma unroll 2  // two rounds a trip (no register rotation), the rest rolled
  for (int r = 0; r < 10; ++r) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const uint64_t p0 = (uint64_t)0xD2511F53u * c[l][0];
      const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[l][2];
      const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[l][1] ^ k0;
      const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[l][3] ^ k1;
      c[l][0] = n0;
      c[l][1] = (uint32_t)p1;
      c[l][2] = n2;
      c[l][3] = (uint32_t)p0;
    }
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}
// open-interval uniform from 32 random bits: ((x >> 9) + 1/2) 2^-23, exact in fp32
__device__ __forceinline__ float rs_uniform(uint32_t x) { return ((float)(x >> 9) + 0.5f) * 0x1p-23f; }
// Gumbel noise -ln(-ln u) from the hardware base-2 logarithm (u in [2^-24, 1): no
// denormal or zero argument reaches either logarithm)
__device__ __forceinline__ float rs_gumbel(float u) {
  constexpr float kLn2 = 0.69314718056f;
  return -kLn2 * __builtin_amdgcn_logf(-kLn2 * __builtin_amdgcn_logf(u));
}

// per candidate: best and second-best perturbed score, the best's token id and logit
struct RsState {
  float s1[kRsCand], s2[kRsCand], z[kRsCand];
  int id[kRsCand];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int c = 0; c < kRsCand; ++c) {
      s1[c] = s2[c] = kNegInf;
      z[c] = 0.f;
      id[c] = -1;
    }
  }
  // ids reach a lane's state in ascending order, so on a tie the state's (smaller)
  // id stays: a strict compare decides, and the runner-up is max(s2, min(s1, sc))
  __device__ __forceinline__ void push(int c, float sc, int v, float zv) {
    const bool w = sc > s1[c];
    s2[c] = fmaxf(s2[c], fminf(s1[c], sc));
    s1[c] = fmaxf(s1[c], sc);
    z[c] = w ? zv : z[c];
    id[c] = w ? v : id[c];
  }
  __device__ __forceinline__ void merge(int c, float os1, float os2, int oid, float oz) {
    const bool w = beats(os1, oid, s1[c], id[c]);
    s2[c] = w ? fmaxf(s1[c], os2) : fmaxf(s2[c], os1);
    s1[c] = w ? os1 : s1[c];
    z[c] = w ? oz : z[c];
    id[c] = w ? oid : id[c];
  }
  __device__ __forceinline__ void merge_xor(int m) {
#pragma unroll
    for (int c = 0; c < kRsCand; ++c)
      merge(c, shfl_xor_f(s1[c], m), shfl_xor_f(s2[c], m), shfl_xor_i(id[c], m), shfl_xor_f(z[c], m));
  }
};

// candidate draws over four consecutive logits z[0..3] (ids v0 + e) of one draft
// row: token v takes the Philox block with counter (v, i, b, 0), word c for
// candidate c
__device__ __forceinline__ void rs_fold4(RsState& rs, const RowCtx& c, const GemmParams& p, const f32x4_t z,
                                         int v0) {
  if (!c.valid || !c.rs) return;
  uint32_t w[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e][0] = (uint32_t)(v0 + e);
    w[e][1] = (uint32_t)c.ri;
    w[e][2] = (uint32_t)c.rb;
    w[e][3] = 0u;
  }
  philox4x32<4>(w, p.rs_key0, p.rs_key1);
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int k = 0; k < kRsCand; ++k) rs.push(k, z[e] + rs_gumbel(rs_uniform(w[e][k])), v0 + e, z[e]);
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
// bf16 MFMA skinny GEMM, stream-K over a DMA ring, with fused epilogues
// ---------------------------------------------------------------------------
// Work units are (block of NB = 64 T output features, chunk of 64 input dims).
// The nblk * kch units are cut into `grid` contiguous ranges, one per persistent
// workgroup (one per CU: the ring takes the whole LDS).  Each chunk of W (NB rows
// x 128 B) and of x (16 MT rows x 128 B) is copied HBM/L2 -> LDS by direct DMA,
// NS chunks deep, and read back as MFMA operands.  A block whose chunk range
// spans several workgroups leaves one fp32 partial per workgroup; per wave slice
// an arrival counter picks the last arriver, which adds the partials in
// workgroup order (deterministic) and runs the epilogue.
// With XF (pair activations) a chunk of x is staged twice, the hi plane then the lo
// plane, each laid out like a bf16 chunk: 16 MT rows x 128 B, 16-byte slots
// swizzled by row.
// G = 2 wave groups (8 waves, two per SIMD): the waves of slot w in both groups own
// the same W rows; group g multiplies k-step g of every 64-dim chunk, and at the end of
// a block group 1 hands its accumulators to group 0 through the stage just consumed.
// Two waves per SIMD hide each other's MFMA and LDS latencies, which bind the pair
// projections at 40 rows with one wave per SIMD.
template <int MT, int T, int XF = 0, int G = 1>
struct RingCfg {
  static constexpr int NB = 64 * T;            // output features per block
  static constexpr int WI = 2 * T;             // W DMA instructions per wave slot per chunk
  static constexpr int WIW = WI / G;           // ... issued by each wave of the slot
  static constexpr int XI = 2 * MT * (XF ? 2 : 1);  // x DMA instructions per chunk (workgroup)
  static constexpr int NX = (XI + 4 * G - 1) / (4 * G);  // x DMA instructions per wave
  static constexpr int NI = WIW + NX;          // DMA instructions per wave per chunk
  static constexpr int WSTAGE = NB * 128;
  static constexpr int STAGEB = WSTAGE + XI * 1024;
  static constexpr int NS_FIT = (160 * 1024) / STAGEB;
  static constexpr int NS = NS_FIT < 6 ? NS_FIT : 6;
  static_assert(G == 1 || G == 2, "one or two wave groups");
  static_assert(WI % G == 0, "W DMA split over the groups");
  // tiles per round of the group hand-over: the largest divisor of T whose
  // [4 slots][TC][MT] accumulators fit one stage
  static constexpr int TC = (4 * T * MT * 1024 <= STAGEB) ? T : (4 * (T / 2) * MT * 1024 <= STAGEB) ? T / 2 : 1;
  static_assert(G == 1 || 4 * TC * MT * 1024 <= STAGEB, "group hand-over fits a stage");
  static_assert(NS >= 3, "ring needs three stages");
  static_assert((NS - 2) * NI <= 63, "vmcnt range");
  static_assert(4 * MT * 16 * (int)sizeof(SelPart) <= NS * STAGEB, "select merge reuses the ring");
};

// 16-byte slot swizzle inside a 128-byte row chunk (r = row % 16): 16 consecutive
// rows at the same chunk land in distinct bank groups.
__device__ __forceinline__ int gswz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// hardware places consecutive workgroups on consecutive XCDs; renumber so that
// consecutive ranges (which share blocks and their partials) sit on one XCD
__device__ __forceinline__ int logical_wg(int b, int P) {
  if (P & 7) return b;
  return (b & 7) * (P >> 3) + (b >> 3);
}


template <int MT, int T, int MODE, int XF = 0, int G = 1>
__global__ __launch_bounds__(256 * G) void gemm_ring_kernel(GemmParams p) {
  using C = RingCfg<MT, T, XF, G>;
  constexpr bool SELECT = select_mode(MODE);
  static_assert(G == 1 || MODE != GM_SAMPLE_RS, "the candidate draws run with one wave group");
  constexpr int NB = C::NB, NS = C::NS, WROWS = 16 * T;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * C::STAGEB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: DMA bases live in SGPRs
  const int wave = wid & 3, grp = wid >> 2;  // W row slot, wave group
  const int lr = lane & 15, lg = lane >> 4;
  const int K = p.K, KCH = p.kch, P = gridDim.x;
  // K-split slices (GM_SPLIT, workgroup me holds slice me % splits): where the slice
  // count divides 8, the hardware numbering keeps every workgroup of an XCD on the
  // same slice, so each XCD's L2 fetches only that slice's columns of x
  const int me = (MODE == GM_SPLIT && 8 % p.splits == 0) ? (int)blockIdx.x : logical_wg(blockIdx.x, P);
  const int64_t tot = (int64_t)p.nblk * KCH;
  const int c_begin = (int)(tot * me / P);
  const int n_it = (int)(tot * (me + 1) / P) - c_begin;
  const bool ragged = (K & 63) != 0;  // last chunk holds one k-step of 32
  const int nx = MODE == GM_RESIDUAL ? p.batch : p.R;
  const uint32_t ring_lds = lds_addr(ring);

  // ---- per-lane DMA offsets (loop invariant) ----
  const int dl8 = lane >> 3;
  const int cq[2] = {(lane & 7) ^ gswz(dl8), (lane & 7) ^ gswz(8 + dl8)};  // chunk fetched, by row parity
  const uint32_t adj[2] = {cq[0] >= 4 ? 64u : 0u, cq[1] >= 4 ? 64u : 0u};
  // this wave's W DMA instructions: WIW of its slot's WI (group g takes the g-th share)
  uint32_t woff[C::WIW];
#pragma unroll
  for (int i = 0; i < C::WIW; ++i) {
    const int iw = grp * C::WIW + i;
    woff[i] = (uint32_t)((iw * 8 + dl8) * K * 2 + cq[iw & 1] * 16);
  }
  uint32_t xoff[C::NX], xlds[C::NX], xadj[C::NX];
#pragma unroll
  for (int ii = 0; ii < C::NX; ++ii) {
    const int j = (wid + 4 * G * ii) < C::XI ? (wid + 4 * G * ii) : C::XI - 1;
    // XF: instruction j moves plane j / (2 MT) (0 = hi, 1 = lo) of the rows of 8-row
    // block j % (2 MT)
    const int plane = XF ? j / (2 * MT) : 0;
    const int jb = XF ? j % (2 * MT) : j;
    const int r = jb * 8 + dl8;
    int xr = 0;
    if (r < nx) {
      if constexpr (MODE == GM_RESIDUAL) {
        const int h = p.acc[r].hidden_row;
        xr = (h >= 0 && h < p.R) ? h : 0;
      } else {
        xr = r;
      }
    }
    xoff[ii] = (uint32_t)(((int64_t)plane * nx + xr) * K * 2 + cq[jb & 1] * 16);
    xadj[ii] = adj[jb & 1];
    xlds[ii] = (uint32_t)(C::WSTAGE + j * 1024);
  }

  // ---- select state ----
  RowCtx ctx[MT];
  RowState st[MT];
  RsState rs[MT];  // SAMPLE_RS only
  if constexpr (SELECT) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ctx[mt] = make_ctx<MODE>(p, mt * 16 + lr);
      st[mt].init();
      if constexpr (MODE == GM_SAMPLE_RS) rs[mt].init();
    }
  }

  // ---- DMA issue of chunk unit (b, kc) into ring stage s ----
  auto issue = [&](int b, int kc, int s) {
    const bool tail = ragged && kc == KCH - 1;
    const uint32_t dst = ring_lds + (uint32_t)(s * C::STAGEB);
    if (p.w_tiled) {
      // one contiguous 1 KiB per instruction: whole DRAM pages instead of 128 bytes from
      // each of 8 rows (zero padding covers the ragged last chunk and block)
      const uint8_t* wt = (const uint8_t*)p.w + ((int64_t)b * KCH + kc) * (NB * 128) + wave * C::WI * 1024;
#pragma unroll
      for (int i = 0; i < C::WIW; ++i) {
        const int iw = grp * C::WIW + i;
        dma16<true, true>(wt + iw * 1024, (uint32_t)(lane * 16), dst + (uint32_t)((wave * C::WI + iw) * 1024));
      }
    } else {
      const int row0 = b * NB + wave * WROWS;
      const uint8_t* wb = (const uint8_t*)p.w + ((int64_t)(row0 < p.N ? row0 : 0) * K + kc * 64) * 2;
#pragma unroll
      for (int i = 0; i < C::WIW; ++i) {
        const int iw = grp * C::WIW + i;
        dma16<true, true>(wb, woff[i] - (tail ? adj[iw & 1] : 0u), dst + (uint32_t)((wave * C::WI + iw) * 1024));
      }
    }
    const uint8_t* xb = (const uint8_t*)p.x + (int64_t)kc * 128;
#pragma unroll
    for (int ii = 0; ii < C::NX; ++ii) dma16(xb, xoff[ii] - (tail ? xadj[ii] : 0u), dst + xlds[ii]);
  };

  // ---- stream-K bookkeeping ----
  auto owner = [&](int64_t c) -> int { return (int)(((c + 1) * P - 1) / tot); };
  // partials [grid][2][nx][NB] fp32 behind a buffer descriptor (byte offsets)
  const __amdgpu_buffer_rsrc_t part_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(p.part, (short)0, (int)(P * 2 * nx * NB * 4), kBufferWord3);
  auto part_off = [&](int w, int sl, int r) -> uint32_t { return (uint32_t)((((w * 2 + sl) * nx + r) * NB) * 4); };
  auto first_block = [&](int w) -> int { return (int)((tot * w / P) / KCH); };
  const int my_first = c_begin / KCH;

  f32x4_t acc[T][MT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // end of this workgroup's range in block b; `full` if it covered the whole block
  auto seg_end = [&](int b, bool full) {
    const int row0 = b * NB + wave * WROWS;
    if (row0 >= p.N) return;  // wave slice past the last feature (uniform per wave)
    if constexpr (MODE == GM_SPLIT) {
      // workgroup me holds K slice me % splits of its block: the partial product goes
      // to that slice of y [splits][rows][N] for the consumer to add up
      float* ys = (float*)p.y + (int64_t)(me % p.splits) * nx * p.N;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = mt * 16 + lr;
          if (r < nx) *(f32x4_t*)(ys + (int64_t)r * p.N + row0 + t * 16 + lg * 4) = acc[t][mt];
        }
      return;
    }
    if (!full) {
      // Partials move through buffer stores / loads with the sc1 (device-coherent)
      // cache policy and the counter through a device-scope atomic: no L2 writeback
      // or invalidation (which a fence would issue) is needed.
      const int slot = b == my_first ? 0 : 1;
      const uint32_t lane_off = (uint32_t)((wave * WROWS + lg * 4) * 4);
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = mt * 16 + lr;
          if (r < nx)
            __builtin_amdgcn_raw_buffer_store_b128(acc[t][mt], part_rsrc,
                                                   part_off(me, slot, r) + lane_off + t * 64, 0, kCoherent);
        }
      wait_vm_n<0>();  // the partial stores have completed before the arrival is counted
      int old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + b * 4 + wave, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readfirstlane(old);
      const int w_lo = owner((int64_t)b * KCH), w_hi = owner((int64_t)b * KCH + KCH - 1);
      if (old != w_hi - w_lo) return;  // another workgroup finishes this slice
      asm volatile("" ::: "memory");
      // sum of the partials in workgroup order (this workgroup's own included),
      // DEPTH segments' loads in flight at a time
      constexpr int DEPTH = T >= 4 ? 1 : 4;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int w0 = w_lo; w0 <= w_hi; w0 += DEPTH) {
        f32x4_t v[DEPTH][T][MT];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          const int w = w0 + d;
          const int sl = (w <= w_hi && b == first_block(w)) ? 0 : 1;
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const int r = mt * 16 + lr;
              v[d][t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
              if (w <= w_hi && r < nx)
                v[d][t][mt] = __builtin_amdgcn_raw_buffer_load_b128(part_rsrc, part_off(w, sl, r) + lane_off + t * 64,
                                                                   0, kCoherent);
            }
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (w0 + d <= w_hi) {
                acc[t][mt][0] += v[d][t][mt][0]; acc[t][mt][1] += v[d][t][mt][1];
                acc[t][mt][2] += v[d][t][mt][2]; acc[t][mt][3] += v[d][t][mt][3];
              }
      }
      // every arrival has been counted: leave the counter zero for the next call
      if (lane == 0) __hip_atomic_store(p.cnt + b * 4 + wave, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // accumulator lane: x row (mt*16 + lr), features row0 + 16 t + 4 lg + {0..3}
    if constexpr (SELECT && MODE != GM_RESIDUAL) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t zt[T];
#pragma unroll
        for (int t = 0; t < T; ++t) zt[t] = acc[t][mt];
        select_fold<MODE, T>(st[mt], ctx[mt], zt, row0 + lg * 4);
        if constexpr (MODE == GM_SAMPLE_RS)
#pragma unroll
          for (int t = 0; t < T; ++t) rs_fold4(rs[mt], ctx[mt], p, zt[t], row0 + lg * 4 + t * 16);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int v0 = row0 + t * 16 + lg * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        const float z[4] = {acc[t][mt][0], acc[t][mt][1], acc[t][mt][2], acc[t][mt][3]};
        if constexpr (SELECT) {
          select_push4<MODE>(st[mt], ctx[mt], z, v0);
        } else if constexpr (MODE == GM_GEGLU) {
          // tile t - 1 holds the gate, tile t (odd) the up projection of the same 16
          // features (weights interleaved by 16 rows).  bf16 activations: both pass through bf16
          // as stored values and the product is stored bf16; pair activations (XF): the
          // product of the fp32 gate and up values is stored as a bf16 pair (hi plane,
          // lo plane [2, R, N/2])
          if ((t & 1) && r < nx) {
            const int c0 = (row0 + 16 * (t - 1)) / 2 + lg * 4;
            if constexpr (XF) {
              float f[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) f[e] = gelu_tanh(acc[t - 1][mt][e]) * acc[t][mt][e];
              uint16_t* y = (uint16_t*)p.y + (int64_t)r * (p.N / 2) + c0;
              const uint32_t h01 = pack_bf16x2(f[0], f[1]), h23 = pack_bf16x2(f[2], f[3]);
              *(uint2*)y = make_uint2(h01, h23);
              *(uint2*)(y + (int64_t)nx * (p.N / 2)) =
                  make_uint2(pack_bf16x2(f[0] - bf16_lo(h01), f[1] - bf16_hi(h01)),
                             pack_bf16x2(f[2] - bf16_lo(h23), f[3] - bf16_hi(h23)));
            } else {
              float f[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                f[e] = gelu_tanh(round_bf16(acc[t - 1][mt][e])) * round_bf16(acc[t][mt][e]);
              *(uint2*)((uint16_t*)p.y + (int64_t)r * (p.N / 2) + c0) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
            }
          }
        } else if constexpr (MODE == GM_STORE_F32) {
          if (r < nx) *(f32x4_t*)((float*)p.y + (int64_t)r * p.N + v0) = acc[t][mt];
        } else if constexpr (MODE == GM_STORE_BF16) {
          if (r < nx)
            *(uint2*)((uint16_t*)p.y + (int64_t)r * p.N + v0) = make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
        } else {  // GM_ADD_F32
          if (r < nx) {
            f32x4_t* d = (f32x4_t*)((float*)p.y + (int64_t)r * p.N + v0);
            f32x4_t o = *d;
            o[0] += z[0]; o[1] += z[1]; o[2] += z[2]; o[3] += z[3];
            *d = o;
          }
        }
      }
    }
  };

  // ---- the ring ----
  int ib = c_begin / KCH, ikc = c_begin - ib * KCH;  // next unit to issue
  const int npro = n_it < NS - 1 ? n_it : NS - 1;
  for (int i = 0; i < npro; ++i) {
    issue(ib, ikc, i);
    if (++ikc == KCH) { ikc = 0; ++ib; }
  }
  int cb = c_begin / KCH, ckc = c_begin - cb * KCH;  // unit being computed
  int seg_kc0 = ckc;                                 // first chunk of the current segment
  int s = 0, si = npro % NS;
  const uint8_t* wrd = ring + (wave * WROWS + lr) * 128;  // + t*2048 + chunk slot
  const uint8_t* xrd = ring + C::WSTAGE + lr * 128;        // + mt*2048 + chunk slot
  const int fsw = gswz(lr);
  for (int it = 0; it < n_it; ++it) {
    const int ahead = (NS - 2) < (n_it - 1 - it) ? (NS - 2) : (n_it - 1 - it);
    wait_stages<C::NI>(ahead);
    lds_barrier();  // unit `it` is in LDS for every wave; unit it-1 is no longer read
    if (it + NS - 1 < n_it) {
      issue(ib, ikc, si);
      if (++ikc == KCH) { ikc = 0; ++ib; }
      si = si + 1 == NS ? 0 : si + 1;
    }
    const int nks = (ragged && ckc == KCH - 1) ? 1 : 2;
    const uint8_t* ws = wrd + s * C::STAGEB;
    const uint8_t* xs = xrd + s * C::STAGEB;
    const int sc = s;  // the stage this iteration reads
    // k-steps of this chunk for this wave: both (one group), or k-step grp (two)
    const int js_end = G == 1 ? nks : (grp < nks ? grp + 1 : 0);
    for (int js = G == 1 ? 0 : grp; js < js_end; ++js) {
      const int so = ((js * 4 + lg) ^ fsw) << 4;
      V16 a[T];
#pragma unroll
      for (int t = 0; t < T; ++t) a[t].u = *(const uint4*)(ws + t * 2048 + so);
      if constexpr (XF) {
        // x W^T = hi W^T + lo W^T: the hi products of every tile pair first, then the lo
        // ones, so the two MFMAs into one accumulator are not back to back
        V16 bh[MT], bl[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bh[mt].u = *(const uint4*)(xs + mt * 2048 + so);
          bl[mt].u = *(const uint4*)(xs + (MT + mt) * 2048 + so);
        }
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(a[t].b, bh[mt].b, acc[t][mt]);
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(a[t].b, bl[mt].b, acc[t][mt]);
      } else {
        V16 bx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) bx[mt].u = *(const uint4*)(xs + mt * 2048 + so);
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16x16x32(a[t].b, bx[mt].b, acc[t][mt]);
      }
    }
    s = s + 1 == NS ? 0 : s + 1;
    if (ckc == KCH - 1 || it == n_it - 1) {
      if constexpr (G == 2) {
        // group 1 hands its k-step sums to group 0 through stage sc, TC tiles per
        // round: every wave has finished reading the stage, and its next DMA is issued
        // only after the next iteration's barrier.  Layout: [slot][tc][mt][lane] f32x4.
        constexpr int TC = C::TC;
        f32x4_t* xch = (f32x4_t*)(ring + sc * C::STAGEB) + (wave * TC * MT) * 64 + lane;
#pragma unroll
        for (int t0 = 0; t0 < T; t0 += TC) {
          lds_barrier();
          if (grp == 1) {
#pragma unroll
            for (int t = 0; t < TC; ++t)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) xch[(t * MT + mt) * 64] = acc[t0 + t][mt];
          }
          lds_barrier();
          if (grp == 0) {
#pragma unroll
            for (int t = 0; t < TC; ++t)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                const f32x4_t o = xch[(t * MT + mt) * 64];
                f32x4_t& a = acc[t0 + t][mt];
                a[0] += o[0]; a[1] += o[1]; a[2] += o[2]; a[3] += o[3];
              }
          }
        }
      }
      if (grp == 0) seg_end(cb, seg_kc0 == 0 && ckc == KCH - 1);
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      seg_kc0 = 0;
    }
    if (++ckc == KCH) { ckc = 0; ++cb; }
  }

  if constexpr (SELECT) {
    // lanes lr, lr+16, lr+32, lr+48 hold the same row: combine, then the 4 waves
    wait_vm_n<0>();
    __syncthreads();  // the ring is idle: reuse it
    SelPart* s_sel = (SelPart*)ring;  // [4][MT][16]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      state_merge_xor(st[mt], 16);
      state_merge_xor(st[mt], 32);
      if (lg == 0 && grp == 0) s_sel[(wave * MT + mt) * 16 + lr] = to_part(st[mt]);  // group 0 folded
    }
    __syncthreads();
    if (wid == 0 && lg == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        RowState a = from_part(s_sel[mt * 16 + lr]);
        for (int w = 1; w < 4; ++w) state_merge(a, from_part(s_sel[(w * MT + mt) * 16 + lr]));
        if (r < nx) p.sel[(int64_t)me * nx + r] = to_part(a);
      }
    }
    if constexpr (MODE == GM_SAMPLE_RS) {
      // candidate states: the same lane / wave combination, then one partial per row
      float* s_rs = (float*)(ring + 4 * MT * 16 * sizeof(SelPart));  // [4][MT][16][kRsCand][4]
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        rs[mt].merge_xor(16);
        rs[mt].merge_xor(32);
        if (lg == 0) {
          float* d = s_rs + (((wave * MT + mt) * 16 + lr) * kRsCand) * 4;
#pragma unroll
          for (int c = 0; c < kRsCand; ++c) {
            d[4 * c] = rs[mt].s1[c];
            d[4 * c + 1] = rs[mt].s2[c];
            d[4 * c + 2] = __int_as_float(rs[mt].id[c]);
            d[4 * c + 3] = rs[mt].z[c];
          }
        }
      }
      __syncthreads();
      if (wave == 0 && lg == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = mt * 16 + lr;
          RsState a = rs[mt];   // wave 0's own combined state
          for (int w = 1; w < 4; ++w) {
            const float* o = s_rs + (((w * MT + mt) * 16 + lr) * kRsCand) * 4;
#pragma unroll
            for (int c = 0; c < kRsCand; ++c) a.merge(c, o[4 * c], o[4 * c + 1], __float_as_int(o[4 * c + 2]), o[4 * c + 3]);
          }
          if (r < nx) {
            float* d = p.rs_part + (((int64_t)me * nx + r) * kRsCand) * 4;
#pragma unroll
            for (int c = 0; c < kRsCand; ++c) {
              d[4 * c] = a.s1[c];
              d[4 * c + 1] = a.s2[c];
              d[4 * c + 2] = __int_as_float(a.id[c]);
              d[4 * c + 3] = a.z[c];
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled weight copy for the ring GEMM: 16-byte unit u of tile (block b, chunk kc) is what
// lane u % 64 of W DMA instruction u / 64 moves into the ring stage, i.e. wave slot
// ins / (2T), rows slot*16T + (ins % 2T)*8 + lane/8 of the block, the 16-byte column
// slot (lane % 8) ^ gswz(row % 16) of the chunk; rows past N and columns past K are zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                           int N, int K, int T, int kch, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int NB = 64 * T, WI = 2 * T, WROWS = 16 * T;
  const int per_tile = NB * 8;  // 16-byte units per tile
  const int64_t tile = u / per_tile;
  const int su = (int)(u - tile * per_tile);
  const int b = (int)(tile / kch), kc = (int)(tile - (int64_t)b * kch);
  const int ins = su >> 6, lane = su & 63, dl8 = lane >> 3;
  const int iw = ins % WI;
  const int row = b * NB + (ins / WI) * WROWS + iw * 8 + dl8;
  const int k0 = kc * 64 + (((lane & 7) ^ gswz(((iw & 1) << 3) + dl8)) << 3);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < N && k0 < K) v = *(const uint4*)(w + (int64_t)row * K + k0);  // K % 32 == 0: k0 + 8 <= K
  *(uint4*)(wt + u * 8) = v;
}

// ---------------------------------------------------------------------------
// Clustered unembedding: centroid scores, kept clusters, logits of their tokens
// ---------------------------------------------------------------------------
struct ClusterParams {
  const uint16_t* h;     // [R, d]
  const uint16_t* cent;  // [C, d]
  const uint16_t* w;     // [V, d] grouped by cluster
  const int32_t* perm;   // [V] token id of each w row
  int R, d, V, C, top, csize, sub, splits;
  int cstride;           // scores row stride: C rounded up to a multiple of 4
  int gs;                // top-k group size in lanes (power of two <= 64)
  float* scores;         // [splits][R][cstride] fp32 slices, summed in slice order
  int32_t* kept;         // [R, top] best first
  float* part;           // [R][top * sub][kClPartWords] per-workgroup select partials
  int32_t* cnt;          // [R] arrivals of a row's logits workgroups
  uint32_t part_bytes;
  sv_row_stats* stats;
  int32_t* clusters;     // optional copy of kept
  int32_t* out_tokens;
  int out_stride;
};
constexpr int kClusterBlock = 64;    // tokens per logits workgroup (16 per wave)
constexpr int kClusterMaxC = 4096;   // clusters per row held by the top-k workgroup
constexpr int kClusterMaxD = 8192;   // hidden width staged in LDS by the logits kernel
constexpr int kClPartWords = 8;      // top1 v/i, top2 v/i, lse m/s, 2 spare
typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));

// grid (ceil(C / 16), R): each wave scores four centroids of one row (used when the
// centroid count or width does not fit the MFMA projection)
__device__ __forceinline__ float wave_dot_bf16(const uint16_t* a, const uint16_t* b, int d, int lane) {
  float acc = 0.f;
  for (int i = lane * 8; i < d; i += 512) {
    const uint4 av = *(const uint4*)(a + i), bv = *(const uint4*)(b + i);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(aw[e]), bf16_lo(bw[e]), acc);
      acc = fmaf(bf16_hi(aw[e]), bf16_hi(bw[e]), acc);
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) acc += shfl_xor_f(acc, m);
  return acc;
}

__global__ __launch_bounds__(256) void cluster_score_kernel(ClusterParams p) {
  const int r = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* hr = p.h + (int64_t)r * p.d;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = blockIdx.x * 16 + wave * 4 + q;
    if (c >= p.C) break;
    const float s = wave_dot_bf16(hr, p.cent + (int64_t)c * p.d, p.d, lane);
    if (lane == 0) p.scores[(int64_t)r * p.cstride + c] = s;
  }
}

// 64-bit ordering key of (score, cluster): larger key = larger score, then lower
// index; -0 is folded into +0 first so equal scores compare equal.  0 means none.
__device__ __forceinline__ uint64_t score_key(float x, int c) {
  const uint32_t u = __float_as_uint(x + 0.f);
  const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)hi << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// grid R, 1024 threads: the top largest cluster scores of row r, best first (ties:
// lowest index; a NaN score counts as -inf).  No sequential selection: thread t
// holds scores 4t .. 4t+3, as 64-bit keys ordered like the result.  (1) The scores
// with the same e = c % 4 in an aligned run of gs lanes form a group (gs a power
// of two <= 64, the largest giving at least 4 top groups, else 1).  The top-th
// largest group maximum is a lower bound of the top-th largest score: the group
// maxima at or above it are that many distinct scores.  (2) Scores at or above the
// bound are gathered in LDS (a little over `top` on typical inputs, all of them at
// worst).  (3) Each candidate's rank is the number of candidates with a larger key
// (eight lanes per candidate); ranks below top are written.  The block also zeroes
// the row's arrival counter of the logits kernel.
constexpr int kTopkThreads = 1024;
__global__ __launch_bounds__(kTopkThreads) void cluster_topk_kernel(ClusterParams p) {
  constexpr int SB = 16;
  static_assert(kClusterMaxC == 4 * kTopkThreads, "one float4 per thread");
  __shared__ uint64_t s_key[kClusterMaxC];   // group maxima, then candidates
  __shared__ int s_n;
  __shared__ uint64_t s_lo;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) {
    s_n = 0;
    s_lo = 0;
    p.cnt[r] = 0;
  }
  // the slices are added in slice order, SB slices' loads in flight at a time
  const int c0 = 4 * tid;
  const bool mine = c0 < p.C;   // scores rows are padded to a multiple of 4
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += SB) {
    f32x4_t x[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) {
      x[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (mine && s0 + q < p.splits) x[q] = *(const f32x4_t*)(p.scores + ((int64_t)(s0 + q) * p.R + r) * p.cstride + c0);
    }
#pragma unroll
    for (int q = 0; q < SB; ++q) v += x[q];
  }
  uint64_t key[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) key[e] = c0 + e >= p.C ? 0ull : score_key(v[e] == v[e] ? v[e] : kNegInf, c0 + e);
  // (1) group maxima: the lane at the start of each group writes its four
  uint64_t g[4] = {key[0], key[1], key[2], key[3]};
  for (int k = p.gs >> 1; k > 0; k >>= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t o = shfl_xor_u64(g[e], k);
      g[e] = o > g[e] ? o : g[e];
    }
  const int ng = 4 * (((p.C + 3) / 4 + p.gs - 1) / p.gs);   // group slots of the threads holding scores
  if ((lane & (p.gs - 1)) == 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_key[(tid / p.gs) * 4 + e] = g[e];
  __syncthreads();
  {
    // rank of each group maximum, eight lanes per slot; the one ranked top - 1 is
    // the bound (absent with fewer than top groups: the bound stays 0, take all)
    const int q = tid & 7;
    for (int i0 = 0; i0 < ng; i0 += kTopkThreads / 8) {
      const int i = i0 + (tid >> 3);
      const uint64_t me = i < ng ? s_key[i] : 0ull;
      int rank = 0;
      if (me != 0ull) {
        int j = q;
        for (; j + 24 < ng; j += 32) {
          uint64_t o[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = s_key[j + 8 * u];
#pragma unroll
          for (int u = 0; u < 4; ++u) rank += o[u] > me ? 1 : 0;
        }
        for (; j < ng; j += 8) rank += s_key[j] > me ? 1 : 0;
      }
      rank += __shfl_xor(rank, 1, 64);
      rank += __shfl_xor(rank, 2, 64);
      rank += __shfl_xor(rank, 4, 64);
      if (me != 0ull && q == 0 && rank == p.top - 1) s_lo = me;
    }
  }
  __syncthreads();
  const uint64_t lo = s_lo;
  __syncthreads();   // every lane has read the maxima before they are overwritten
  // (2) candidates
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool take = key[e] != 0ull && key[e] >= lo;
    const uint64_t mask = __ballot(take);
    const int nw = __popcll(mask);
    int base = 0;
    if (lane == 0 && nw) base = atomicAdd(&s_n, nw);
    base = __shfl(base, 0, 64);
    if (take) s_key[base + __popcll(mask & ((1ull << lane) - 1ull))] = key[e];
  }
  __syncthreads();
  // (3) ranks: eight lanes per candidate; lane q takes candidates q, q + 8, ...
  const int n = s_n, q = tid & 7;
  for (int i0 = 0; i0 < n; i0 += kTopkThreads / 8) {
    const int i = i0 + (tid >> 3);
    const bool act = i < n;
    const uint64_t me = act ? s_key[i] : 0ull;
    int rank = 0;
    if (act) {
      int j = q;
      for (; j + 24 < n; j += 32) {
        uint64_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = s_key[j + 8 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += o[u] > me ? 1 : 0;
      }
      for (; j < n; j += 8) rank += s_key[j] > me ? 1 : 0;
    }
    rank += __shfl_xor(rank, 1, 64);
    rank += __shfl_xor(rank, 2, 64);
    rank += __shfl_xor(rank, 4, 64);
    if (act && q == 0 && rank < p.top) {
      const int ci = (int)(0xFFFFFFFFu - (uint32_t)me);
      p.kept[(int64_t)r * p.top + rank] = ci;
      if (p.clusters) p.clusters[(int64_t)r * p.top + rank] = ci;
    }
  }
}

__device__ __forceinline__ void fma_bf16x8(float& acc, const uint4& a, const uint4& b) {
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf16_lo(aw[e]), bf16_lo(bw[e]), acc);
    acc = fmaf(bf16_hi(aw[e]), bf16_hi(bw[e]), acc);
  }
}

// grid (top * sub, R), 256 threads: logits of row r for up to kClusterBlock tokens of
// one kept cluster.  The row sits in LDS; each wave takes 16 tokens, four at a time
// with two 512-wide slices of each in flight (eight 16-byte loads per lane), then
// folds them into a running top-2 (by token id) and log-sum-exp.  The workgroup's
// partial goes to the device coherence point; the row's last workgroup to arrive
// merges all of them in slot order and writes the statistics.
__global__ __launch_bounds__(256) void cluster_logits_kernel(ClusterParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_h[kClusterMaxD];
  __shared__ RowState s_st[4];
  __shared__ int s_last;
  const int r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = blockIdx.x, nslot = p.top * p.sub;
  const int i = slot / p.sub, sb = slot - i * p.sub;
  const uint16_t* hr = p.h + (int64_t)r * p.d;
  for (int e = tid * 8; e < p.d; e += 2048) *(uint4*)(s_h + e) = *(const uint4*)(hr + e);
  const int c = p.kept[(int64_t)r * p.top + i];
  const bool ok = c >= 0 && c < p.C;   // always true: top <= C leaves a cluster to take
  const int j0 = ok ? c * p.csize + sb * kClusterBlock : 0;
  const int j1 = ok ? min(j0 + kClusterBlock, (c + 1) * p.csize) : 0;
  __syncthreads();
  RowState st;
  st.init();
  constexpr int TPW = kClusterBlock / 4, G = 4;
  for (int g = 0; g < TPW; g += G) {
    const int jb = j0 + wave * TPW + g;
    if (jb >= j1) break;
    const uint16_t* wr[G];
    int id[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int j = min(jb + t, j1 - 1);   // a ragged group repeats its last token; only valid ones count
      wr[t] = p.w + (int64_t)j * p.d;
      id[t] = p.perm[j];
    }
    float acc[G] = {0.f, 0.f, 0.f, 0.f};
    for (int e0 = lane * 8; e0 < p.d; e0 += 1024) {
      const int e1 = e0 + 512;
      uint4 a0[G], a1[G];
#pragma unroll
      for (int t = 0; t < G; ++t) a0[t] = *(const uint4*)(wr[t] + e0);
      if (e1 < p.d) {
#pragma unroll
        for (int t = 0; t < G; ++t) a1[t] = *(const uint4*)(wr[t] + e1);
      }
      const uint4 h0 = *(const uint4*)(s_h + e0);
#pragma unroll
      for (int t = 0; t < G; ++t) fma_bf16x8(acc[t], h0, a0[t]);
      if (e1 < p.d) {
        const uint4 h1 = *(const uint4*)(s_h + e1);
#pragma unroll
        for (int t = 0; t < G; ++t) fma_bf16x8(acc[t], h1, a1[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
#pragma unroll
      for (int k = 32; k > 0; k >>= 1) acc[t] += shfl_xor_f(acc[t], k);
    }
#pragma unroll
    for (int t = 0; t < G; ++t) {
      if (jb + t < j1) {
        st.a.push(acc[t], id[t]);
        st.l.merge(acc[t], 1.f);
      }
    }
  }
  if (lane == 0) s_st[wave] = st;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(p.part, (short)0, p.part_bytes, kBufferWord3);
  if (tid == 0) {
    RowState a = s_st[0];
    for (int w = 1; w < 4; ++w) state_merge(a, s_st[w]);
    const uint32_t off = (uint32_t)(((int64_t)r * nslot + slot) * kClPartWords * 4);
    const u32x4_t q0 = {__float_as_uint(a.a.v1), (uint32_t)a.a.i1, __float_as_uint(a.a.v2), (uint32_t)a.a.i2};
    const u32x4_t q1 = {__float_as_uint(a.l.m), __float_as_uint(a.l.s), 0u, 0u};
    __builtin_amdgcn_raw_buffer_store_b128(q0, rsrc, off, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(q1, rsrc, off + 16, 0, kCoherent);
    wait_vm_n<0>();
    s_last = __hip_atomic_fetch_add(p.cnt + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nslot - 1;
  }
  __syncthreads();
  if (!s_last || wave != 0) return;
  RowState a;
  a.init();
  for (int k = lane; k < nslot; k += 64) {
    const uint32_t off = (uint32_t)(((int64_t)r * nslot + k) * kClPartWords * 4);
    const u32x4_t q0 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kCoherent);
    const u32x4_t q1 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16, 0, kCoherent);
    RowState b;
    b.init();
    b.a.v1 = __uint_as_float(q0[0]); b.a.i1 = (int)q0[1]; b.a.v2 = __uint_as_float(q0[2]); b.a.i2 = (int)q0[3];
    b.l.m = __uint_as_float(q1[0]); b.l.s = __uint_as_float(q1[1]);
    state_merge(a, b);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) state_merge_xor(a, m);
  if (lane != 0) return;
  sv_row_stats o;
  o.top1_id = a.a.i1;
  o.top2_id = a.a.i2;
  o.top1 = a.a.v1;
  o.top2 = a.a.v2;
  o.lse = a.l.m + logf(a.l.s);
  o.draft_logit = __builtin_nanf("");
  o.sample_id = -1;
  o.sample_s1 = 0.f;
  o.sample_s2 = 0.f;
  p.stats[r] = o;
  if (p.out_tokens) p.out_tokens[(int64_t)r * p.out_stride] = a.a.i1;
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
  if constexpr (MODE == GM_SAMPLE_RS) {
    // wave c merges candidate c of a draft row over the workgroups' partials
    const int b = r / (p.kdr + 1), i = r % (p.kdr + 1), c = tid >> 6, lane = tid & 63;
    if (i < p.kdr && c < kRsCand) {
      RsState a;
      a.init();
      for (int w = lane; w < nparts; w += 64) {
        const float* o = p.rs_part + (((int64_t)w * nrows + r) * kRsCand + c) * 4;
        a.merge(c, o[0], o[1], __float_as_int(o[2]), o[3]);
      }
#pragma unroll
      for (int m = 32; m > 0; m >>= 1)
        a.merge(c, shfl_xor_f(a.s1[c], m), shfl_xor_f(a.s2[c], m), shfl_xor_i(a.id[c], m), shfl_xor_f(a.z[c], m));
      if (lane == 0) {
        sv_rs_cand o;
        o.id = a.id[c];
        o.z = a.z[c];
        o.s1 = a.s1[c];
        o.s2 = a.s2[c];
        o.pad = 0;
        p.rs_out[((int64_t)b * p.kdr + i) * kRsCand + c] = o;
      }
    }
  }
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
    o.sample_id = sample_mode(MODE) ? f.s.i1 : -1;
    o.sample_s1 = sample_mode(MODE) ? f.s.v1 : 0.f;
    o.sample_s2 = sample_mode(MODE) ? f.s.v2 : 0.f;
    stats[r] = o;
    if (out_tokens) out_tokens[(int64_t)r * p.out_stride] = f.a.i1;
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
static constexpr int kMaxWG = 256;   // persistent workgroups at most (workspace sizing)
// Arrival counters sit at the start of every workspace in a region of fixed size, so
// calls with different descriptors can share one workspace.
static constexpr int kCntWords = 65536;
static constexpr int kSelT = 4;      // W tiles per wave in the LM head
// W tiles per wave in the projections: one for small weights (more, shorter blocks:
// fewer workgroups share a block, so the ordered sum of split partials is short),
// two otherwise (half the x re-reads per weight byte)
static int lin_tiles(const sv_linear_desc& d) {
  if (d.epilogue == SV_EPI_GEGLU) return 2;  // a wave's two tiles pair gate and up rows
  if (d.epilogue == SV_EPI_SPLIT_F32) return 2;  // no fixup: fewer x re-reads per weight byte win
  return (int64_t)d.in_features * d.out_features < ((int64_t)24 << 20) ? 1 : 2;
}

struct RingPlan {
  int T, nx, nblk, kch, grid;
  size_t cnt_bytes, part_bytes;
};

static RingPlan ring_plan(int T, int nx, int K, int N, int max_wg) {
  RingPlan pl{};
  pl.T = T;
  pl.nx = nx;
  pl.nblk = (N + 64 * T - 1) / (64 * T);
  pl.kch = (K + 63) / 64;
  const int64_t tot = (int64_t)pl.nblk * pl.kch;
  pl.grid = (int)(tot < max_wg ? tot : max_wg);
  // Prefer a grid in which every workgroup takes one equal slice of one block
  // (nblk * S workgroups, S dividing the chunk count) or whole blocks (a divisor
  // of nblk): a slice boundary never falls inside a workgroup's range, so no
  // workgroup stops its stream midway to publish a partial sum.
  int aligned = 0;
  if (pl.nblk <= max_wg) {
    for (int S = max_wg / pl.nblk; S >= 1 && !aligned; --S)
      if (pl.kch % S == 0) aligned = pl.nblk * S;
  } else {
    for (int g = max_wg; g > max_wg / 2 && !aligned; --g)
      if (pl.nblk % g == 0) aligned = g;
  }
  if (aligned * 8 >= max_wg * 7) pl.grid = aligned;
  pl.cnt_bytes = (size_t)kCntWords * sizeof(int32_t);
  pl.part_bytes = align_up((size_t)kMaxWG * 2 * nx * 64 * T * sizeof(float), 256);
  return pl;
}

// K-split plan of SV_EPI_SPLIT_F32: nblk * S workgroups, S the largest divisor of
// the chunk count with nblk * S <= max_wg, so workgroup me takes exactly slice
// me % S of block me / S.  0 if the blocks alone exceed max_wg.
static int split_count(const RingPlan& pl, int max_wg) {
  if (pl.nblk > max_wg) return 0;
  for (int S = max_wg / pl.nblk; S >= 1; --S)
    if (pl.kch % S == 0) return S;
  return 1;
}

static int live_wg() {
  const int c = device_cus();
  return c < kMaxWG ? c : kMaxWG;
}

static int lm_rows(const sv_lmhead_desc& d) { return d.batch * (d.k + 1); }
static int sel_rows(const sv_lmhead_desc& d) { return d.mode == SV_SELECT_RESIDUAL ? d.batch : lm_rows(d); }
static int f32_grid(const sv_lmhead_desc& d) { return (d.vocab + 255) / 256; }

static int validate_lmhead(const sv_lmhead_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->batch <= 0 || d->k < 0 || d->d_model <= 0 || d->vocab <= 0) return SV_ERR_ARG;
  if (d->mode != SV_SELECT_GREEDY && d->mode != SV_SELECT_SAMPLE && d->mode != SV_SELECT_RESIDUAL &&
      d->mode != SV_SELECT_SAMPLE_RS)
    return SV_ERR_ARG;
  if (d->mode == SV_SELECT_RESIDUAL && d->k == 0) return SV_ERR_ARG;
  if (d->mode == SV_SELECT_SAMPLE_RS && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->out_stride < 0) return SV_ERR_ARG;
  if (d->vocab % 64) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->d_model % 32) return SV_ERR_ARG;
    if (lm_rows(*d) > 64) return SV_ERR_UNSUPPORTED;
    if ((int64_t)(d->vocab + 64 * kSelT - 1) / (64 * kSelT) * 4 > kCntWords) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if (lm_rows(*d) > 256) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  return SV_OK;
}

// Pair-activation projections and the LM head's greedy / sampling / residual selects
// run two wave groups (8 waves); the single-pass candidate draws keep one (their
// per-row state does not fit two waves per SIMD).
template <int MT, int T, int MODE, int XF>
static void launch_ring(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int G = ((XF && !select_mode(MODE)) || (select_mode(MODE) && MODE != GM_SAMPLE_RS)) ? 2 : 1;
  hipLaunchKernelGGL((gemm_ring_kernel<MT, T, MODE, XF, G>), dim3(grid), dim3(256 * G), 0, s, p);
}

template <int T, int MODE, int XF = 0>
static int dispatch_ring(const GemmParams& p, int nx, int grid, hipStream_t s) {
  switch ((nx + 15) / 16) {
    case 1: launch_ring<1, T, MODE, XF>(p, grid, s); break;
    case 2: launch_ring<2, T, MODE, XF>(p, grid, s); break;
    case 3: launch_ring<3, T, MODE, XF>(p, grid, s); break;
    case 4: launch_ring<4, T, MODE, XF>(p, grid, s); break;
    default: return SV_ERR_UNSUPPORTED;
  }
  return SV_OK;
}

static int validate_linear(const sv_linear_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->rows <= 0 || d->in_features <= 0 || d->out_features <= 0) return SV_ERR_ARG;
  if (d->epilogue != SV_EPI_STORE && d->epilogue != SV_EPI_ADD_F32 && d->epilogue != SV_EPI_GEGLU &&
      d->epilogue != SV_EPI_SPLIT_F32)
    return SV_ERR_ARG;
  if (d->epilogue == SV_EPI_SPLIT_F32 && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->act_pair < 0 || d->act_pair > 2) return SV_ERR_ARG;
  if (d->act_pair && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->w_layout != SV_W_ROWMAJOR && d->w_layout != SV_W_TILED) return SV_ERR_ARG;
  if (d->w_layout == SV_W_TILED && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->out_features % 64) return SV_ERR_ARG;
  if (d->epilogue == SV_EPI_GEGLU && (d->dtype != SV_BF16 || d->out_features % 128)) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->in_features % 32) return SV_ERR_ARG;
    if (d->rows > 64) return SV_ERR_UNSUPPORTED;
    if ((int64_t)(d->out_features + 63) / 64 * 4 > kCntWords) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if ((int64_t)d->rows * d->out_features > ((int64_t)1 << 28)) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  return SV_OK;
}

}  // namespace sv

using namespace sv;

static int validate_cluster(const sv_cluster_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->rows <= 0 || d->d_model <= 0 || d->vocab <= 0 || d->n_clusters <= 0 || d->top_clusters <= 0)
    return SV_ERR_ARG;
  if (d->dtype != SV_BF16 || d->d_model % 8 || d->vocab % d->n_clusters) return SV_ERR_ARG;
  if (d->top_clusters > d->n_clusters) return SV_ERR_ARG;
  if (d->rows > 64 || d->n_clusters > kClusterMaxC || d->top_clusters > 64 || d->d_model > kClusterMaxD)
    return SV_ERR_UNSUPPORTED;
  const int64_t sub = (d->vocab / d->n_clusters + kClusterBlock - 1) / kClusterBlock;
  if ((int64_t)d->rows * d->top_clusters * sub * kClPartWords * 4 > ((int64_t)1 << 31)) return SV_ERR_UNSUPPORTED;
  return SV_OK;
}

// Cluster scores come from the MFMA projection with K-split fp32 slices when the
// centroid count and width fit it, else from the plain per-centroid kernel.
static bool cluster_scores_by_gemm(const sv_cluster_desc& d) {
  return d.n_clusters % 64 == 0 && d.d_model % 32 == 0;
}

// Lanes per top-k group: the largest power of two <= 64 for which at least 4 top
// groups hold a score, else 1 (every score its own group).  Thread t holds scores
// 4t + e; the scores of residue e live on the first ceil((C - e) / 4) threads.
static int topk_group_lanes(int C, int top) {
  for (int gs = 64; gs > 1; gs >>= 1) {
    int groups = 0;
    for (int e = 0; e < 4 && e < C; ++e) {
      const int ne = (C - e + 3) / 4;
      groups += (ne + gs - 1) / gs;
    }
    if (groups >= 4 * top) return gs;
  }
  return 1;
}

struct ClusterPlan {
  int csize, sub, nslot;
  size_t scores, kept, part, cnt, total;
};
static ClusterPlan cluster_plan(const sv_cluster_desc& d) {
  ClusterPlan pl{};
  pl.csize = d.vocab / d.n_clusters;
  pl.sub = (pl.csize + kClusterBlock - 1) / kClusterBlock;
  pl.nslot = d.top_clusters * pl.sub;
  int smax = 1;   // slices at most (the split count only shrinks with fewer compute units)
  if (cluster_scores_by_gemm(d)) {
    const RingPlan rp = ring_plan(2, d.rows, d.d_model, d.n_clusters, kMaxWG);
    smax = split_count(rp, kMaxWG);
    if (smax < 1) smax = 1;
  }
  pl.scores = align_up((size_t)smax * d.rows * ((d.n_clusters + 3) / 4 * 4) * 4, 256);
  pl.kept = align_up((size_t)d.rows * d.top_clusters * 4, 256);
  pl.part = align_up((size_t)d.rows * pl.nslot * kClPartWords * 4, 256);
  pl.cnt = align_up((size_t)d.rows * 4, 256);
  pl.total = pl.scores + pl.kept + pl.part + pl.cnt;
  return pl;
}

extern "C" size_t sv_cluster_unembed_workspace(const sv_cluster_desc* d) {
  if (validate_cluster(d) != SV_OK) return 0;
  return cluster_plan(*d).total;
}

extern "C" int sv_cluster_unembed(const sv_cluster_desc* d, const void* hidden, const void* centroids,
                                  const void* w_perm, const int32_t* perm, sv_row_stats* stats, int32_t* clusters,
                                  int32_t* out_tokens, int32_t out_stride, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  int rc = validate_cluster(d);
  if (rc != SV_OK) return rc;
  if (!hidden || !centroids || !w_perm || !perm || !stats || out_stride < 0) return SV_ERR_ARG;
  if (((uintptr_t)hidden | (uintptr_t)centroids | (uintptr_t)w_perm) & 15) return SV_ERR_ARG;
  const ClusterPlan pl = cluster_plan(*d);
  if (!workspace || workspace_bytes < pl.total) return SV_ERR_WORKSPACE;
  rc = check_device();
  if (rc != SV_OK) return rc;
  ClusterParams p{};
  p.h = (const uint16_t*)hidden;
  p.cent = (const uint16_t*)centroids;
  p.w = (const uint16_t*)w_perm;
  p.perm = perm;
  p.R = d->rows;
  p.d = d->d_model;
  p.V = d->vocab;
  p.C = d->n_clusters;
  p.top = d->top_clusters;
  p.csize = pl.csize;
  p.sub = pl.sub;
  p.cstride = (p.C + 3) / 4 * 4;
  p.gs = topk_group_lanes(p.C, p.top);
  char* ws = (char*)workspace;
  p.scores = (float*)ws;
  p.kept = (int32_t*)(ws + pl.scores);
  p.part = (float*)(ws + pl.scores + pl.kept);
  p.part_bytes = (uint32_t)pl.part;
  p.cnt = (int32_t*)(ws + pl.scores + pl.kept + pl.part);
  p.stats = stats;
  p.clusters = clusters;
  p.out_tokens = out_tokens;
  p.out_stride = out_stride > 0 ? out_stride : 1;
  hipStream_t s = (hipStream_t)stream;
  p.splits = 0;
  if (cluster_scores_by_gemm(*d)) {
    RingPlan rp = ring_plan(2, d->rows, d->d_model, d->n_clusters, live_wg());
    const int S = split_count(rp, live_wg());
    if (S >= 1) {
      GemmParams g{};
      g.x = p.h;
      g.w = p.cent;
      g.R = p.R;
      g.K = p.d;
      g.N = p.C;
      g.nblk = rp.nblk;
      g.kch = rp.kch;
      g.y = p.scores;
      g.splits = S;
      rc = dispatch_ring<2, GM_SPLIT>(g, p.R, rp.nblk * S, s);
      if (rc != SV_OK) return rc;
      p.splits = S;
    }
  }
  if (p.splits == 0) {
    p.splits = 1;
    hipLaunchKernelGGL(cluster_score_kernel, dim3((p.C + 15) / 16, p.R), dim3(256), 0, s, p);
  }
  hipLaunchKernelGGL(cluster_topk_kernel, dim3(p.R), dim3(kTopkThreads), 0, s, p);
  hipLaunchKernelGGL(cluster_logits_kernel, dim3(pl.nslot, p.R), dim3(256), 0, s, p);
  return launch_status();
}

extern "C" size_t sv_lmhead_workspace(const sv_lmhead_desc* d) {
  if (validate_lmhead(d) != SV_OK) return 0;
  const int nrows = sel_rows(*d);
  if (d->dtype == SV_F32) return align_up((size_t)f32_grid(*d) * nrows * sizeof(SelPart), 256);
  const RingPlan pl = ring_plan(kSelT, nrows, d->d_model, d->vocab, kMaxWG);
  return pl.cnt_bytes + pl.part_bytes + align_up((size_t)kMaxWG * nrows * sizeof(SelPart), 256) +
         (d->mode == SV_SELECT_SAMPLE_RS ? align_up((size_t)kMaxWG * nrows * kRsCand * 16, 256) : 0);
}

static int lmhead_select(const sv_lmhead_desc* d, const void* hidden, const void* w, const int32_t* drafts,
                         const float* u_tok, const float* q_rows, sv_row_stats* stats, sv_accept_out* acc,
                         int32_t* out_tokens, uint32_t key0, uint32_t key1, sv_rs_cand* cands, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int rc = validate_lmhead(d);
  if (rc != SV_OK) return rc;
  if (d->mode == SV_SELECT_SAMPLE_RS && d->k > 0 && !cands) return SV_ERR_ARG;
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
  p.batch = d->batch;
  p.kdr = d->k;
  p.drafts = drafts;
  p.u_tok = u_tok;
  p.q_rows = q_rows;
  p.stats_in = stats;
  p.acc = acc;
  p.out_stride = d->out_stride > 0 ? d->out_stride : 1;
  p.rs_key0 = key0;
  p.rs_key1 = key1;
  p.rs_out = cands;
  const int nrows = sel_rows(*d);
  hipStream_t s = (hipStream_t)stream;
  int grid;

  if (d->dtype == SV_BF16) {
    const RingPlan pl = ring_plan(kSelT, nrows, d->d_model, d->vocab, live_wg());
    p.nblk = pl.nblk;
    p.kch = pl.kch;
    p.cnt = (int32_t*)workspace;
    p.part = (float*)((char*)workspace + pl.cnt_bytes);
    p.sel = (SelPart*)((char*)workspace + pl.cnt_bytes + pl.part_bytes);
    p.rs_part = (float*)((char*)workspace + pl.cnt_bytes + pl.part_bytes +
                         align_up((size_t)kMaxWG * nrows * sizeof(SelPart), 256));
    grid = pl.grid;
    switch (d->mode) {
      case SV_SELECT_GREEDY: rc = dispatch_ring<kSelT, GM_GREEDY>(p, nrows, grid, s); break;
      case SV_SELECT_SAMPLE: rc = dispatch_ring<kSelT, GM_SAMPLE>(p, nrows, grid, s); break;
      case SV_SELECT_SAMPLE_RS: rc = dispatch_ring<kSelT, GM_SAMPLE_RS>(p, nrows, grid, s); break;
      default: rc = dispatch_ring<kSelT, GM_RESIDUAL>(p, nrows, grid, s); break;
    }
    if (rc != SV_OK) return rc;
  } else {
    p.sel = (SelPart*)workspace;
    grid = f32_grid(*d);
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
    case SV_SELECT_SAMPLE_RS:
      hipLaunchKernelGGL(lmhead_merge_kernel<GM_SAMPLE_RS>, dim3(nrows), dim3(256), 0, s, p, grid, stats, out_tokens);
      break;
    default:
      hipLaunchKernelGGL(lmhead_merge_kernel<GM_RESIDUAL>, dim3(nrows), dim3(256), 0, s, p, grid, stats, out_tokens);
      break;
  }
  return launch_status();
}

extern "C" int sv_lmhead_select(const sv_lmhead_desc* d, const void* hidden, const void* w,
                                const int32_t* drafts, const float* u_tok, const float* q_rows,
                                sv_row_stats* stats, sv_accept_out* acc, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (d && d->mode == SV_SELECT_SAMPLE_RS) return SV_ERR_ARG;  // sv_lmhead_select_rs
  return lmhead_select(d, hidden, w, drafts, u_tok, q_rows, stats, acc, out_tokens, 0, 0, nullptr, workspace,
                       workspace_bytes, stream);
}

extern "C" int sv_lmhead_select_rs(const sv_lmhead_desc* d, const void* hidden, const void* w, const int32_t* drafts,
                                   const float* u_tok, uint32_t key0, uint32_t key1, sv_row_stats* stats,
                                   sv_rs_cand* cands, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!d || d->mode != SV_SELECT_SAMPLE_RS) return SV_ERR_ARG;
  return lmhead_select(d, hidden, w, drafts, u_tok, nullptr, stats, nullptr, out_tokens, key0, key1, cands,
                       workspace, workspace_bytes, stream);
}

extern "C" int32_t sv_linear_splits(const sv_linear_desc* d) {
  if (validate_linear(d) != SV_OK || d->epilogue != SV_EPI_SPLIT_F32) return 0;
  if (check_device() != SV_OK) return 0;
  return split_count(ring_plan(lin_tiles(*d), d->rows, d->in_features, d->out_features, live_wg()), live_wg());
}

extern "C" size_t sv_linear_workspace(const sv_linear_desc* d) {
  if (validate_linear(d) != SV_OK) return 0;
  if (d->dtype == SV_F32 || d->epilogue == SV_EPI_SPLIT_F32) return 0;
  const RingPlan pl = ring_plan(lin_tiles(*d), d->rows, d->in_features, d->out_features, kMaxWG);
  return pl.cnt_bytes + pl.part_bytes;
}

// The tiled copy holds every (block, chunk) tile of the ring plan whole: nblk * kch tiles
// of 64T rows x 128 bytes.  T comes from the descriptor (epilogue, K, N), never from the
// device, so the size is a property of the descriptor alone.
extern "C" size_t sv_linear_tiled_bytes(const sv_linear_desc* d) {
  if (validate_linear(d) != SV_OK || d->dtype != SV_BF16) return 0;
  const int T = lin_tiles(*d);
  const int64_t nblk = (d->out_features + 64 * T - 1) / (64 * T), kch = (d->in_features + 63) / 64;
  return (size_t)(nblk * kch * (64 * T) * 128);
}

extern "C" int sv_linear_tile_weights(const sv_linear_desc* d, const void* w, void* w_tiled, void* stream) {
  const int rc = validate_linear(d);
  if (rc != SV_OK) return rc;
  if (d->dtype != SV_BF16) return SV_ERR_ARG;
  if (!w || !w_tiled || ((uintptr_t)w & 15) || ((uintptr_t)w_tiled & 15)) return SV_ERR_ARG;
  const int drc = check_device();
  if (drc != SV_OK) return drc;
  const int T = lin_tiles(*d);
  const int kch = (d->in_features + 63) / 64;
  const int64_t units = (int64_t)sv_linear_tiled_bytes(d) / 16;
  hipLaunchKernelGGL(tile_weights_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)w, (uint16_t*)w_tiled, d->out_features, d->in_features, T, kch, units);
  return launch_status();
}

extern "C" int sv_linear(const sv_linear_desc* d, const void* x, const void* w, void* y,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_linear(d);
  if (rc != SV_OK) return rc;
  if (!x || !w || !y) return SV_ERR_ARG;
  if (d->w_layout == SV_W_TILED && ((uintptr_t)w & 15)) return SV_ERR_ARG;
  const size_t need = sv_linear_workspace(d);
  if (need && (!workspace || workspace_bytes < need)) return SV_ERR_WORKSPACE;
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
  RingPlan pl = ring_plan(lin_tiles(*d), d->rows, d->in_features, d->out_features, live_wg());
  GemmParams p{};
  if (d->epilogue == SV_EPI_SPLIT_F32) {
    p.splits = split_count(pl, live_wg());
    if (p.splits == 0) return SV_ERR_UNSUPPORTED;
    pl.grid = pl.nblk * p.splits;
  }
  p.x = x;
  p.w = (const uint16_t*)w;
  p.w_tiled = d->w_layout == SV_W_TILED;
  p.R = d->rows;
  p.K = d->in_features;
  p.N = d->out_features;
  p.nblk = pl.nblk;
  p.kch = pl.kch;
  p.y = y;
  p.cnt = (int32_t*)workspace;
  p.part = (float*)((char*)workspace + pl.cnt_bytes);
  if (d->act_pair) {
    // pair activations: x read as its hi and lo bf16 planes; STORE writes fp32 (act_pair
    // 1) or bf16 (act_pair 2), GEGLU a pair
    auto go = [&](auto tiles) {
      constexpr int T = decltype(tiles)::value;
      switch (d->epilogue) {
        case SV_EPI_GEGLU: return T == 1 ? (int)SV_ERR_UNSUPPORTED : dispatch_ring<T, GM_GEGLU, 1>(p, d->rows, pl.grid, s);
        case SV_EPI_SPLIT_F32: return dispatch_ring<T, GM_SPLIT, 1>(p, d->rows, pl.grid, s);
        case SV_EPI_STORE:
          return d->act_pair == 2 ? dispatch_ring<T, GM_STORE_BF16, 1>(p, d->rows, pl.grid, s)
                                  : dispatch_ring<T, GM_STORE_F32, 1>(p, d->rows, pl.grid, s);
        default: return dispatch_ring<T, GM_ADD_F32, 1>(p, d->rows, pl.grid, s);
      }
    };
    rc = pl.T == 1 ? go(std::integral_constant<int, 1>{})
                   : pl.T == 2 ? go(std::integral_constant<int, 2>{}) : go(std::integral_constant<int, 4>{});
    if (rc != SV_OK) return rc;
    return launch_status();
  }
  if (d->epilogue == SV_EPI_GEGLU)
    rc = dispatch_ring<2, GM_GEGLU>(p, d->rows, pl.grid, s);
  else if (d->epilogue == SV_EPI_SPLIT_F32)
    rc = pl.T == 1 ? dispatch_ring<1, GM_SPLIT>(p, d->rows, pl.grid, s) : dispatch_ring<2, GM_SPLIT>(p, d->rows, pl.grid, s);
  else if (pl.T == 1)
    rc = d->epilogue == SV_EPI_STORE ? dispatch_ring<1, GM_STORE_BF16>(p, d->rows, pl.grid, s)
                                     : dispatch_ring<1, GM_ADD_F32>(p, d->rows, pl.grid, s);
  else
    rc = d->epilogue == SV_EPI_STORE ? dispatch_ring<2, GM_STORE_BF16>(p, d->rows, pl.grid, s)
                                     : dispatch_ring<2, GM_ADD_F32>(p, d->rows, pl.grid, s);
  if (rc != SV_OK) return rc;
  return launch_status();
}
