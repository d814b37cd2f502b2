// attn.hip -- verify attention over a shared KV cache (CDNA4 / gfx950).
//
// One call = three stream-ordered kernels:
//   1. rope_append: rotates the queries (into the workspace) and the new keys at
//      their absolute positions and writes the new key / value rows into the
//      cache ("Gemma 4 拆解" (marsggbo), section 2: p-RoPE on global layers, the
//      value reuses the key; the cache is the one the drafter also reads,
//      section 4.2).
//   2. attn_mfma (bf16) or attn_f32: multi-query decode attention.  All
//      (k+1) x (Hq/Hkv) query rows of one sequence and KV head form one block of
//      rows that shares a single coalesced stream of that head's cache; the key
//      range of the whole batch is cut into equal pieces, one per workgroup, so
//      every CU streams the same number of bytes whatever the per-sequence
//      lengths (split-KV); each piece leaves an unnormalised partial (m, l, acc).
//   3. attn_merge: online-softmax combination of the partials of each
//      (sequence, KV head, row): O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
#include "sv_device.h"
#include "sv_host.h"

namespace sv {

struct AttnParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;          // == k_cache when keys are reused as values
  const int32_t* cache_len;
  void* out;
  void* q_rot;            // workspace: rotated queries [B, nq, Hq, D]
  float* part_acc;        // workspace: [slots][M][D]
  float* part_ml;         // workspace: [slots][M][2]  (m in log2 units, l)
  int32_t* dev_status;
  int64_t cap;
  int64_t q_stride, kv_stride;  // elements between consecutive (b, j) rows of q / k_new, v_new
  double log2_base;       // log2(rope_base)
  float scale_log2;       // softmax_scale * log2(e)
  float scale;
  int B, nq, Hq, Hkv, G, D, M;
  int window, rope_dims, n_new, qoff, k_is_v;
  int nwg;                // workgroups of the attention kernel
  int min_chunk;          // smallest key piece per workgroup
};

// ---------------------------------------------------------------------------
// key range of sequence b: union over its query rows of the visible keys
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool seq_ok(const AttnParams& p, int64_t L) {
  if (L < 0) return false;
  if (p.n_new > 0) return L + p.n_new <= p.cap;
  return L <= p.cap;
}

__device__ __forceinline__ void seq_range(const AttnParams& p, int b, int64_t& lo, int64_t& len) {
  const int64_t L = p.cache_len[b];
  lo = 0;
  len = 0;
  if (!seq_ok(p, L)) return;
  const int64_t pf = L + p.qoff;
  const int64_t pl = pf + p.nq - 1;
  const int64_t last = L + p.n_new - 1;
  const int64_t hi = (pl < last ? pl : last) + 1;
  int64_t l0 = 0;
  if (p.window > 0) {
    l0 = pf - p.window + 1;
    if (l0 < 0) l0 = 0;
  }
  lo = l0;
  len = hi > l0 ? hi - l0 : 0;
}

__device__ __forceinline__ int64_t total_keys(const AttnParams& p) {
  int64_t t = 0;
  for (int b = 0; b < p.B; ++b) {
    int64_t lo, len;
    seq_range(p, b, lo, len);
    t += len * p.Hkv;
  }
  return t;
}

// keys per workgroup piece (a multiple of 32)
__device__ __forceinline__ int64_t piece_chunk(const AttnParams& p, int64_t total) {
  int64_t c = (total + p.nwg - 1) / p.nwg;
  c = (c + 31) & ~int64_t(31);
  return c < p.min_chunk ? p.min_chunk : c;
}

// ---------------------------------------------------------------------------
// 1. RoPE + append
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ double ld_elem(const void* base, int64_t i) {
  if constexpr (sizeof(T) == 2) return (double)bf16_to_f32(((const uint16_t*)base)[i]);
  else return (double)((const float*)base)[i];
}
template <typename T>
__device__ __forceinline__ void st_elem(void* base, int64_t i, double v) {
  float f = __double2float_rn(v);
  if constexpr (sizeof(T) == 2) ((uint16_t*)base)[i] = (uint16_t)f32_to_bf16_bits(f);
  else ((float*)base)[i] = f;
}

// rotate-half RoPE of element d of a head vector x (pre-rotation values) at position pos
template <typename T>
__device__ __forceinline__ double rope_elem(const void* src, int64_t head_off, int d, int r,
                                            double log2_base, double pos) {
  const double x = ld_elem<T>(src, head_off + d);
  if (d >= r) return x;
  const int half = r >> 1;
  const int i = d < half ? d : d - half;
  const double theta = exp2(-(2.0 * (double)i / (double)r) * log2_base);
  double sn, cs;
  sincos(pos * theta, &sn, &cs);
  if (d < half) return x * cs - ld_elem<T>(src, head_off + d + half) * sn;
  return x * cs + ld_elem<T>(src, head_off + d - half) * sn;
}

template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(AttnParams p) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t L = p.cache_len[b];
  if (!seq_ok(p, L)) {
    if (threadIdx.x == 0 && j == 0) set_status(p.dev_status, L < 0 ? SV_DEV_BAD_LENGTH : SV_DEV_CACHE_OVERFLOW);
    return;
  }
  const int D = p.D;
  const double pos = (double)(L + p.qoff + j);
  const int nqe = p.Hq * D;
  const int nke = p.n_new > 0 ? p.Hkv * D : 0;
  const int nve = (p.n_new > 0 && !p.k_is_v) ? p.Hkv * D : 0;
  for (int e = threadIdx.x; e < nqe + nke + nve; e += blockDim.x) {
    if (e < nqe) {
      const int h = e / D, d = e % D;
      const int64_t src = ((int64_t)b * p.nq + j) * p.q_stride + (int64_t)h * D;
      const int64_t dst = (((int64_t)b * p.nq + j) * p.Hq + h) * D;
      st_elem<T>(p.q_rot, dst + d, rope_elem<T>(p.q, src, d, p.rope_dims, p.log2_base, pos));
    } else if (e < nqe + nke) {
      const int e2 = e - nqe, h = e2 / D, d = e2 % D;
      const int64_t src = ((int64_t)b * p.nq + j) * p.kv_stride + (int64_t)h * D;
      const int64_t dst = (((int64_t)b * p.Hkv + h) * p.cap + L + j) * D;
      st_elem<T>(p.k_cache, dst + d, rope_elem<T>(p.k_new, src, d, p.rope_dims, p.log2_base, pos));
    } else {
      const int e2 = e - nqe - nke, h = e2 / D, d = e2 % D;
      const int64_t src = ((int64_t)b * p.nq + j) * p.kv_stride + (int64_t)h * D;
      const int64_t dst = (((int64_t)b * p.Hkv + h) * p.cap + L + j) * D;
      st_elem<T>(p.v_cache, dst + d, ld_elem<T>(p.v_new, src + d));
    }
  }
}

// ---------------------------------------------------------------------------
// 2a. bf16 multi-query attention on MFMA
//
// Workgroup = 4 waves; wave w owns the dims [w*D/4, (w+1)*D/4) of the head.
// Per tile of 32 keys:
//   QK : each wave forms the partial scores S^T[key, row] over its dims with
//        16x16x32 MFMAs (A = key rows straight from HBM, B = rotated queries),
//        the four partials meet in LDS and every wave sums them in the same
//        order (one barrier per tile, double-buffered);
//   softmax: per row, running max m and sum l in log2 units; the row of a
//        lane is fixed (lane % 16) so the rescale of its accumulators is local;
//   PV : O^T[dim, row] += V^T[dim, key] P^T[key, row]; V^T comes from the
//        wave's own key/value registers transposed through a private LDS tile,
//        P^T straight from the score registers (same lane layout).
// ---------------------------------------------------------------------------
template <int D, int MT, bool KV_SAME>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnParams p) {
  constexpr int DS = D / 4;   // dims per wave
  constexpr int KS = DS / 32; // 32-dim k-steps of QK per wave
  constexpr int DT = DS / 16; // 16-dim output tiles of PV per wave
  constexpr int TK = 32;      // keys per tile
  constexpr int VTS = TK + 8; // bf16 per V^T row in LDS (16-byte aligned rows)
  static_assert(KS >= 1 && DT >= 1, "head_dim too small");

  __shared__ __attribute__((aligned(16))) float s_part[2][4][MT * 2][64 * 4];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[4][DS * VTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int M = p.M, G = p.G;

  const int64_t total = total_keys(p);
  if (total == 0) return;
  const int64_t chunk = piece_chunk(p, total);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= total) return;
  const int64_t end = start + chunk < total ? start + chunk : total;

  const uint16_t* qrot = (const uint16_t*)p.q_rot;
  const uint16_t* kc = (const uint16_t*)p.k_cache;
  const uint16_t* vcache = (const uint16_t*)p.v_cache;
  int buf = 0;

  int64_t seg_off = 0;
  for (int b = 0; b < p.B && seg_off < end; ++b) {
    int64_t lo, len;
    seq_range(p, b, lo, len);
    if (len == 0) continue;
    const int64_t L = p.cache_len[b];
    const int64_t last = L + p.n_new - 1;
    for (int kvh = 0; kvh < p.Hkv; ++kvh, seg_off += len) {
      const int64_t s0 = seg_off, s1 = seg_off + len;
      if (s1 <= start) continue;
      if (s0 >= end) break;
      const int64_t a0 = (start > s0 ? start : s0) - s0 + lo;  // first key of the piece
      const int64_t a1 = (end < s1 ? end : s1) - s0 + lo;      // one past its last key
      const int slot = blockIdx.x + b * p.Hkv + kvh;

      // ---- queries of this (sequence, kv head) as MFMA B operands
      V16 qreg[MT][KS];
      int64_t row_hi[MT], row_lo[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        if (r < M) {
          const int j = r / G, hg = r - (r / G) * G;
          const uint16_t* src = qrot + (((int64_t)b * p.nq + j) * p.Hq + kvh * G + hg) * D + wave * DS + lg * 8;
#pragma unroll
          for (int s = 0; s < KS; ++s) qreg[mt][s].u = *(const uint4*)(src + s * 32);
          const int64_t pos = L + p.qoff + j;
          row_hi[mt] = pos < last ? pos : last;
          row_lo[mt] = p.window > 0 ? pos - p.window + 1 : 0;
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s) qreg[mt][s].u = make_uint4(0, 0, 0, 0);
          row_hi[mt] = INT64_MAX;  // padded rows: no causal limit (results discarded)
          row_lo[mt] = INT64_MIN;
        }
      }

      f32x4_t O[DT][MT];
      float m_run[MT], l_run[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = kNegInf;
        l_run[mt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

      const int64_t head_base = ((int64_t)b * p.Hkv + kvh) * p.cap * D + wave * DS + lg * 8;
      auto load_tile = [&](int64_t t0, V16 (&kr)[2][KS], V16 (&vr)[2][KS]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int64_t key = t0 + kt * 16 + lr;
          const bool ok = key < a1;
          const int64_t off = head_base + key * D;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            kr[kt][s].u = ok ? *(const uint4*)(kc + off + s * 32) : make_uint4(0, 0, 0, 0);
            if constexpr (!KV_SAME)
              vr[kt][s].u = ok ? *(const uint4*)(vcache + off + s * 32) : make_uint4(0, 0, 0, 0);
          }
        }
      };

      V16 kcur[2][KS], vcur[2][KS], knext[2][KS], vnext[2][KS];
      load_tile(a0, kcur, vcur);

      for (int64_t t0 = a0; t0 < a1; t0 += TK) {
        // ---- partial scores over this wave's dims
        f32x4_t sp[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = mfma16x16x32(kcur[kt][s].b, qreg[mt][s].b, acc);
            sp[mt][kt] = acc;
          }
        float* myp = &s_part[buf][wave][0][0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) *(f32x4_t*)(myp + ((mt * 2 + kt) * 64 + lane) * 4) = sp[mt][kt];

        // ---- this wave's values, transposed into its private LDS tile:
        // key 16*kt + lr goes to column 8*(lr/4) + 2*(lr%4) + kt of row `dim`
        {
          uint16_t* vt = s_vt[wave];
          const int col = 8 * (lr >> 2) + 2 * (lr & 3);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const V16& v0 = KV_SAME ? kcur[0][s] : vcur[0][s];
            const V16& v1 = KV_SAME ? kcur[1][s] : vcur[1][s];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t w0 = v0.w[e >> 1], w1 = v1.w[e >> 1];
              const uint32_t h0 = (e & 1) ? (w0 >> 16) : (w0 & 0xffffu);
              const uint32_t h1 = (e & 1) ? (w1 >> 16) : (w1 & 0xffffu);
              const int dim = s * 32 + lg * 8 + e;
              *(uint32_t*)(vt + dim * VTS + col) = h0 | (h1 << 16);
            }
          }
        }

        // ---- prefetch the next tile
        const bool more = t0 + TK < a1;
        if (more) load_tile(t0 + TK, knext, vnext);

        __syncthreads();

        // ---- full scores, softmax update, P operands
        V16 preg[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          float sc[2][4];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            f32x4_t a = *(const f32x4_t*)(&s_part[buf][0][mt * 2 + kt][lane * 4]);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
              const f32x4_t o = *(const f32x4_t*)(&s_part[buf][w][mt * 2 + kt][lane * 4]);
              a[0] += o[0]; a[1] += o[1]; a[2] += o[2]; a[3] += o[3];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t key = t0 + kt * 16 + lg * 4 + i;
              const bool vis = key < a1 && key <= row_hi[mt] && key >= row_lo[mt];
              sc[kt][i] = vis ? a[i] * p.scale_log2 : kNegInf;
            }
          }
          float mx = kNegInf;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kt][i]);
          mx = fmaxf(mx, shfl_xor_f(mx, 16));
          mx = fmaxf(mx, shfl_xor_f(mx, 32));
          const float m_new = fmaxf(m_run[mt], mx);
          float alpha = 1.f;
          float pv[2][4];
          if (m_new == kNegInf) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) pv[kt][i] = 0.f;
          } else {
            alpha = exp2f(m_run[mt] - m_new);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) pv[kt][i] = round_bf16(exp2f(sc[kt][i] - m_new));
          }
          float rs = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) rs += pv[kt][i];
          rs += shfl_xor_f(rs, 16);
          rs += shfl_xor_f(rs, 32);
          l_run[mt] = l_run[mt] * alpha + rs;
          m_run[mt] = m_new;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            O[dt][mt][0] *= alpha; O[dt][mt][1] *= alpha;
            O[dt][mt][2] *= alpha; O[dt][mt][3] *= alpha;
          }
          // slot 2*i + kt of lane group lg holds key 16*kt + 4*lg + i
#pragma unroll
          for (int i = 0; i < 4; ++i) preg[mt].w[i] = pack_bf16x2(pv[0][i], pv[1][i]);
        }

        // ---- O^T += V^T P^T
        {
          const uint16_t* vt = s_vt[wave];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            V16 a;
            a.u = *(const uint4*)(vt + (dt * 16 + lr) * VTS + lg * 8);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) O[dt][mt] = mfma16x16x32(a.b, preg[mt].b, O[dt][mt]);
          }
        }

        buf ^= 1;
        if (more) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              kcur[kt][s] = knext[kt][s];
              if constexpr (!KV_SAME) vcur[kt][s] = vnext[kt][s];
            }
        }
      }

      // ---- unnormalised partial of this piece
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        if (r < M) {
          float* dst = p.part_acc + ((int64_t)slot * M + r) * D + wave * DS + lg * 4;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(dst + dt * 16) = O[dt][mt];
          if (wave == 0 && lg == 0) {
            p.part_ml[((int64_t)slot * M + r) * 2 + 0] = m_run[mt];
            p.part_ml[((int64_t)slot * M + r) * 2 + 1] = l_run[mt];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. fp32 attention (small caches; one workgroup per query row and head)
// ---------------------------------------------------------------------------
constexpr int kF32MaxKeys = 4096;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnParams p) {
  __shared__ float s_q[512];
  __shared__ float s_w[kF32MaxKeys];
  __shared__ float s_red[256];
  const int h = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int64_t L = p.cache_len[b];
  if (!seq_ok(p, L)) return;
  const int D = p.D, kvh = h / p.G, tid = threadIdx.x;
  const float* qrot = (const float*)p.q_rot;
  const float* kcache = (const float*)p.k_cache;
  const float* vcache = (const float*)p.v_cache;
  float* out = (float*)p.out + (((int64_t)b * p.nq + j) * p.Hq + h) * D;
  for (int d = tid; d < D; d += blockDim.x) s_q[d] = qrot[(((int64_t)b * p.nq + j) * p.Hq + h) * D + d];
  const int64_t pos = L + p.qoff + j, last = L + p.n_new - 1;
  const int64_t hi = pos < last ? pos : last;
  int64_t lo = 0;
  if (p.window > 0 && pos - p.window + 1 > 0) lo = pos - p.window + 1;
  const int n = hi >= lo ? (int)(hi - lo + 1) : 0;
  __syncthreads();
  if (n == 0) {
    for (int d = tid; d < D; d += blockDim.x) out[d] = 0.f;
    return;
  }
  const int64_t base = ((int64_t)b * p.Hkv + kvh) * p.cap;
  float mx = kNegInf;
  for (int t = tid; t < n; t += blockDim.x) {
    const float* kr = kcache + (base + lo + t) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(s_q[d], kr[d], acc);
    acc *= p.scale;
    s_w[t] = acc;
    mx = fmaxf(mx, acc);
  }
  s_red[tid] = mx;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) s_red[tid] = fmaxf(s_red[tid], s_red[tid + st]);
    __syncthreads();
  }
  mx = s_red[0];
  __syncthreads();
  float sum = 0.f;
  for (int t = tid; t < n; t += blockDim.x) {
    const float e = expf(s_w[t] - mx);
    s_w[t] = e;
    sum += e;
  }
  s_red[tid] = sum;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) s_red[tid] += s_red[tid + st];
    __syncthreads();
  }
  const float inv = 1.f / s_red[0];
  for (int d = tid; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int t = 0; t < n; ++t) acc = fmaf(s_w[t], vcache[(base + lo + t) * D + d], acc);
    out[d] = acc * inv;
  }
}

// ---------------------------------------------------------------------------
// 3. merge of the split-KV partials (bf16 path)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnParams p) {
  const int r = blockIdx.x;          // row within the (sequence, kv head) block
  const int seg = blockIdx.y;        // b * Hkv + kvh
  const int b = seg / p.Hkv, kvh = seg % p.Hkv;
  const int64_t L = p.cache_len[b];
  if (!seq_ok(p, L)) return;
  const int64_t total = total_keys(p);
  const int64_t chunk = piece_chunk(p, total);
  int64_t off = 0, lo = 0, len = 0;
  for (int bb = 0; bb <= b; ++bb) {
    seq_range(p, bb, lo, len);
    if (bb < b) off += len * p.Hkv;
  }
  off += (int64_t)kvh * len;
  const int D = p.D, G = p.G;
  const int j = r / G, hg = r % G;
  uint16_t* out = (uint16_t*)p.out + (((int64_t)b * p.nq + j) * p.Hq + kvh * G + hg) * D;
  const int d0 = threadIdx.x * 4;
  if (d0 >= D) return;
  if (len == 0) {
    *(uint2*)(out + d0) = make_uint2(0, 0);
    return;
  }
  const int64_t w0 = off / chunk, w1 = (off + len - 1) / chunk;
  float Mx = kNegInf;
  for (int64_t w = w0; w <= w1; ++w) Mx = fmaxf(Mx, p.part_ml[((w + seg) * p.M + r) * 2]);
  float l = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (Mx != kNegInf) {
    for (int64_t w = w0; w <= w1; ++w) {
      const int64_t slot = w + seg;
      const float m = p.part_ml[(slot * p.M + r) * 2];
      if (m == kNegInf) continue;
      const float f = exp2f(m - Mx);
      l += f * p.part_ml[(slot * p.M + r) * 2 + 1];
      const f32x4_t v = *(const f32x4_t*)(p.part_acc + (slot * p.M + r) * D + d0);
      a0 += f * v[0]; a1 += f * v[1]; a2 += f * v[2]; a3 += f * v[3];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  *(uint2*)(out + d0) = make_uint2(pack_bf16x2(a0 * inv, a1 * inv), pack_bf16x2(a2 * inv, a3 * inv));
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int kAttnNwgMax = 2048;

struct AttnPlan {
  size_t q_rot_bytes, acc_bytes, ml_bytes, total;
  int M, slots;
};

static AttnPlan attn_plan(const sv_attn_desc& d) {
  AttnPlan pl{};
  const size_t elt = d.dtype == SV_BF16 ? 2 : 4;
  pl.M = (d.n_heads_q / d.n_heads_kv) * d.n_q;
  pl.q_rot_bytes = align_up((size_t)d.batch * d.n_q * d.n_heads_q * d.head_dim * elt, 256);
  if (d.dtype == SV_BF16) {
    pl.slots = kAttnNwgMax + d.batch * d.n_heads_kv;
    pl.acc_bytes = align_up((size_t)pl.slots * pl.M * d.head_dim * 4, 256);
    pl.ml_bytes = align_up((size_t)pl.slots * pl.M * 2 * 4, 256);
  }
  pl.total = pl.q_rot_bytes + pl.acc_bytes + pl.ml_bytes;
  return pl;
}

static int validate_attn(const sv_attn_desc* d) {
  if (!d) return SV_ERR_ARG;
  if (d->batch <= 0 || d->n_q <= 0 || d->n_heads_q <= 0 || d->n_heads_kv <= 0) return SV_ERR_ARG;
  if (d->n_heads_q % d->n_heads_kv) return SV_ERR_ARG;
  if (d->head_dim <= 0 || d->head_dim % 8) return SV_ERR_ARG;
  if (d->window < 0 || d->rope_dims < 0 || d->rope_dims > d->head_dim || (d->rope_dims & 1)) return SV_ERR_ARG;
  if (d->k_is_v != 0 && d->k_is_v != 1) return SV_ERR_ARG;
  if (d->append != 0 && d->append != 1) return SV_ERR_ARG;
  if (d->append && d->q_pos_offset != 0) return SV_ERR_ARG;
  if (d->reserved != 0 || d->reserved_f != 0.f) return SV_ERR_ARG;
  if (d->cache_capacity <= 0) return SV_ERR_ARG;
  if (d->q_row_stride < 0 || d->kv_row_stride < 0) return SV_ERR_ARG;
  if (d->q_row_stride && d->q_row_stride < (int64_t)d->n_heads_q * d->head_dim) return SV_ERR_ARG;
  if (d->kv_row_stride && d->kv_row_stride < (int64_t)d->n_heads_kv * d->head_dim) return SV_ERR_ARG;
  if (d->rope_dims > 0 && !(d->rope_base > 1.0)) return SV_ERR_ARG;
  if (!(d->softmax_scale > 0.f)) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->head_dim != 128 && d->head_dim != 256 && d->head_dim != 512) return SV_ERR_UNSUPPORTED;
    if ((d->n_heads_q / d->n_heads_kv) * d->n_q > 64) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if (d->head_dim > 512) return SV_ERR_UNSUPPORTED;
    if (d->cache_capacity > kF32MaxKeys) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  if ((int64_t)d->batch * d->n_q * d->n_heads_q > (int64_t)1 << 24) return SV_ERR_UNSUPPORTED;
  return SV_OK;
}

template <int D, int MT, bool KVS>
static void launch_mfma(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, MT, KVS>), dim3(p.nwg), dim3(256), 0, s, p);
}

template <int D>
static int dispatch_mfma(const AttnParams& p, int MT, bool kvs, hipStream_t s) {
  switch (MT) {
    case 1: kvs ? launch_mfma<D, 1, true>(p, s) : launch_mfma<D, 1, false>(p, s); break;
    case 2: kvs ? launch_mfma<D, 2, true>(p, s) : launch_mfma<D, 2, false>(p, s); break;
    case 3: kvs ? launch_mfma<D, 3, true>(p, s) : launch_mfma<D, 3, false>(p, s); break;
    case 4: kvs ? launch_mfma<D, 4, true>(p, s) : launch_mfma<D, 4, false>(p, s); break;
    default: return SV_ERR_UNSUPPORTED;
  }
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_verify_attn_workspace(const sv_attn_desc* d) {
  if (validate_attn(d) != SV_OK) return 0;
  return attn_plan(*d).total;
}

extern "C" int sv_verify_attn(const sv_attn_desc* d, const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* cache_len, void* out, void* workspace,
                              size_t workspace_bytes, int32_t* dev_status, void* stream) {
  int rc = validate_attn(d);
  if (rc != SV_OK) return rc;
  if (!q || !k_cache || !cache_len || !out) return SV_ERR_ARG;
  if (d->append && !k_new) return SV_ERR_ARG;
  if (!d->append && (k_new || v_new)) return SV_ERR_ARG;
  if (d->k_is_v && (v_cache || v_new)) return SV_ERR_ARG;
  if (!d->k_is_v && !v_cache) return SV_ERR_ARG;
  if (!d->k_is_v && d->append && !v_new) return SV_ERR_ARG;
  const AttnPlan pl = attn_plan(*d);
  if (!workspace || workspace_bytes < pl.total) return SV_ERR_WORKSPACE;
  rc = check_device();
  if (rc != SV_OK) return rc;

  AttnParams p{};
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = d->k_is_v ? k_cache : v_cache;
  p.cache_len = cache_len;
  p.out = out;
  char* ws = (char*)workspace;
  p.q_rot = ws;
  p.part_acc = (float*)(ws + pl.q_rot_bytes);
  p.part_ml = (float*)(ws + pl.q_rot_bytes + pl.acc_bytes);
  p.dev_status = dev_status;
  p.cap = d->cache_capacity;
  p.q_stride = d->q_row_stride ? d->q_row_stride : (int64_t)d->n_heads_q * d->head_dim;
  p.kv_stride = d->kv_row_stride ? d->kv_row_stride : (int64_t)d->n_heads_kv * d->head_dim;
  p.log2_base = d->rope_dims > 0 ? std::log2(d->rope_base) : 0.0;
  p.scale = d->softmax_scale;
  p.scale_log2 = d->softmax_scale * kLog2e;
  p.B = d->batch;
  p.nq = d->n_q;
  p.Hq = d->n_heads_q;
  p.Hkv = d->n_heads_kv;
  p.G = d->n_heads_q / d->n_heads_kv;
  p.D = d->head_dim;
  p.M = pl.M;
  p.window = d->window;
  p.rope_dims = d->rope_dims;
  p.n_new = d->append ? d->n_q : 0;
  p.qoff = d->q_pos_offset;
  p.k_is_v = d->k_is_v;
  p.nwg = 512;
  p.min_chunk = 64;

  hipStream_t s = (hipStream_t)stream;
  if (d->dtype == SV_BF16) {
    hipLaunchKernelGGL(rope_append_kernel<uint16_t>, dim3(d->n_q, d->batch), dim3(256), 0, s, p);
    const int MT = (pl.M + 15) / 16;
    switch (d->head_dim) {
      case 128: rc = dispatch_mfma<128>(p, MT, d->k_is_v, s); break;
      case 256: rc = dispatch_mfma<256>(p, MT, d->k_is_v, s); break;
      case 512: rc = dispatch_mfma<512>(p, MT, d->k_is_v, s); break;
      default: rc = SV_ERR_UNSUPPORTED;
    }
    if (rc != SV_OK) return rc;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(pl.M, d->batch * d->n_heads_kv), dim3(d->head_dim / 4),
                       0, s, p);
  } else {
    hipLaunchKernelGGL(rope_append_kernel<float>, dim3(d->n_q, d->batch), dim3(256), 0, s, p);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(d->n_heads_q, d->n_q, d->batch), dim3(256), 0, s, p);
  }
  return launch_status();
}
