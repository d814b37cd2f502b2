// attn.hip -- verify attention over a shared KV cache (CDNA4 / gfx950).
//
// One call = two stream-ordered kernels:
//   1. rope_append: rotates the queries (into the workspace) and the new keys at
//      their absolute positions and writes the new key / value rows into the
//      cache ("Gemma 4 拆解" (marsggbo), section 2: p-RoPE on global layers, the
//      value reuses the key; the cache is the one the drafter also reads,
//      section 4.2).  It also zeroes the per-segment arrival counters and the
//      output rows of sequences that have no visible keys.
//   2. attn_mfma (bf16) or attn_f32: multi-query decode attention.  All
//      (k+1) x (Hq/Hkv) query rows of one sequence and KV head form one block of
//      rows that shares a single coalesced stream of that head's cache; each such
//      segment of keys is cut into tile-aligned pieces, about equal across the
//      batch, one per workgroup (split-KV).  Each piece leaves an unnormalised
//      partial (m, l, acc), combined by online softmax:
//      O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s -- for a small block of
//      rows by the last piece of the segment to finish, otherwise by
//   3. attn_merge, one workgroup per (sequence, KV head, row).
#include "sv_device.h"
#include "sv_host.h"

#include <atomic>
#include <mutex>
#include <type_traits>

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
  int32_t* seg_cnt;       // workspace: [B * Hkv] arrivals of a segment's pieces
  int32_t* plan;          // workspace: the work split {chunk, pieces}, set by rope_append
  int in_splits;          // > 0: q, k_new, v_new are fp32 K-split partial products
  int act_pair;           // pair activations: q, k_new, v_new read as fp32 (no bf16 rounding
                          // before RoPE / the cache store), out written as a bf16 pair
  int64_t out_plane;      // pair activations: elements between out's hi and lo planes
  int fp8;                // caches hold fp8 E4M3 codes seen through per-channel scales
  const float* k_scale;   // fp8: [Hkv, D] scales of the key cache (also the values when K = V)
  const float* v_scale;   // fp8: [Hkv, D] scales of the value cache
  int part_acc_bytes, part_ml_bytes;
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

__device__ __forceinline__ void seq_range_of(const AttnParams& p, int64_t L, int64_t& lo, int64_t& len) {
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
__device__ __forceinline__ void seq_range(const AttnParams& p, int b, int64_t& lo, int64_t& len) {
  seq_range_of(p, p.cache_len[b], lo, len);
}

// Work split: each (sequence, kv head) segment of keys is cut into pieces of
// `chunk` keys (a multiple of the 64-key tile; the last piece of a segment may be
// shorter), one workgroup per piece.  chunk is the smallest such size for which the
// pieces number at most nwg (or one piece per segment when there are at least nwg
// segments), so no workgroup's keys cross a segment boundary.  Every workgroup and
// the merge derive the same plan from the cache lengths.
// The plan (chunk, piece count) is computed once per call by the first wave of
// rope_append_kernel and left in the workspace; a workgroup then only locates its
// piece.  Both run wave-parallel over the batch: lane l holds the key counts of
// sequences l, l + 64, ... (up to kPlanGroups * 64 of them, key counts below 2^31)
// and sums or scans them with cross-lane shuffles.  All 64 lanes must be active.
constexpr int kPlanGroups = 4;  // batch up to 256
struct Pieces {
  int chunk;
  int n;
};
struct BatchLens {
  int len[kPlanGroups];  // key count of sequence lane + 64 g (0 past the batch)
  int L[kPlanGroups];    // its committed length
};

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}
__device__ __forceinline__ int ceil_div_u(int n, int d) { return (int)(((unsigned)n + (unsigned)d - 1u) / (unsigned)d); }

__device__ __forceinline__ BatchLens batch_lens(const AttnParams& p) {
  const int lane = threadIdx.x & 63;
  BatchLens bl;
#pragma unroll
  for (int g = 0; g < kPlanGroups; ++g) {
    const int b = lane + 64 * g;
    int64_t lo = 0, len = 0;
    const int L = b < p.B ? p.cache_len[b] : 0;
    if (b < p.B) seq_range_of(p, L, lo, len);
    bl.len[g] = (int)len;
    bl.L[g] = L;
  }
  return bl;
}

__device__ __forceinline__ int pieces_at(const AttnParams& p, const BatchLens& bl, int c) {
  int n = 0;
#pragma unroll
  for (int g = 0; g < kPlanGroups; ++g) n += ceil_div_u(bl.len[g], c);
  return wave_sum_i(n) * p.Hkv;
}

__device__ __forceinline__ Pieces piece_plan(const AttnParams& p, const BatchLens& bl) {
  // per-lane partial sums stay far below 2^31 before the cross-lane sums; the four
  // reductions share their shuffle steps so their latencies overlap
  int64_t tl = 0;
  int nseg = 0, maxlen = 0;
#pragma unroll
  for (int g = 0; g < kPlanGroups; ++g) {
    tl += bl.len[g];
    nseg += bl.len[g] > 0 ? 1 : 0;
    maxlen = max(maxlen, bl.len[g]);
  }
  int lo32 = (int)(tl & 0xffff), hi32 = (int)(tl >> 16);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const int a = __shfl_xor(lo32, m, 64), b = __shfl_xor(hi32, m, 64);
    const int c = __shfl_xor(nseg, m, 64), d = __shfl_xor(maxlen, m, 64);
    lo32 += a;
    hi32 += b;
    nseg += c;
    maxlen = max(maxlen, d);
  }
  const int64_t total = (((int64_t)hi32 << 16) + lo32) * p.Hkv;
  nseg *= p.Hkv;
  if (total == 0) return {64, 0};
  auto up64 = [](int64_t x) { return (int)((x + 63) & ~int64_t(63)); };
  int c = up64((total + p.nwg - 1) / p.nwg);
  if (c < p.min_chunk) c = p.min_chunk;
  int n = pieces_at(p, bl, c);
  if (n > p.nwg) {
    if (nseg >= p.nwg) {
      c = up64(maxlen);
    } else {
      // sum of ceil(len / c) <= total / c + nseg, so this size is small enough
      int hi = up64((total + (p.nwg - nseg) - 1) / (p.nwg - nseg));
      int lo = c;  // too small
      while (hi - lo > 64) {
        const int mid = ((lo + hi) / 2) & ~63;
        const int m = mid <= lo ? lo + 64 : mid;
        if (pieces_at(p, bl, m) <= p.nwg) hi = m; else lo = m;
      }
      c = hi;
    }
    n = pieces_at(p, bl, c);
  }
  return {c, n};
}

// piece q -> sequence b, kv head kvh, its keys [a0, a1), and the pieces of its
// segment [first, first + count)
__device__ __forceinline__ void piece_locate(const AttnParams& p, const BatchLens& bl, int chunk, int q, int& b,
                                             int& kvh, int64_t& a0, int64_t& a1, int& first, int& count,
                                             int64_t& Lb) {
  const int lane = threadIdx.x & 63;
  int base = 0;  // pieces of the sequences before this group
  b = -1;
#pragma unroll
  for (int g = 0; g < kPlanGroups; ++g) {
    const int cnt = ceil_div_u(bl.len[g], chunk) * p.Hkv;
    const int incl = base + wave_incl_scan_i(cnt, lane);
    const uint64_t hit = __ballot(q < incl && q >= incl - cnt);
    if (b < 0 && hit) {
      const int l = __builtin_ctzll(hit);
      b = l + 64 * g;
      const int excl = __shfl(incl, l, 64) - __shfl(cnt, l, 64);
      const int nb = __shfl(cnt, l, 64) / p.Hkv;
      const int rem = q - excl;
      kvh = rem / nb;
      const int pi = rem - kvh * nb;
      int64_t lo, len;
      Lb = __shfl(bl.L[g], l, 64);  // the committed length, without reloading it
      seq_range_of(p, Lb, lo, len);
      a0 = lo + (int64_t)pi * chunk;
      a1 = lo + ((int64_t)(pi + 1) * chunk < len ? (int64_t)(pi + 1) * chunk : len);
      first = q - pi;
      count = nb;
    }
    base = __shfl(incl, 63, 64);
  }
  if (b < 0) {  // not reached for q below the piece count
    b = 0;
    kvh = 0;
    a0 = a1 = 0;
    first = q;
    count = 1;
    Lb = 0;
  }
}

// first piece and piece count of segment (b, kvh)
__device__ __forceinline__ void segment_pieces(const AttnParams& p, const BatchLens& bl, int chunk, int b, int kvh,
                                               int& first, int& count) {
  const int lane = threadIdx.x & 63;
  int before = 0, nb = 0;
#pragma unroll
  for (int g = 0; g < kPlanGroups; ++g) {
    const int bb = lane + 64 * g;
    const int c = ceil_div_u(bl.len[g], chunk);
    if (bb < b) before += c;
    if (bb == b) nb = c;
  }
  before = wave_sum_i(before) * p.Hkv;
  nb = wave_sum_i(nb);
  first = before + kvh * nb;
  count = nb;
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

// An input tensor (q, k_new or v_new): values in T, or (splits > 0, bf16 only) the
// fp32 K-split partial products of a projection, `splits` slices `slice` elements
// apart, summed in slice order and rounded to bf16 -- the value the projection would
// have stored.  With f32 (fp32 activations) the values are fp32 (the split sum is
// used as it is).
struct InView {
  const void* base;
  int64_t slice;
  int splits;
  int f32;
};

template <typename T>
__device__ __forceinline__ double ld_in(const InView& v, int64_t i) {
  if (v.splits == 0) return v.f32 ? ld_elem<float>(v.base, i) : ld_elem<T>(v.base, i);
  const float* f = (const float*)v.base + i;
  float a = 0.f;
  for (int s = 0; s < v.splits; ++s) a += f[(int64_t)s * v.slice];
  if (v.f32) return (double)a;
  return (double)bf16_to_f32((uint16_t)f32_to_bf16_bits(a));
}

// four consecutive output elements: bf16, or with pair activations the bf16 pair
// hi = bf16(a), lo = bf16(a - hi) in two planes
__device__ __forceinline__ void st_out4(const AttnParams& p, int64_t i, float a0, float a1, float a2, float a3) {
  const uint32_t h01 = pack_bf16x2(a0, a1), h23 = pack_bf16x2(a2, a3);
  *(uint2*)((uint16_t*)p.out + i) = make_uint2(h01, h23);
  if (p.act_pair)
    *(uint2*)((uint16_t*)p.out + p.out_plane + i) =
        make_uint2(pack_bf16x2(a0 - bf16_lo(h01), a1 - bf16_hi(h01)), pack_bf16x2(a2 - bf16_lo(h23), a3 - bf16_hi(h23)));
}

// rotate-half RoPE of element d of a head vector x (pre-rotation values) at position pos
template <typename T>
__device__ __forceinline__ double rope_elem(const InView& src, int64_t head_off, int d, int r,
                                            double log2_base, double pos) {
  const double x = ld_in<T>(src, head_off + d);
  if (d >= r) return x;
  const int half = r >> 1;
  const int i = d < half ? d : d - half;
  // angle in fp64 (positions reach ~1e5 rad), reduced to [-pi, pi] before the fp32 sincos
  const double theta = exp2(-(2.0 * (double)i / (double)r) * log2_base);
  const double ang = pos * theta;
  const double two_pi = 6.283185307179586476925286766559;
  const float red = (float)(ang - two_pi * rint(ang / two_pi));
  float snf, csf;
  sincosf(red, &snf, &csf);
  const double sn = snf, cs = csf;
  if (d < half) return x * cs - ld_in<T>(src, head_off + d + half) * sn;
  return x * cs + ld_in<T>(src, head_off + d - half) * sn;
}

// fp8 E4M3 code of a finite fp32 value: round to nearest with ties to even, values
// beyond +-448 (the largest finite E4M3 magnitude) saturating; NaN gives 0x7F.
// The quotient by the binade's quantum (2^(e-3), or 2^-9 below 2^-6) is exact, so
// rintf does the rounding; a value that rounds up to the next binade gets its code.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a > 448.f) return sign | 0x7Eu;
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  if (e < -6) e = -6;
  const float v = ldexpf(rintf(ldexpf(a, 3 - e)), e - 3);   // <= 448: 448 is on every grid above
  if (v < 0.015625f) return sign | (uint32_t)ldexpf(v, 9);  // subnormal: m 2^-9
  const uint32_t u = __float_as_uint(v);
  return sign | ((((u >> 23) & 0xFFu) - 120u) << 3) | ((u >> 20) & 7u);  // exponent bias 127 -> 7
}

// an appended cache element: bf16 rounding as in a bf16 cache, then (fp8) the code
// of value / scale, the quotient correctly rounded in fp32
__device__ __forceinline__ void st_cache(const AttnParams& p, void* base, const float* scale, int64_t i, int sidx,
                                         double v) {
  const uint32_t bits = f32_to_bf16_bits(__double2float_rn(v));
  if (!p.fp8) {
    ((uint16_t*)base)[i] = (uint16_t)bits;
    return;
  }
  ((uint8_t*)base)[i] = (uint8_t)e4m3_code(__fdiv_rn(bf16_to_f32((uint16_t)bits), scale[sidx]));
}

// one workgroup per (sequence, row, head); one thread per element of the head
template <typename T>
__global__ __launch_bounds__(512) void rope_append_kernel(AttnParams p) {
  const int b = blockIdx.x / p.nq, j = blockIdx.x % p.nq;
  const int hs = blockIdx.y;  // [0, Hq): query head, then key heads, then value heads
  const int d = threadIdx.x;
  if constexpr (sizeof(T) == 2) {
    // the attention kernel counts each segment's finished pieces from zero and reads
    // the work split computed here once (the first wave of block (0, 0); all 64
    // lanes take part in the plan's cross-lane sums)
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      for (int i = d; i < p.B * p.Hkv; i += blockDim.x) p.seg_cnt[i] = 0;
      if (d < 64) {
        const BatchLens bl = batch_lens(p);
        const Pieces pc = piece_plan(p, bl);
        if (d == 0) {
          p.plan[0] = pc.chunk;
          p.plan[1] = pc.n;
        }
      }
    }
    // a sequence without visible keys has no pieces: its output rows are zero (a
    // skipped sequence's rows are left untouched)
    if (hs < p.Hq && d < p.D && seq_ok(p, p.cache_len[b])) {
      int64_t lo, len;
      seq_range(p, b, lo, len);
      if (len == 0) {
        const int64_t oi = (((int64_t)b * p.nq + j) * p.Hq + hs) * p.D + d;
        ((uint16_t*)p.out)[oi] = 0;
        if (p.act_pair) ((uint16_t*)p.out)[p.out_plane + oi] = 0;
      }
    }
  }
  const int64_t L = p.cache_len[b];
  if (!seq_ok(p, L)) {
    if (d == 0 && j == 0 && hs == 0) set_status(p.dev_status, L < 0 ? SV_DEV_BAD_LENGTH : SV_DEV_CACHE_OVERFLOW);
    return;
  }
  const int D = p.D;
  if (d >= D) return;
  const double pos = (double)(L + p.qoff + j);
  if (hs < p.Hq) {
    const int64_t src = ((int64_t)b * p.nq + j) * p.q_stride + (int64_t)hs * D;
    const int64_t dst = (((int64_t)b * p.nq + j) * p.Hq + hs) * D;
    const InView qv{p.q, (int64_t)p.B * p.nq * p.q_stride, p.in_splits, p.act_pair};
    st_elem<T>(p.q_rot, dst + d, rope_elem<T>(qv, src, d, p.rope_dims, p.log2_base, pos));
  } else if (hs < p.Hq + p.Hkv) {
    const int h = hs - p.Hq;
    const int64_t src = ((int64_t)b * p.nq + j) * p.kv_stride + (int64_t)h * D;
    const int64_t dst = (((int64_t)b * p.Hkv + h) * p.cap + L + j) * D;
    const InView kv{p.k_new, (int64_t)p.B * p.nq * p.kv_stride, p.in_splits, p.act_pair};
    const double kr = rope_elem<T>(kv, src, d, p.rope_dims, p.log2_base, pos);
    if constexpr (sizeof(T) == 2) st_cache(p, p.k_cache, p.k_scale, dst + d, h * D + d, kr);
    else st_elem<T>(p.k_cache, dst + d, kr);
  } else {
    const int h = hs - p.Hq - p.Hkv;
    const int64_t src = ((int64_t)b * p.nq + j) * p.kv_stride + (int64_t)h * D;
    const int64_t dst = (((int64_t)b * p.Hkv + h) * p.cap + L + j) * D;
    const InView vv{p.v_new, (int64_t)p.B * p.nq * p.kv_stride, p.in_splits, p.act_pair};
    if constexpr (sizeof(T) == 2) st_cache(p, p.v_cache, p.v_scale, dst + d, h * D + d, ld_in<T>(vv, src + d));
    else st_elem<T>(p.v_cache, dst + d, ld_in<T>(vv, src + d));
  }
}

// ---------------------------------------------------------------------------
// 2a. bf16 multi-query attention on MFMA
//
// Workgroup = 4 waves, one workgroup per CU.  Key tiles of 64 keys (and values,
// unless the layer reuses the keys) stream HBM -> LDS by direct-to-LDS DMA
// through a ring of NS stages.  Per tile:
//   QK : wave w scores its own 16 keys against all rows over the full head
//        dimension (16x16x32 MFMAs; A = key rows read from the staged tile, B =
//        the rotated queries, held in registers for the whole piece), so every
//        score is produced and exponentiated by exactly one wave;
//   max: the waves exchange their per-row tile maxima; the reference max of a
//        row only moves when the tile max exceeds it by more than 2^8 (lazy
//        rescaling), so p = 2^(s - m) <= 256 and the accumulators are rescaled
//        only when some row needs it;
//   P  : each wave writes its bf16 weights to LDS in exactly the lane layout the
//        PV product reads them in (an 8-byte same-lane transfer);
//   PV : wave w owns the dims [w*D/4, (w+1)*D/4): O^T[dim, row] += V^T[dim, key]
//        P^T[key, row]; V^T is read from the staged row-major tile with the LDS
//        transpose read.
// Staged rows are unpadded; 16-byte chunk c of key row r lives in slot
// c ^ swz(r), which spreads both the row-wise and the transposed reads over the
// LDS banks.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) ^ ((r >> 2) & 1); }

// A small block of rows (sliding-window layers) is combined by the last piece of its
// segment to finish; a large one by attn_merge, which spreads the work over the chip.
constexpr bool attn_fuse_merge(int D, int MT) { return D * 16 * MT <= 4096; }

// Two workgroups per compute unit: fp8 keys of the 512-dim heads with one row tile.
// Two stages of half-size (fp8) tiles fit twice in LDS and the kernel fits 128
// registers of each kind without spilling, so a second workgroup's tile chain
// (LDS reads, widening, MFMA, the softmax exchange) fills the latency of the
// first one's; the chip then holds twice as many pieces (measured 16 % faster at
// 8 x 131k keys).  With two row tiles the queries alone need the 128 registers, and
// the 256-dim sliding-window heads, whose pieces are a few tiles long, measured no
// gain.
constexpr bool attn_two_per_cu(int D, int MT, bool FP8) { return FP8 && D == 512 && MT == 1; }

template <int D, int MT, bool KV_SAME, bool FP8>
struct AttnCfg {
  static constexpr int DS = D / 4;              // PV dims per wave
  static constexpr int KS = D / 32;             // 32-dim k-steps of QK (full head)
  static constexpr int DT = DS / 16;            // 16-dim output tiles of PV per wave
  static constexpr int TK = 64;                 // keys per tile (16 per wave)
  static constexpr int ROWB = FP8 ? D : D * 2;  // bytes per key row (fp8 codes or bf16)
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per DMA instruction
  static constexpr int NTEN = KV_SAME ? 1 : 2;  // staged tensors
  static constexpr int TILEB = TK * ROWB;
  static constexpr int STAGEB = TILEB * NTEN;
  static constexpr int NI = (TK / RPI) * NTEN / 4;  // DMA instructions per wave per tile
  static constexpr int SMALLB = 4 * MT * 64 * 8 + 2 * 4 * MT * 16 * 4;  // P and max/sum exchange
  static constexpr int NS_FIT = (160 * 1024 - SMALLB) / STAGEB;
  static constexpr int NS = attn_two_per_cu(D, MT, FP8) ? 2 : (NS_FIT < 4 ? NS_FIT : 4);  // ring stages
  static_assert(NS >= 2, "tile does not fit twice in LDS");
  static_assert(DT >= 1 && RPI >= 1 && NI >= 1, "unsupported head_dim");
  static_assert((NS - 2) * NI <= 63, "vmcnt range");
};

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

// eight fp8 E4M3 codes (byte e = element e) as eight bf16 values (exact: every
// E4M3 value is a bf16 value)
__device__ __forceinline__ V16 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  V16 r;
  r.w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false));
  r.w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true));
  r.w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false));
  r.w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true));
  return r;
}

template <int D, int MT, bool KV_SAME, bool FP8>
__global__ __launch_bounds__(256, attn_two_per_cu(D, MT, FP8) ? 2 : 1) void attn_mfma_kernel(AttnParams p) {
  using C = AttnCfg<D, MT, KV_SAME, FP8>;
  constexpr int DS = C::DS, KS = C::KS, DT = C::DT, TK = C::TK, ROWB = C::ROWB, CPR = C::CPR,
                RPI = C::RPI, TILEB = C::TILEB, STAGEB = C::STAGEB, NI = C::NI, NS = C::NS;

  // one LDS object per ring stage (the stage loop is kept rolled: unrolling it by NS
  // lets the scheduler stretch live ranges across stages and costs spills)
  __shared__ __attribute__((aligned(16))) unsigned char s_st0[STAGEB];
  __shared__ __attribute__((aligned(16))) unsigned char s_st1[STAGEB];
  __shared__ __attribute__((aligned(16))) unsigned char s_st2[NS > 2 ? STAGEB : 16];
  __shared__ __attribute__((aligned(16))) unsigned char s_st3[NS > 3 ? STAGEB : 16];
  __shared__ __attribute__((aligned(16))) uint2 s_p[4][MT][64];      // bf16 weights, PV lane layout
  __shared__ float s_max[4][MT][16];                                 // per-wave row maxima of a tile
  __shared__ float s_sum[4][MT][16];                                 // per-wave row sums of a piece
  __shared__ int s_flag[4];                                          // wave's rows passed the reference
  auto stage_of = [&](int u) -> unsigned char* {
    return u == 0 ? s_st0 : u == 1 ? s_st1 : u == 2 ? s_st2 : s_st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int M = p.M, G = p.G;

  const BatchLens bl = batch_lens(p);
  const Pieces pc = {p.plan[0], p.plan[1]};   // computed once by rope_append_kernel
  const int slot = blockIdx.x;  // this workgroup's piece
  if (slot >= pc.n) return;
  int b, kvh, first, count;
  int64_t a0, a1;  // keys [a0, a1) of sequence b, kv head kvh
  int64_t L;       // committed length of sequence b
  piece_locate(p, bl, pc.chunk, slot, b, kvh, a0, a1, first, count, L);
  // the piece is the same for the whole workgroup: in scalar registers, every tile-level
  // decision below (tile count, stage waits, masking, the last partial tile) is a
  // scalar branch rather than an exec-mask one
  auto uni64 = [](int64_t v) {
    const uint64_t u = (uint64_t)v;
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
  };
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  first = __builtin_amdgcn_readfirstlane(first);
  count = __builtin_amdgcn_readfirstlane(count);
  a0 = uni64(a0);
  a1 = uni64(a1);
  L = uni64(L);

  const uint16_t* qrot = (const uint16_t*)p.q_rot;
  const unsigned char* kcache = (const unsigned char*)p.k_cache;
  const unsigned char* vcache = (const unsigned char*)p.v_cache;
  {
    {
      const int64_t last = L + p.n_new - 1;
      const int ntiles = (int)((a1 - a0 + TK - 1) / TK);

      // every real row sees keys [seg_max_lo, seg_min_hi] (row 0 has the lowest causal
      // limit, the last row the highest window start)
      const int64_t seg_min_hi = (L + p.qoff) < last ? (L + p.qoff) : last;
      const int64_t seg_max_lo = p.window > 0 ? L + p.qoff + p.nq - p.window : INT64_MIN;
      const int64_t head_row0 = ((int64_t)b * p.Hkv + kvh) * p.cap;  // row index of key 0
      // DMA of tile t into its ring stage: wave w moves NI instructions of 1 KB each;
      // lane l carries 16 B of row (l / CPR) of the instruction's row block.  The row
      // block's address is wave-uniform; the per-lane byte offsets (row within the
      // block, swizzled chunk) repeat every tile and are computed once.  Only a tile
      // that runs past the piece clamps rows to its last row (finite data, masked out
      // of the softmax) with per-lane offsets.
      uint32_t off_pre[NI];
#pragma unroll
      for (int jj = 0; jj < NI; ++jj) {
        const int rb = (wave * NI + jj) % (TK / RPI);
        const int row = rb * RPI + lane / CPR;
        off_pre[jj] = (uint32_t)((lane / CPR) * ROWB + (((lane % CPR) ^ swz(row)) << 4));
      }
      auto issue_one = [&](int t, unsigned char* stage, int jj) __attribute__((always_inline)) {
        const int64_t t0 = a0 + (int64_t)t * TK;
        const bool partial = t0 + TK > a1;
        {
          const int ii = wave * NI + jj;
          const int ten = ii / (TK / RPI);
          const int rb = ii % (TK / RPI);
          const unsigned char* tbase = (KV_SAME || ten == 0) ? kcache : vcache;
          const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr(stage + ten * TILEB + rb * RPI * ROWB));
          int64_t brow = t0 + rb * RPI;  // first row of the block
          uint32_t off = off_pre[jj];
          if (partial) {
            if (brow > a1 - 1) brow = a1 - 1;
            const int row = rb * RPI + lane / CPR;
            int64_t key = t0 + row;
            if (key > a1 - 1) key = a1 - 1;
            off = (uint32_t)((key - brow) * ROWB + (((lane % CPR) ^ swz(row)) << 4));
          }
          dma16<true, true>((const void*)(tbase + (head_row0 + brow) * ROWB), off, lds);
        }
      };
      auto issue = [&](int t, unsigned char* stage) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < NI; ++jj) issue_one(t, stage, jj);
      };

      // the first tiles' DMA goes out before anything else
#pragma unroll
      for (int u = 0; u < NS - 1; ++u)
        if (u < ntiles) issue(u, stage_of(u));


      // ---- queries of this (sequence, kv head), full head dim, as MFMA B operands
      // The 4 x MT (key tile, row tile) pairs of a tile's scores go to the waves.  With
      // two row tiles (KM) wave w takes key tile w against both, so each key operand is
      // read from LDS (and, for fp8 keys, widened) once and feeds two MFMAs (measured
      // 1.5 % faster with bf16 keys, 9 % with fp8); otherwise the pairs go in
      // row-tile-major order, MT consecutive pairs per wave, and a wave scores at most
      // two row tiles (one unless MT == 3), so it holds only those rows of the queries.
      constexpr bool KM = MT == 2 || MT == 3;
      constexpr int NQ = KM ? MT : (MT == 3 ? 2 : 1);
      const int mq0 = KM ? 0 : (wave * MT) >> 2;  // the wave's first row tile
      V16 qreg[NQ][KS];
#pragma unroll
      for (int lt = 0; lt < NQ; ++lt) {
        const int r = (mq0 + lt) * 16 + lr;
        if (mq0 + lt < MT && r < M) {
          const int j = r / G, hg = r - (r / G) * G;
          const uint16_t* src = qrot + (((int64_t)b * p.nq + j) * p.Hq + kvh * G + hg) * D + lg * 8;
#pragma unroll
          for (int s = 0; s < KS; ++s) qreg[lt][s].u = *(const uint4*)(src + s * 32);
          if constexpr (FP8) {
            // fp8 keys are scale * code: the per-channel key scales are folded into the
            // queries (rounded to bf16), so the products take the codes as they are
            const float* ksc = p.k_scale + kvh * D + lg * 8;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              const f32x4_t a = *(const f32x4_t*)(ksc + s * 32), c = *(const f32x4_t*)(ksc + s * 32 + 4);
              const float sc[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                qreg[lt][s].w[e] = pack_bf16x2(bf16_lo(qreg[lt][s].w[e]) * sc[2 * e], bf16_hi(qreg[lt][s].w[e]) * sc[2 * e + 1]);
            }
          }
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s) qreg[lt][s].u = make_uint4(0, 0, 0, 0);
        }
      }
      // consume the query loads here (the compiler then waits for them once, not
      // inside the tile loop, which also waits for the first tiles: their DMA went out
      // before the queries were requested, so the two latencies overlap)
#pragma unroll
      for (int lt = 0; lt < NQ; ++lt)
#pragma unroll
        for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qreg[lt][s].b));
      wait_vm_n<0>();

      f32x4_t O[DT][MT];
      float m_run[MT], l_run[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        m_run[mt] = kNegInf;
        l_run[mt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

      for (int tb = 0; tb < ntiles; tb += NS) {
#pragma unroll 1
      for (int u = 0; u < NS; ++u) {
        const int t = tb + u;  // tile t lives in stage u
        if (t >= ntiles) break;
        const int64_t t0 = a0 + (int64_t)t * TK;
        const int ahead = (NS - 2) < (ntiles - 1 - t) ? (NS - 2) : (ntiles - 1 - t);
        wait_stages<NI>(ahead);
        lds_barrier();  // tile t is in LDS for every wave; tile t-1 is no longer read
        // The next tile's DMA goes out spread over the score MFMAs below, so the
        // memory pipe's issue back-pressure overlaps matrix work.  A full next tile
        // takes a branch-free path (wave-uniform row base, per-lane offsets fixed); a
        // partial one (the last of a piece) is issued up front with clamped rows.
        const bool more = t + NS - 1 < ntiles;
        const int64_t tn0 = a0 + (int64_t)(t + NS - 1) * TK;
        const bool nfull = more && tn0 + TK <= a1;
        unsigned char* nstage = stage_of((u + NS - 1) % NS);
        if (more && !nfull) issue(t + NS - 1, nstage);

        const unsigned char* kst = stage_of(u);
        const unsigned char* vst = kst + (KV_SAME ? 0 : TILEB);

        // ---- scores of the wave's pairs: pair j = (key tile kt, row tile mt) holds
        // S^T[key, row] with row mt*16 + lr and keys 16*kt + 4*lg + {0..3}.  The key
        // operands are read KPF k-steps ahead of their MFMAs; with few pairs, NCH
        // chains over alternate k-steps keep the MFMA pipe busy (with fp8 keys and two
        // row tiles the widening between the MFMAs already hides their latency: one
        // chain measured 1.7 % faster there).
        constexpr int NCH = MT == 1 ? 4 : (MT == 2 && !FP8 ? 2 : 1);
        constexpr int PER = (NI + KS - 1) / KS;  // DMA instructions per k-step
        constexpr int KPF = FP8 ? (KS < 2 ? KS : 2) : (KS < 4 ? KS : 4);
        constexpr int NK = KM ? 1 : MT;  // distinct key tiles of the wave's pairs
        int pkt[MT], pmt[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          pkt[j] = KM ? wave : (wave * MT + j) & 3;
          pmt[j] = KM ? j : (wave * MT + j) >> 2;
        }
        f32x4_t sacc[MT];
        auto scores = [&](auto dma) {
          constexpr bool DMA = decltype(dma)::value;
          f32x4_t sch[NCH][MT];
#pragma unroll
          for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int j = 0; j < MT; ++j) sch[c][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const unsigned char* krow[NK];
          int sw[NK];
#pragma unroll
          for (int j = 0; j < NK; ++j) {
            const int r = pkt[j] * 16 + lr;
            krow[j] = kst + r * ROWB;
            sw[j] = swz(r);
          }
          // key operands: 8 dims of a key row per lane (16 bytes of bf16, or 8 fp8 codes
          // widened to bf16 when used)
          auto kaddr = [&](int s, int j) -> const unsigned char* {
            if constexpr (FP8) return krow[j] + (((2 * s + (lg >> 1)) ^ sw[j]) << 4) + ((lg & 1) << 3);
            else return krow[j] + (((4 * s + lg) ^ sw[j]) << 4);
          };
          using KQ = typename std::conditional<FP8, uint2, uint4>::type;
          KQ kq[KPF][NK];
#pragma unroll
          for (int s = 0; s < KPF; ++s)
#pragma unroll
            for (int j = 0; j < NK; ++j) kq[s][j] = *(const KQ*)kaddr(s, j);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            if constexpr (DMA) {
#pragma unroll
              for (int q = 0; q < PER; ++q) {
                const int jj = s * PER + q;
                if (jj < NI) {
                  const int ii = wave * NI + jj;
                  const int ten = ii / (TK / RPI);
                  const int rb = ii % (TK / RPI);
                  const unsigned char* tbase = (KV_SAME || ten == 0) ? kcache : vcache;
                  dma16<false, true>((const void*)(tbase + (head_row0 + tn0 + rb * RPI) * ROWB), off_pre[jj],
                               lds_addr(nstage + ten * TILEB + rb * RPI * ROWB));
                }
              }
            }
            V16 kreg[NK];
#pragma unroll
            for (int j = 0; j < NK; ++j) {
              if constexpr (FP8) kreg[j] = fp8x8_to_bf16(kq[s % KPF][j].x, kq[s % KPF][j].y);
              else kreg[j].u = kq[s % KPF][j];
              if (s + KPF < KS) kq[s % KPF][j] = *(const KQ*)kaddr(s + KPF, j);
            }
#pragma unroll
            for (int j = 0; j < MT; ++j) {
              const bf16x8_t qv = KM ? qreg[j][s].b : ((NQ == 1 || pmt[j] == mq0) ? qreg[0][s].b : qreg[NQ - 1][s].b);
              sch[s % NCH][j] = mfma16x16x32(kreg[KM ? 0 : j].b, qv, sch[s % NCH][j]);
            }
          }
          if constexpr (FP8) {
            // keep KPF k-steps of key reads ahead; each step's codes are widened right
            // before its MFMAs, so only one step of widened operands is live
            __builtin_amdgcn_sched_group_barrier(0x100, KPF * NK, 0);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              __builtin_amdgcn_sched_group_barrier(0x002, 4 * NK, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
              if (s + KPF < KS) __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
            }
          } else {
            // keep KPF k-steps of key reads ahead of the MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, KPF * NK, 0);
#pragma unroll
            for (int s = 0; s < KS - KPF; ++s) {
              __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KPF * MT, 0);
          }
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            f32x4_t a = sch[0][j];
#pragma unroll
            for (int c = 1; c < NCH; ++c) {
              a[0] += sch[c][j][0]; a[1] += sch[c][j][1]; a[2] += sch[c][j][2]; a[3] += sch[c][j][3];
            }
            sacc[j] = a;
          }
        };
        if (nfull) scores(std::true_type{});
        else scores(std::false_type{});

        // the running max of row tile mt (a uniform index) without indexing registers
        auto pick = [&](const float (&v)[MT], int mt) {
          float x = v[0];
#pragma unroll
          for (int m = 1; m < MT; ++m) x = mt == m ? v[m] : x;
          return x;
        };
        const bool full = (t0 + TK <= a1) && (t0 + TK - 1 <= seg_min_hi) && (t0 >= seg_max_lo);
        float sc[MT][4];
        bool over = false;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          int lo_l = -1, hi_l = TK;
          if (!full) {
            // causal and window limits of row pmt[j]*16 + lr (padded rows: none)
            const int r = pmt[j] * 16 + lr;
            int64_t rhi = INT64_MAX, rlo = INT64_MIN;
            if (r < M) {
              const int64_t pos = L + p.qoff + r / G;
              rhi = pos < last ? pos : last;
              rlo = p.window > 0 ? pos - p.window + 1 : 0;
            }
            const int64_t hi = (rhi < a1 - 1 ? rhi : a1 - 1) - t0;
            const int64_t lo2 = rlo - t0;
            hi_l = hi < -1 ? -1 : (hi > TK ? TK : (int)hi);
            lo_l = lo2 < -1 ? -1 : (lo2 > TK ? TK : (int)lo2);
          }
          float mx = kNegInf;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kl = pkt[j] * 16 + lg * 4 + i;
            // (full tiles keep lo_l = -1, hi_l = TK; the test is written with bitwise
            // operators so that it compiles to compares and a select, not branches)
            sc[j][i] = ((kl >= lo_l) & (kl <= hi_l)) ? sacc[j][i] * p.scale_log2 : kNegInf;
            mx = fmaxf(mx, sc[j][i]);
          }
          mx = row4_max(mx);
          if (lg == 0) s_max[pkt[j]][pmt[j]][lr] = mx;
          over |= mx > pick(m_run, pmt[j]) + 8.f;
        }
        // The reference max of a row only moves when some key exceeds it by more than
        // 2^8 (lazy rescaling).  Each wave computes its weights against the current
        // reference straight away and flags whether any of its rows went over; only
        // then do the waves combine their maxima, move the reference and redo the
        // weights (one extra barrier, rare after the first tile of a piece).
        const bool wover = __any(over);  // vote with every lane active
        if (lane == 0) s_flag[wave] = wover ? 1 : 0;
        float rsum[MT];
        auto weights = [&]() {
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            const float m = pick(m_run, pmt[j]);
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = m == kNegInf ? 0.f : __builtin_amdgcn_exp2f(sc[j][i] - m);
            uint2 w2;
            w2.x = pack_bf16x2(pv[0], pv[1]);
            w2.y = pack_bf16x2(pv[2], pv[3]);
            s_p[pkt[j]][pmt[j]][lane] = w2;
            // the normaliser sums exactly the (bf16) weights the PV product uses
            float rs = bf16_lo(w2.x) + bf16_hi(w2.x) + bf16_lo(w2.y) + bf16_hi(w2.y);
            rs = row4_sum(rs);
            rsum[j] = rs;
          }
        };
        weights();
        lds_barrier();  // weights, maxima and flags of every wave visible

        // the same decision on every wave (a scalar branch: the rescale of the output
        // accumulators then stays inside this rare path)
        if (__builtin_amdgcn_readfirstlane(s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3])) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const float tmax = fmaxf(fmaxf(s_max[0][mt][lr], s_max[1][mt][lr]), fmaxf(s_max[2][mt][lr], s_max[3][mt][lr]));
            // rows whose maximum moved get the new reference; the others keep theirs
            // (alpha = 1), without a branch per lane
            const bool mv = tmax > m_run[mt] + 8.f;
            const float m_new = mv ? tmax : m_run[mt];
            const float alpha = !mv ? 1.f : (m_run[mt] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[mt] - m_new));
            l_run[mt] *= alpha;
            m_run[mt] = m_new;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              // (an empty statement that takes the accumulators where the MFMAs keep
              // them: their copies for the multiply are then made here, in this rare
              // branch, and not at the top of every tile)
              asm volatile("" : "+a"(O[dt][mt]));
              O[dt][mt][0] *= alpha; O[dt][mt][1] *= alpha;
              O[dt][mt][2] *= alpha; O[dt][mt][3] *= alpha;
            }
          }
          weights();
          lds_barrier();  // the redone weights visible
        }
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (pmt[j] == mt) l_run[mt] += rsum[j];

        // ---- O^T += V^T P^T over the tile's two 32-key halves.  Lane i of a 16-lane
        // group feeds row 32*ks + 16*h + 4*lg + i/4, dims 4*(i%4)..+3 of the tile; the
        // transpose read returns dim (lane % 16) of rows 32*ks + 16*h + 4*lg + {0..3},
        // matching P slots 4*h + e (written by wave 2*ks + h).
        {
          const int i = lane & 15;
          const int a = i & 3;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            V16 pb[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const uint2 p0 = s_p[2 * ks][mt][lane], p1 = s_p[2 * ks + 1][mt][lane];
              pb[mt].u = make_uint4(p0.x, p0.y, p1.x, p1.y);
            }
            // value operands are read one dim tile ahead of their MFMAs
            auto read_v = [&](int dt) {
              if constexpr (FP8) {
                // 8-bit transpose read: lane 2k + h of the 16-lane group points at key
                // slot k, dims 16 c16 + 8h; lane i gets dim 16 c16 + i of the 8 keys
                const int c16 = wave * (DS / 16) + dt;
                const int k = i >> 1;
                const int r = 32 * ks + 16 * (k >> 2) + 4 * lg + (k & 3);
                const unsigned char* ad = vst + r * ROWB + ((c16 ^ swz(r)) << 4) + ((i & 1) << 3);
                const v2i_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)ad);
                return fp8x8_to_bf16((uint32_t)v[0], (uint32_t)v[1]);
              }
              const int c = wave * (DS / 8) + 2 * dt + (a >> 1);
              V16 av;
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int r = 32 * ks + 16 * h + 4 * lg + (i >> 2);
                const unsigned char* ad = vst + r * ROWB + ((c ^ swz(r)) << 4) + ((a & 1) << 3);
                const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)ad);
                av.w[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                av.w[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
              }
              return av;
            };
            V16 avq[2];
            avq[0] = read_v(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              if (dt + 1 < DT) avq[(dt + 1) & 1] = read_v(dt + 1);
              const V16 av = avq[dt & 1];
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) O[dt][mt] = mfma16x16x32(av.b, pb[mt].b, O[dt][mt]);
            }
          }
        }
      }
      }

      if constexpr (FP8) {
        // values are scale * code: the per-channel value scales multiply the output
        const float* vsc = (KV_SAME ? p.k_scale : p.v_scale) + kvh * D + wave * DS + lg * 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4_t sc = *(const f32x4_t*)(vsc + dt * 16);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            O[dt][mt][0] *= sc[0]; O[dt][mt][1] *= sc[1]; O[dt][mt][2] *= sc[2]; O[dt][mt][3] *= sc[3];
          }
        }
      }
      // ---- unnormalised partial of this piece: the row sums of the four waves
      // (each over its own keys, all on the same reference) add up
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (lg == 0) s_sum[wave][mt][lr] = l_run[mt];
      __syncthreads();
      if constexpr (!attn_fuse_merge(D, MT)) {
        // combined by attn_merge, a later kernel
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = mt * 16 + lr;
          if (r < M) {
            float* dst = p.part_acc + ((int64_t)slot * M + r) * D + wave * DS + lg * 4;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(dst + dt * 16) = O[dt][mt];
            if (wave == 0 && lg == 0) {
              p.part_ml[((int64_t)slot * M + r) * 2 + 0] = m_run[mt];
              p.part_ml[((int64_t)slot * M + r) * 2 + 1] =
                  (s_sum[0][mt][lr] + s_sum[1][mt][lr]) + (s_sum[2][mt][lr] + s_sum[3][mt][lr]);
            }
          }
        }
        return;
      }
      // partials go through the device coherence point to the segment's last piece
      const __amdgpu_buffer_rsrc_t acc_rsrc =
          __builtin_amdgcn_make_buffer_rsrc(p.part_acc, (short)0, p.part_acc_bytes, kBufferWord3);
      const __amdgpu_buffer_rsrc_t ml_rsrc =
          __builtin_amdgcn_make_buffer_rsrc(p.part_ml, (short)0, p.part_ml_bytes, kBufferWord3);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + lr;
        if (r < M) {
          const uint32_t off = (uint32_t)((((int64_t)slot * M + r) * D + wave * DS + lg * 4) * 4);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) __builtin_amdgcn_raw_buffer_store_b128(O[dt][mt], acc_rsrc, off + dt * 64, 0, kCoherent);
          if (wave == 0 && lg == 0) {
            const float l = (s_sum[0][mt][lr] + s_sum[1][mt][lr]) + (s_sum[2][mt][lr] + s_sum[3][mt][lr]);
            const uint32_t mo = (uint32_t)((((int64_t)slot * M + r) * 2) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run[mt]), ml_rsrc, mo, 0, kCoherent);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), ml_rsrc, mo + 4, 0, kCoherent);
          }
        }
      }
      // count this piece once its stores have completed; the last of the segment merges
      wait_vm_n<0>();
      __syncthreads();
      const int seg = b * p.Hkv + kvh;
      if (tid == 0) s_flag[0] = __hip_atomic_fetch_add(p.seg_cnt + seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_flag[0] != count - 1) return;

      // ---- merge of the segment's pieces [first, first + count) in one pass: each
      // thread keeps, for its output quads, the running reference mx, the sum l and
      // the output rescaled to it, so that out = sum_w 2^(m_w - mx) O_w /
      // sum_w 2^(m_w - mx) l_w needs one round of loads per batch of PB pieces (with
      // all of a batch's loads in flight; slots past the segment re-read its last
      // piece, so that every loaded value is finite, and are masked out).  Up to PB
      // pieces, mx is the largest reference of the row and no rescaling happens.
      auto ld_ml = [&](int w, int r, int e) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            ml_rsrc, (uint32_t)((((int64_t)w * M + r) * 2 + e) * 4), 0, kCoherent));
      };
      const int wend = first + count;
      // two output quads per thread and pass; batches of 4 pieces where that is all
      // there are (fewer redundant loads), else of 8
      constexpr int DQ = D / 4;
      constexpr int NIT = 2;
      auto merge = [&](auto pb) __attribute__((always_inline)) {
      constexpr int PB = decltype(pb)::value;
      for (int i0 = tid; i0 < M * DQ; i0 += 256 * NIT) {
        f32x4_t acc[NIT];
        float mx[NIT], l[NIT];
        int rr[NIT], dd[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int i = i0 + it * 256 < M * DQ ? i0 + it * 256 : i0;
          rr[it] = i / DQ;
          dd[it] = (i - rr[it] * DQ) * 4;
          acc[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          mx[it] = kNegInf;
          l[it] = 0.f;
        }
        for (int w0 = first; w0 < wend; w0 += PB) {
          float mv[NIT][PB], lv[NIT][PB];
          f32x4_t v[NIT][PB];
#pragma unroll
          for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int k = 0; k < PB; ++k) {
              const int wk = w0 + k < wend ? w0 + k : wend - 1;
              mv[it][k] = ld_ml(wk, rr[it], 0);
              lv[it][k] = ld_ml(wk, rr[it], 1);
              v[it][k] = __builtin_amdgcn_raw_buffer_load_b128(
                  acc_rsrc, (uint32_t)((((int64_t)wk * M + rr[it]) * D + dd[it]) * 4), 0, kCoherent);
            }
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            // a piece that saw no key of this row has m = -inf and acc = 0
            float nmx = mx[it];
#pragma unroll
            for (int k = 0; k < PB; ++k) nmx = (w0 + k < wend) ? fmaxf(nmx, mv[it][k]) : nmx;
            // without per-lane branches: a = 1 leaves the state as it is (also when no
            // piece so far saw a key of this row, nmx = -inf, where every f below is 0)
            const float a = mx[it] == nmx ? 1.f : (mx[it] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mx[it] - nmx));
            l[it] *= a;
            acc[it][0] *= a; acc[it][1] *= a; acc[it][2] *= a; acc[it][3] *= a;
            mx[it] = nmx;
#pragma unroll
            for (int k = 0; k < PB; ++k) {
              const float f = (w0 + k < wend && mv[it][k] != kNegInf) ? __builtin_amdgcn_exp2f(mv[it][k] - nmx) : 0.f;
              l[it] += f * lv[it][k];
              acc[it][0] += f * v[it][k][0]; acc[it][1] += f * v[it][k][1];
              acc[it][2] += f * v[it][k][2]; acc[it][3] += f * v[it][k][3];
            }
          }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          if (i0 + it * 256 >= M * DQ) continue;
          const int r = rr[it];
          const float inv = l[it] > 0.f ? 1.f / l[it] : 0.f;
          const int j = r / G, hg = r - (r / G) * G;
          st_out4(p, (((int64_t)b * p.nq + j) * p.Hq + kvh * G + hg) * D + dd[it], acc[it][0] * inv,
                  acc[it][1] * inv, acc[it][2] * inv, acc[it][3] * inv);
        }
      }
      };
      if (count <= 4) merge(std::integral_constant<int, 4>{});
      else merge(std::integral_constant<int, 8>{});
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
// 3. merge of the split-KV partials (bf16 path) in a kernel of its own, for blocks of
//    rows too large for the last arriving piece to combine quickly
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnParams p) {
  const int r = blockIdx.x;          // row within the (sequence, kv head) block
  const int seg = blockIdx.y;        // b * Hkv + kvh
  const int b = seg / p.Hkv, kvh = seg % p.Hkv;
  const int64_t L = p.cache_len[b];
  if (!seq_ok(p, L)) return;
  const BatchLens bl = batch_lens(p);
  const Pieces pc = {p.plan[0], p.plan[1]};
  int first, nb;
  segment_pieces(p, bl, pc.chunk, b, kvh, first, nb);
  int64_t lo, len;
  seq_range(p, b, lo, len);
  const int64_t w0 = first, w1 = (int64_t)first + nb - 1;
  const int D = p.D, G = p.G;
  const int j = r / G, hg = r % G;
  const int64_t out0 = (((int64_t)b * p.nq + j) * p.Hq + kvh * G + hg) * D;
  const int d0 = threadIdx.x * 4;
  if (d0 >= D) return;
  if (len == 0) {
    st_out4(p, out0 + d0, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  // one pass over the pieces in batches of PB, all of a batch's loads in flight:
  // the running reference mx, the sum l and the output a rescaled to it (slots
  // past the segment re-read its last piece and are masked out)
  constexpr int PB = 8;
  float mx = kNegInf, l = 0.f;
  f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t wb = w0; wb <= w1; wb += PB) {
    float mv[PB], lv[PB];
    f32x4_t v[PB];
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const int64_t slot = wb + k <= w1 ? wb + k : w1;
      mv[k] = p.part_ml[(slot * p.M + r) * 2];
      lv[k] = p.part_ml[(slot * p.M + r) * 2 + 1];
      v[k] = *(const f32x4_t*)(p.part_acc + (slot * p.M + r) * D + d0);
    }
    float nmx = mx;
#pragma unroll
    for (int k = 0; k < PB; ++k) nmx = wb + k <= w1 ? fmaxf(nmx, mv[k]) : nmx;
    // a piece that saw no key of this row has m = -inf, acc = 0; c = 1 leaves the state
    // as it is, without a per-lane branch
    const float c = mx == nmx ? 1.f : (mx == kNegInf ? 0.f : exp2f(mx - nmx));
    l *= c;
    a[0] *= c; a[1] *= c; a[2] *= c; a[3] *= c;
    mx = nmx;
#pragma unroll
    for (int k = 0; k < PB; ++k) {
      const float f = (wb + k <= w1 && mv[k] != kNegInf) ? exp2f(mv[k] - nmx) : 0.f;
      l += f * lv[k];
      a[0] += f * v[k][0]; a[1] += f * v[k][1]; a[2] += f * v[k][2]; a[3] += f * v[k][3];
    }
  }
  const float a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  st_out4(p, out0 + d0, a0 * inv, a1 * inv, a2 * inv, a3 * inv);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int kAttnNwgMax = 2048;

struct AttnPlan {
  size_t q_rot_bytes, acc_bytes, ml_bytes, cnt_bytes, plan_bytes, total;
  int M, slots;
};

// Workspace layout.  The attention cuts the keys into at most max(nwg, B * Hkv)
// pieces (nwg = the device's compute units, twice that where two workgroups share
// a compute unit), each with one partial slot; the
// public size query allows nwg up to kAttnNwgMax so that it does not depend on the
// device, the static scratch of sv_verify_attn_noalloc is laid out for the
// current device's nwg.
static AttnPlan attn_plan(const sv_attn_desc& d, int nwg_max = kAttnNwgMax) {
  AttnPlan pl{};
  const size_t elt = d.dtype == SV_BF16 ? 2 : 4;
  pl.M = (d.n_heads_q / d.n_heads_kv) * d.n_q;
  pl.q_rot_bytes = align_up((size_t)d.batch * d.n_q * d.n_heads_q * d.head_dim * elt, 256);
  if (d.dtype == SV_BF16) {
    pl.slots = nwg_max + d.batch * d.n_heads_kv;
    pl.acc_bytes = align_up((size_t)pl.slots * pl.M * d.head_dim * 4, 256);
    pl.ml_bytes = align_up((size_t)pl.slots * pl.M * 2 * 4, 256);
    pl.cnt_bytes = align_up((size_t)d.batch * d.n_heads_kv * 4, 256);
    pl.plan_bytes = 256;
  }
  pl.total = pl.q_rot_bytes + pl.acc_bytes + pl.ml_bytes + pl.cnt_bytes + pl.plan_bytes;
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
  if (d->in_splits < 0 || d->reserved_f != 0.f || d->reserved_i != 0) return SV_ERR_ARG;
  if (d->act_pair != 0 && d->act_pair != 1) return SV_ERR_ARG;
  if (d->act_pair && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->in_splits > 0 && d->dtype != SV_BF16) return SV_ERR_ARG;
  if (d->cache_capacity <= 0) return SV_ERR_ARG;
  if (d->q_row_stride < 0 || d->kv_row_stride < 0) return SV_ERR_ARG;
  if (d->q_row_stride && d->q_row_stride < (int64_t)d->n_heads_q * d->head_dim) return SV_ERR_ARG;
  if (d->kv_row_stride && d->kv_row_stride < (int64_t)d->n_heads_kv * d->head_dim) return SV_ERR_ARG;
  if (d->rope_dims > 0 && !(d->rope_base > 1.0)) return SV_ERR_ARG;
  if (!(d->softmax_scale > 0.f)) return SV_ERR_ARG;
  if (d->dtype == SV_BF16) {
    if (d->head_dim != 128 && d->head_dim != 256 && d->head_dim != 512) return SV_ERR_UNSUPPORTED;
    // a 64-key tile of separate 512-wide keys and values (128 KB) cannot be double-buffered in LDS
    if (d->head_dim == 512 && !d->k_is_v) return SV_ERR_UNSUPPORTED;
    if ((d->n_heads_q / d->n_heads_kv) * d->n_q > 64) return SV_ERR_UNSUPPORTED;
    // the work split handles up to 256 sequences with key counts below 2^31
    if (d->batch > 64 * kPlanGroups || d->cache_capacity > INT32_MAX - 4096) return SV_ERR_UNSUPPORTED;
  } else if (d->dtype == SV_F32) {
    if (d->head_dim > 512) return SV_ERR_UNSUPPORTED;
    if (d->cache_capacity > kF32MaxKeys) return SV_ERR_UNSUPPORTED;
  } else {
    return SV_ERR_ARG;
  }
  if ((int64_t)d->batch * d->n_q * d->n_heads_q > (int64_t)1 << 24) return SV_ERR_UNSUPPORTED;
  return SV_OK;
}

template <int D, int MT, bool KVS, bool FP8>
static void launch_mfma(const AttnParams& p, hipStream_t s) {
  // one workgroup per piece: at most nwg pieces, or one per segment when there are more segments
  const int grid = p.nwg > p.B * p.Hkv ? p.nwg : p.B * p.Hkv;
  hipLaunchKernelGGL((attn_mfma_kernel<D, MT, KVS, FP8>), dim3(grid), dim3(256), 0, s, p);
}

template <int D, bool KVS, bool FP8>
static int dispatch_mfma(const AttnParams& p, int MT, hipStream_t s) {
  switch (MT) {
    case 1: launch_mfma<D, 1, KVS, FP8>(p, s); break;
    case 2: launch_mfma<D, 2, KVS, FP8>(p, s); break;
    case 3: launch_mfma<D, 3, KVS, FP8>(p, s); break;
    case 4: launch_mfma<D, 4, KVS, FP8>(p, s); break;
    default: return SV_ERR_UNSUPPORTED;
  }
  return SV_OK;
}

template <bool FP8>
static int dispatch_attn(const sv_attn_desc* d, const AttnParams& p, int MT, hipStream_t s) {
  switch (d->head_dim * 2 + (d->k_is_v ? 1 : 0)) {
    case 256: return dispatch_mfma<128, false, FP8>(p, MT, s);
    case 257: return dispatch_mfma<128, true, FP8>(p, MT, s);
    case 512: return dispatch_mfma<256, false, FP8>(p, MT, s);
    case 513: return dispatch_mfma<256, true, FP8>(p, MT, s);
    case 1025: return dispatch_mfma<512, true, FP8>(p, MT, s);
    default: return SV_ERR_UNSUPPORTED;
  }
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_verify_attn_workspace(const sv_attn_desc* d) {
  if (validate_attn(d) != SV_OK) return 0;
  return attn_plan(*d).total;
}

static int verify_attn(const sv_attn_desc* d, const void* q, const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, const float* k_scale, const float* v_scale, bool fp8,
                       const int32_t* cache_len, void* out, void* workspace, size_t workspace_bytes,
                       int32_t* dev_status, void* stream, int nwg_max = kAttnNwgMax) {
  int rc = validate_attn(d);
  if (rc != SV_OK) return rc;
  if (fp8) {
    if (d->dtype != SV_BF16) return SV_ERR_ARG;
    if (!k_scale || ((uintptr_t)k_scale & 15)) return SV_ERR_ARG;
    if (d->k_is_v ? v_scale != nullptr : (!v_scale || ((uintptr_t)v_scale & 15))) return SV_ERR_ARG;
  }
  if (!q || !k_cache || !cache_len || !out) return SV_ERR_ARG;
  if (d->append && !k_new) return SV_ERR_ARG;
  if (!d->append && (k_new || v_new)) return SV_ERR_ARG;
  if (d->k_is_v && (v_cache || v_new)) return SV_ERR_ARG;
  if (!d->k_is_v && !v_cache) return SV_ERR_ARG;
  if (!d->k_is_v && d->append && !v_new) return SV_ERR_ARG;
  const AttnPlan pl = attn_plan(*d, nwg_max);
  if (!workspace || workspace_bytes < pl.total) return SV_ERR_WORKSPACE;
  rc = check_device();
  if (rc != SV_OK) return rc;
  // pieces: one per workgroup the chip holds at once
  const int nwg = attn_two_per_cu(d->head_dim, (pl.M + 15) / 16, fp8) ? 2 * device_cus() : device_cus();
  if (nwg > nwg_max) return SV_ERR_UNSUPPORTED;  // more pieces than partial slots

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
  p.seg_cnt = (int32_t*)(ws + pl.q_rot_bytes + pl.acc_bytes + pl.ml_bytes);
  p.plan = (int32_t*)(ws + pl.q_rot_bytes + pl.acc_bytes + pl.ml_bytes + pl.cnt_bytes);
  p.part_acc_bytes = (int)pl.acc_bytes;
  p.part_ml_bytes = (int)pl.ml_bytes;
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
  p.nwg = nwg;
  p.min_chunk = 64;
  p.in_splits = d->in_splits;
  p.act_pair = d->act_pair;
  p.out_plane = (int64_t)d->batch * d->n_q * d->n_heads_q * d->head_dim;
  p.fp8 = fp8 ? 1 : 0;
  p.k_scale = k_scale;
  p.v_scale = d->k_is_v ? k_scale : v_scale;

  hipStream_t s = (hipStream_t)stream;
  const int heads = d->n_heads_q + (d->append ? d->n_heads_kv * (d->k_is_v ? 1 : 2) : 0);
  const int rope_threads = (d->head_dim + 63) / 64 * 64;
  if (d->dtype == SV_BF16) {
    hipLaunchKernelGGL(rope_append_kernel<uint16_t>, dim3(d->batch * d->n_q, heads), dim3(rope_threads), 0, s, p);
    const int MT = (pl.M + 15) / 16;
    rc = fp8 ? dispatch_attn<true>(d, p, MT, s) : dispatch_attn<false>(d, p, MT, s);
    if (rc != SV_OK) return rc;
    if (!attn_fuse_merge(d->head_dim, MT))
      // (at least one full wave: the piece plan works across 64 lanes)
      hipLaunchKernelGGL(attn_merge_kernel, dim3(pl.M, d->batch * d->n_heads_kv),
                         dim3(d->head_dim / 4 > 64 ? d->head_dim / 4 : 64), 0, s, p);
  } else {
    hipLaunchKernelGGL(rope_append_kernel<float>, dim3(d->batch * d->n_q, heads), dim3(rope_threads), 0, s, p);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(d->n_heads_q, d->n_q, d->batch), dim3(256), 0, s, p);
  }
  return launch_status();
}

extern "C" int sv_verify_attn(const sv_attn_desc* d, const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* cache_len, void* out, void* workspace,
                              size_t workspace_bytes, int32_t* dev_status, void* stream) {
  return verify_attn(d, q, k_new, v_new, k_cache, v_cache, nullptr, nullptr, false, cache_len, out, workspace,
                     workspace_bytes, dev_status, stream);
}

extern "C" int sv_verify_attn_fp8(const sv_attn_desc* d, const void* q, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                                  const int32_t* cache_len, void* out, void* workspace, size_t workspace_bytes,
                                  int32_t* dev_status, void* stream) {
  return verify_attn(d, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, true, cache_len, out, workspace,
                     workspace_bytes, dev_status, stream);
}

// ---------------------------------------------------------------------------
// The variant that allocates nothing: the workspace is a static device array.
// ---------------------------------------------------------------------------
// One copy per GPU, held from the library's first use on that GPU until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: kernels get the address that hipGetSymbolAddress returns for
// the current device (kept per device in g_scratch).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
std::atomic<char*> g_scratch[kScratchDevices];

// The current device's copy of `scratch` (nullptr if the runtime cannot give it).
char* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  char* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr = (char*)a;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}
}  // namespace

extern "C" int sv_verify_attn_noalloc(const sv_attn_desc* d, const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* cache_len, void* out,
                                      int32_t* dev_status, void* stream) {
  int rc = validate_attn(d);
  if (rc != SV_OK) return rc;
  rc = check_device();  // (also caches the compute-unit count the layout uses)
  if (rc != SV_OK) return rc;
  const int nwg = device_cus();
  if (attn_plan(*d, nwg).total > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  char* ws = device_scratch();
  if (!ws) return SV_ERR_DEVICE;
  // every call sets what the kernels need at a known value itself (arrival
  // counters, work split), so nothing left by an earlier call is read
  return verify_attn(d, q, k_new, v_new, k_cache, v_cache, nullptr, nullptr, false, cache_len, out, ws,
                     (size_t)SV_NOALLOC_SCRATCH_BYTES, dev_status, stream, nwg);
}
