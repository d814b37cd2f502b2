// stack.hip -- the small elementwise pieces of a decoder layer around the verify
// attention: tied-embedding lookup, RMSNorm and the GeGLU gate.  The target's
// own forward over the k+1 verify rows ("Gemma 4 拆解" (marsggbo), section 4.2:
// main_model.verify) is built from these plus sv_linear and sv_verify_attn.
#include "sv_device.h"
#include "sv_host.h"

namespace sv {

// One workgroup per row.  Rows of d_model % 4 == 0 move as 4-element vectors
// (8-byte bf16 / 16-byte fp32 loads, 16-byte fp32 stores); others element-wise.
__global__ __launch_bounds__(256) void embed_kernel(int d_model, int vocab, int bf16, const int32_t* tokens,
                                                    const void* table, float scale, float* x,
                                                    int32_t* dev_status) {
  const int r = blockIdx.x;
  const int tok = tokens[r];
  float* dst = x + (int64_t)r * d_model;
  const bool ok = tok >= 0 && tok < vocab;
  if (!ok && threadIdx.x == 0) set_status(dev_status, SV_DEV_BAD_TOKEN);
  if ((d_model & 3) == 0 && (((uintptr_t)table | (uintptr_t)x) & 15) == 0) {
    const int n4 = d_model / 4;
    for (int i = threadIdx.x; i < n4; i += 256) {
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (ok) {
        if (bf16) {
          const uint2 w = *(const uint2*)((const uint16_t*)table + (int64_t)tok * d_model + 4 * i);
          v = f32x4_t{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        } else {
          v = *(const f32x4_t*)((const float*)table + (int64_t)tok * d_model + 4 * i);
        }
      }
      *(f32x4_t*)(dst + 4 * i) = f32x4_t{scale * v[0], scale * v[1], scale * v[2], scale * v[3]};
    }
    return;
  }
  for (int i = threadIdx.x; i < d_model; i += 256) {
    float v = 0.f;
    if (ok) {
      const int64_t o = (int64_t)tok * d_model + i;
      v = bf16 ? bf16_to_f32(((const uint16_t*)table)[o]) : ((const float*)table)[o];
    }
    dst[i] = scale * v;
  }
}

// One workgroup per row: the row is read once into registers (4-element vectors,
// up to kNormVec per thread), squared and summed with wavefront shuffles and one
// exchange between the four waves, then scaled and stored.
constexpr int kNormVec = 8;  // rows up to 256 * 4 * 8 = 8192 elements take the register path

// Norm output y[i..i+3] in the output type: 0 fp32, 1 bf16, 2 bf16 pair (hi plane,
// then the lo plane `plane` elements further: hi = bf16(o), lo = bf16(o - hi)).
__device__ __forceinline__ void st_norm4(void* y, int mode, int64_t i, int64_t plane, const f32x4_t& o) {
  if (mode == 0) {
    *(f32x4_t*)((float*)y + i) = o;
    return;
  }
  const uint32_t h01 = pack_bf16x2(o[0], o[1]), h23 = pack_bf16x2(o[2], o[3]);
  *(uint2*)((uint16_t*)y + i) = make_uint2(h01, h23);
  if (mode == 2)
    *(uint2*)((uint16_t*)y + plane + i) =
        make_uint2(pack_bf16x2(o[0] - bf16_lo(h01), o[1] - bf16_hi(h01)), pack_bf16x2(o[2] - bf16_lo(h23), o[3] - bf16_hi(h23)));
}
__device__ __forceinline__ void st_norm1(void* y, int mode, int64_t i, int64_t plane, float o) {
  if (mode == 0) {
    ((float*)y)[i] = o;
    return;
  }
  const uint32_t h = f32_to_bf16_bits(o);
  ((uint16_t*)y)[i] = (uint16_t)h;
  if (mode == 2) ((uint16_t*)y)[plane + i] = (uint16_t)f32_to_bf16_bits(o - bf16_to_f32((uint16_t)h));
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(int dim, float eps, const float* x, const float* gain,
                                                      void* y, int mode) {
  const int64_t plane = (int64_t)gridDim.x * dim;
  __shared__ float s_red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (int64_t)r * dim;
  const bool vec = (dim & 3) == 0 && dim <= 256 * 4 * kNormVec &&
                   (((uintptr_t)x | (uintptr_t)y | (uintptr_t)gain) & 15) == 0;
  f32x4_t v[kNormVec];
  float ss = 0.f;
  if (vec) {
    const int n4 = dim / 4;
#pragma unroll
    for (int k = 0; k < kNormVec; ++k) {
      const int i = tid + 256 * k;
      v[k] = i < n4 ? *(const f32x4_t*)(xr + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < kNormVec; ++k)
      ss = fmaf(v[k][0], v[k][0], fmaf(v[k][1], v[k][1], fmaf(v[k][2], v[k][2], fmaf(v[k][3], v[k][3], ss))));
  } else {
    for (int i = tid; i < dim; i += 256) ss = fmaf(xr[i], xr[i], ss);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) ss += shfl_xor_f(ss, m);
  if ((tid & 63) == 0) s_red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float inv = 1.f / sqrtf(tot / (float)dim + eps);
  if (vec) {
    const int n4 = dim / 4;
#pragma unroll
    for (int k = 0; k < kNormVec; ++k) {
      const int i = tid + 256 * k;
      if (i >= n4) break;
      f32x4_t o = f32x4_t{v[k][0] * inv, v[k][1] * inv, v[k][2] * inv, v[k][3] * inv};
      if (gain) {
        const f32x4_t g = *(const f32x4_t*)(gain + 4 * i);
        o = f32x4_t{o[0] * g[0], o[1] * g[1], o[2] * g[2], o[3] * g[3]};
      }
      st_norm4(y, mode, (int64_t)r * dim + 4 * i, plane, o);
    }
    return;
  }
  for (int i = tid; i < dim; i += 256) {
    float o = xr[i] * inv;
    if (gain) o *= gain[i];
    st_norm1(y, mode, (int64_t)r * dim + i, plane, o);
  }
}

// Residual add of K-split partial products, then RMSNorm: one workgroup of 1024
// threads per row, at most kAddVec 4-element vectors of the row per thread, so that
// a row and kSplitBatch slices of it are in flight at once.  The slices are summed
// in slice order (a = ((p0 + p1) + p2) + ...), then added to the row, which is
// written back.
constexpr int kAddThreads = 1024, kAddVec = 2, kSplitBatch = 8;

__global__ __launch_bounds__(kAddThreads) void add_rmsnorm_kernel(int rows, int dim, float eps, float* x,
                                                                  const float* parts, int splits,
                                                                  const float* gain, void* y, int mode) {
  __shared__ float s_red[kAddThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n4 = dim / 4;
  float* xr = x + (int64_t)r * dim;
  f32x4_t v[kAddVec], a[kAddVec];
#pragma unroll
  for (int k = 0; k < kAddVec; ++k) {
    const int i = tid + kAddThreads * k;
    v[k] = i < n4 ? *(const f32x4_t*)(xr + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    a[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int s0 = 0; s0 < splits; s0 += kSplitBatch) {
    f32x4_t pv[kSplitBatch][kAddVec];
#pragma unroll
    for (int j = 0; j < kSplitBatch; ++j)
#pragma unroll
      for (int k = 0; k < kAddVec; ++k) {
        const int i = tid + kAddThreads * k;
        pv[j][k] = (s0 + j < splits && i < n4)
                       ? *(const f32x4_t*)(parts + ((int64_t)(s0 + j) * rows + r) * dim + 4 * i)
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int j = 0; j < kSplitBatch; ++j)
      if (s0 + j < splits)
#pragma unroll
        for (int k = 0; k < kAddVec; ++k)
          a[k] = f32x4_t{a[k][0] + pv[j][k][0], a[k][1] + pv[j][k][1], a[k][2] + pv[j][k][2], a[k][3] + pv[j][k][3]};
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kAddVec; ++k) {
    if (splits > 0) v[k] = f32x4_t{v[k][0] + a[k][0], v[k][1] + a[k][1], v[k][2] + a[k][2], v[k][3] + a[k][3]};
    ss = fmaf(v[k][0], v[k][0], fmaf(v[k][1], v[k][1], fmaf(v[k][2], v[k][2], fmaf(v[k][3], v[k][3], ss))));
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) ss += shfl_xor_f(ss, m);
  if ((tid & 63) == 0) s_red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kAddThreads / 64; w += 2) tot += s_red[w] + s_red[w + 1];
  const float inv = 1.f / sqrtf(tot / (float)dim + eps);
#pragma unroll
  for (int k = 0; k < kAddVec; ++k) {
    const int i = tid + kAddThreads * k;
    if (i >= n4) break;
    if (splits > 0) *(f32x4_t*)(xr + 4 * i) = v[k];
    f32x4_t o = f32x4_t{v[k][0] * inv, v[k][1] * inv, v[k][2] * inv, v[k][3] * inv};
    if (gain) {
      const f32x4_t g = *(const f32x4_t*)(gain + 4 * i);
      o = f32x4_t{o[0] * g[0], o[1] * g[1], o[2] * g[2], o[3] * g[3]};
    }
    st_norm4(y, mode, (int64_t)r * dim + 4 * i, (int64_t)rows * dim, o);
  }
}

// Drafter input stage: one workgroup per sequence; the gathered hidden row and the
// scaled embedding row are each RMS-normalised (sums of squares in fp32, one
// wavefront-shuffle and one LDS exchange per part) and written side by side in bf16.
__device__ __forceinline__ float block_sum_256(float v, float* s_red) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += shfl_xor_f(v, m);
  __syncthreads();  // s_red free from any previous use
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

__global__ __launch_bounds__(256) void draft_input_kernel(int d_main, int d_draft, float eps, const uint16_t* hidden,
                                                          int rows_h, const int32_t* hidden_row, int row_stride,
                                                          const uint16_t* emb, int vocab, const int32_t* tokens,
                                                          int tok_stride, float emb_scale, uint16_t* cat, int pair,
                                                          float* x, int32_t* dev_status) {
  __shared__ float s_red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int dc = d_main + d_draft;
  const int hr = hidden_row[(int64_t)b * row_stride];
  const int tok = tokens[(int64_t)b * tok_stride];
  const bool hok = hr >= 0 && hr < rows_h, tok_ok = tok >= 0 && tok < vocab;
  if (tid == 0 && !(hok && tok_ok)) set_status(dev_status, SV_DEV_BAD_TOKEN);
  const uint16_t* hrow = hidden + (int64_t)(hok ? hr : 0) * d_main;
  const uint16_t* erow = emb + (int64_t)(tok_ok ? tok : 0) * d_draft;
  float ss = 0.f;
  for (int i = tid; i < d_main; i += 256) {
    const float v = bf16_to_f32(hrow[i]);
    ss = fmaf(v, v, ss);
  }
  const float hinv = hok ? 1.f / sqrtf(block_sum_256(ss, s_red) / (float)d_main + eps) : 0.f;
  ss = 0.f;
  for (int i = tid; i < d_draft; i += 256) {
    const float v = emb_scale * bf16_to_f32(erow[i]);
    ss = fmaf(v, v, ss);
  }
  const float einv = tok_ok ? 1.f / sqrtf(block_sum_256(ss, s_red) / (float)d_draft + eps) : 0.f;
  // bf16, or the pair: plane 0 bf16(v), plane 1 bf16(v - plane 0), planes gridDim.x * dc apart
  uint16_t* crow = cat + (int64_t)b * dc;
  const int64_t plane = (int64_t)gridDim.x * dc;
  auto put = [&](int i, float v) {
    const uint32_t h = f32_to_bf16_bits(v);
    crow[i] = (uint16_t)h;
    if (pair) crow[plane + i] = (uint16_t)f32_to_bf16_bits(v - bf16_to_f32((uint16_t)h));
  };
  for (int i = tid; i < d_main; i += 256) put(i, bf16_to_f32(hrow[i]) * hinv);
  for (int i = tid; i < d_draft; i += 256) put(d_main + i, emb_scale * bf16_to_f32(erow[i]) * einv);
  for (int i = tid; i < d_draft; i += 256) x[(int64_t)b * d_draft + i] = 0.f;
}

__global__ __launch_bounds__(256) void geglu_kernel(int rows, int dff, int bf16, const void* gu, void* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * dff) return;
  const int64_t r = i / dff, c = i % dff;
  const int64_t gi = r * 2 * dff + c, ui = gi + dff;
  float g, u;
  if (bf16) {
    g = bf16_to_f32(((const uint16_t*)gu)[gi]);
    u = bf16_to_f32(((const uint16_t*)gu)[ui]);
  } else {
    g = ((const float*)gu)[gi];
    u = ((const float*)gu)[ui];
  }
  const float f = gelu_tanh(g) * u;
  if (bf16) ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_bits(f);
  else ((float*)out)[i] = f;
}

}  // namespace sv

using namespace sv;

extern "C" int sv_embed(int32_t rows, int32_t d_model, int32_t vocab, sv_dtype dtype, const int32_t* tokens,
                        const void* table, float scale, float* x, int32_t* dev_status, void* stream) {
  if (rows <= 0 || d_model <= 0 || vocab <= 0 || !tokens || !table || !x) return SV_ERR_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, (hipStream_t)stream, d_model, vocab,
                     dtype == SV_BF16 ? 1 : 0, tokens, table, scale, x, dev_status);
  return launch_status();
}

extern "C" int sv_rmsnorm(int32_t rows, int32_t dim, float eps, const float* x, const float* gain, void* y,
                          sv_dtype out_dtype, void* stream) {
  if (rows <= 0 || dim <= 0 || !x || !y || !(eps >= 0.f)) return SV_ERR_ARG;
  if (out_dtype != SV_F32 && out_dtype != SV_BF16 && out_dtype != SV_BF16X2) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, (hipStream_t)stream, dim, eps, x, gain, y,
                     out_dtype == SV_F32 ? 0 : out_dtype == SV_BF16 ? 1 : 2);
  return launch_status();
}

extern "C" int sv_add_rmsnorm(int32_t rows, int32_t dim, float eps, float* x, const float* parts, int32_t splits,
                              const float* gain, void* y, sv_dtype out_dtype, void* stream) {
  if (rows <= 0 || dim <= 0 || !x || !y || !(eps >= 0.f) || splits < 0) return SV_ERR_ARG;
  if (out_dtype != SV_F32 && out_dtype != SV_BF16 && out_dtype != SV_BF16X2) return SV_ERR_ARG;
  if (!parts) splits = 0;
  if (dim % 4 || (((uintptr_t)x | (uintptr_t)parts | (uintptr_t)gain | (uintptr_t)y) & 15)) return SV_ERR_ARG;
  if (dim > kAddThreads * 4 * kAddVec) return SV_ERR_UNSUPPORTED;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(rows), dim3(kAddThreads), 0, (hipStream_t)stream, rows, dim, eps, x,
                     parts, splits, gain, y, out_dtype == SV_F32 ? 0 : out_dtype == SV_BF16 ? 1 : 2);
  return launch_status();
}

extern "C" int sv_draft_input(int32_t batch, int32_t d_main, int32_t d_draft, float eps, const void* hidden,
                              int32_t rows_h, const int32_t* hidden_row, int32_t row_stride, const void* emb,
                              int32_t vocab, const int32_t* tokens, int32_t tok_stride, float emb_scale, void* cat,
                              sv_dtype cat_dtype, float* x, int32_t* dev_status, void* stream) {
  if (batch <= 0 || d_main <= 0 || d_draft <= 0 || rows_h <= 0 || vocab <= 0 || !(eps >= 0.f)) return SV_ERR_ARG;
  if (cat_dtype != SV_BF16 && cat_dtype != SV_BF16X2) return SV_ERR_ARG;
  if (!hidden || !hidden_row || !emb || !tokens || !cat || !x || row_stride < 0 || tok_stride < 0) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(draft_input_kernel, dim3(batch), dim3(256), 0, (hipStream_t)stream, d_main, d_draft, eps,
                     (const uint16_t*)hidden, rows_h, hidden_row, row_stride, (const uint16_t*)emb, vocab, tokens,
                     tok_stride, emb_scale, (uint16_t*)cat, cat_dtype == SV_BF16X2 ? 1 : 0, x, dev_status);
  return launch_status();
}

extern "C" int sv_geglu(int32_t rows, int32_t d_ff, sv_dtype dtype, const void* gate_up, void* out,
                        void* stream) {
  if (rows <= 0 || d_ff <= 0 || !gate_up || !out) return SV_ERR_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  const int64_t n = (int64_t)rows * d_ff;
  hipLaunchKernelGGL(geglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, rows,
                     d_ff, dtype == SV_BF16 ? 1 : 0, gate_up, out);
  return launch_status();
}
