// stack.hip -- the small elementwise pieces of a decoder layer around the verify
// attention: tied-embedding lookup, RMSNorm and the GeGLU gate.  The target's
// own forward over the k+1 verify rows ("Gemma 4 拆解" (marsggbo), section 4.2:
// main_model.verify) is built from these plus sv_linear and sv_verify_attn.
#include "sv_device.h"
#include "sv_host.h"

namespace sv {

__global__ __launch_bounds__(256) void embed_kernel(int d_model, int vocab, int bf16, const int32_t* tokens,
                                                    const void* table, float scale, float* x,
                                                    int32_t* dev_status) {
  const int r = blockIdx.x;
  const int tok = tokens[r];
  float* dst = x + (int64_t)r * d_model;
  const bool ok = tok >= 0 && tok < vocab;
  if (!ok && threadIdx.x == 0) set_status(dev_status, SV_DEV_BAD_TOKEN);
  for (int i = threadIdx.x; i < d_model; i += 256) {
    float v = 0.f;
    if (ok) {
      const int64_t o = (int64_t)tok * d_model + i;
      v = bf16 ? bf16_to_f32(((const uint16_t*)table)[o]) : ((const float*)table)[o];
    }
    dst[i] = scale * v;
  }
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(int dim, float eps, const float* x, const float* gain,
                                                      void* y, int bf16) {
  __shared__ float s_red[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (int64_t)r * dim;
  float ss = 0.f;
  for (int i = tid; i < dim; i += 256) ss = fmaf(xr[i], xr[i], ss);
  s_red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) s_red[tid] += s_red[tid + s];
    __syncthreads();
  }
  const float inv = 1.f / sqrtf(s_red[0] / (float)dim + eps);
  for (int i = tid; i < dim; i += 256) {
    float v = xr[i] * inv;
    if (gain) v *= gain[i];
    if (bf16) ((uint16_t*)y)[(int64_t)r * dim + i] = (uint16_t)f32_to_bf16_bits(v);
    else ((float*)y)[(int64_t)r * dim + i] = v;
  }
}

// gelu, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;
  return 0.5f * x * (1.f + tanhf(c * (x + 0.044715f * x * x * x)));
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
  if (out_dtype != SV_F32 && out_dtype != SV_BF16) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, (hipStream_t)stream, dim, eps, x, gain, y,
                     out_dtype == SV_BF16 ? 1 : 0);
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
