// accept.hip -- longest-accepted-prefix rule with KV append / rollback indices.
//
// "Gemma 4 拆解" (marsggbo), sections 4.1 / 4.2 (accept_longest_prefix: keep the
// drafts the target agrees with, cut at the first wrong one, restart from
// there); "Accelerating Gemma 4 ..." (Lighthouse), section 3 (the target adds
// one token of its own).  Sampling mode applies the standard speculative
// rejection rule (accept draft i with probability min(1, p/q)), whose only
// property the pages state is that the output distribution is unchanged
// ("Gemma 4 与 Gemini Nano" (kongchang), section "草稿模型").
//
// Single-pass sampling takes the residual token after a rejection from the first
// pass's candidates of the rejected row by rejection (see sv_accept_rs).
//
// One thread per sequence; the committed length moves from L_b to L_b + n_b + 1,
// rows [L_b + n_b + 1, L_b + k + 1) are rolled back by not being committed (the
// next verify step appends over them), so no cache data moves.
#include "sv_device.h"
#include "sv_host.h"

namespace sv {

template <bool SAMPLE, bool RS>
__global__ __launch_bounds__(64) void accept_kernel(sv_accept_desc d, const int32_t* drafts,
                                                    const sv_row_stats* stats, const float* q_rows,
                                                    const float* u_acc, int32_t* cache_len,
                                                    int32_t* out_tokens, sv_accept_out* acc,
                                                    int32_t* dev_status, const sv_rs_cand* cands,
                                                    const float* u_rs) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= d.batch) return;
  const int k = d.k, base = b * (k + 1);
  int n = 0;
  for (int i = 0; i < k; ++i) {
    const int dt = drafts[b * k + i];
    if (dt < 0 || dt >= d.vocab) {
      set_status(dev_status, SV_DEV_BAD_TOKEN);
      break;
    }
    const sv_row_stats& s = stats[base + i];
    if constexpr (SAMPLE) {
      const float p = expf(s.draft_logit - s.lse);
      const float q = q_rows[((int64_t)b * k + i) * d.vocab + dt];
      const float u = u_acc[b * k + i];
      if (!(u * q < p)) break;
    } else {
      if (dt != s.top1_id) break;
    }
    ++n;
  }
  int y, res = -1;
  float margin;
  const sv_row_stats& last = stats[base + n];
  if constexpr (SAMPLE) {
    if (n == k) {
      y = last.sample_id;
      margin = last.sample_s1 - last.sample_s2;
    } else {
      y = -1;
      res = base + n;
      margin = 0.f;
      if constexpr (RS) {
        // the residual by rejection: candidate x (a draw from p of this row) is taken
        // iff u p(x) < p(x) - q(x)
        const float* qrow = q_rows + ((int64_t)b * k + n) * d.vocab;
        for (int c = 0; c < SV_RS_CANDIDATES; ++c) {
          const sv_rs_cand x = cands[((int64_t)b * k + n) * SV_RS_CANDIDATES + c];
          if (x.id < 0 || x.id >= d.vocab) continue;
          const float p = expf(x.z - last.lse);
          const float u = u_rs[b * SV_RS_CANDIDATES + c];
          if (u * p < p - qrow[x.id]) {
            y = x.id;
            res = -1;
            margin = x.s1 - x.s2;
            break;
          }
        }
      }
    }
  } else {
    y = last.top1_id;
    margin = last.top1 - last.top2;
  }
  const int L = cache_len[b];
  for (int i = 0; i <= k; ++i) out_tokens[base + i] = i < n ? drafts[b * k + i] : (i == n ? y : -1);
  sv_accept_out o;
  o.n_accepted = n;
  o.next_token = y;
  o.new_len = L + n + 1;
  o.keep_begin = L;
  o.keep_end = L + n + 1;
  o.drop_begin = L + n + 1;
  o.drop_end = L + k + 1;
  o.hidden_row = base + n;
  o.residual_row = res;
  o.draw_margin = margin;
  acc[b] = o;
  cache_len[b] = L + n + 1;
}

}  // namespace sv

using namespace sv;

extern "C" int sv_accept(const sv_accept_desc* d, const int32_t* drafts, const sv_row_stats* stats,
                         const float* q_rows, const float* u_accept, int32_t* cache_len,
                         int32_t* out_tokens, sv_accept_out* acc, int32_t* dev_status, void* stream) {
  if (!d) return SV_ERR_ARG;
  if (d->batch <= 0 || d->k < 0 || d->vocab <= 0) return SV_ERR_ARG;
  if (d->mode != SV_SELECT_GREEDY && d->mode != SV_SELECT_SAMPLE) return SV_ERR_ARG;  // SAMPLE_RS: sv_accept_rs
  if (!stats || !cache_len || !out_tokens || !acc) return SV_ERR_ARG;
  if (d->k > 0 && !drafts) return SV_ERR_ARG;
  if (d->mode == SV_SELECT_SAMPLE && d->k > 0 && (!q_rows || !u_accept)) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const unsigned g = (unsigned)((d->batch + 63) / 64);
  if (d->mode == SV_SELECT_SAMPLE)
    hipLaunchKernelGGL((accept_kernel<true, false>), dim3(g), dim3(64), 0, s, *d, drafts, stats, q_rows, u_accept,
                       cache_len, out_tokens, acc, dev_status, nullptr, nullptr);
  else
    hipLaunchKernelGGL((accept_kernel<false, false>), dim3(g), dim3(64), 0, s, *d, drafts, stats, q_rows, u_accept,
                       cache_len, out_tokens, acc, dev_status, nullptr, nullptr);
  return launch_status();
}

extern "C" int sv_accept_rs(const sv_accept_desc* d, const int32_t* drafts, const sv_row_stats* stats,
                            const sv_rs_cand* cands, const float* q_rows, const float* u_accept, const float* u_rs,
                            int32_t* cache_len, int32_t* out_tokens, sv_accept_out* acc, int32_t* dev_status,
                            void* stream) {
  if (!d) return SV_ERR_ARG;
  if (d->batch <= 0 || d->k < 0 || d->vocab <= 0 || d->mode != SV_SELECT_SAMPLE_RS) return SV_ERR_ARG;
  if (!stats || !cache_len || !out_tokens || !acc) return SV_ERR_ARG;
  if (d->k > 0 && (!drafts || !q_rows || !u_accept || !cands || !u_rs)) return SV_ERR_ARG;
  int rc = check_device();
  if (rc != SV_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const unsigned g = (unsigned)((d->batch + 63) / 64);
  hipLaunchKernelGGL((accept_kernel<true, true>), dim3(g), dim3(64), 0, s, *d, drafts, stats, q_rows, u_accept,
                     cache_len, out_tokens, acc, dev_status, cands, u_rs);
  return launch_status();
}
