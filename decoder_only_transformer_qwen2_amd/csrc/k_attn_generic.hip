// Generic causal grouped-query attention over the KV cache (vector ALUs).
//
// "LLM Speedrun: Architecture": section "Attention" (scores q.k scaled by
// 1/sqrt(d_k), softmax over keys, weighted sum of values), "Every token with
// every other token" (causal: a query at position p sees keys 0..p) and
// "Grouped Query Attention GQA" (query head h reads KV head floor(h / g)).
//
// One wavefront per (query row, query head).  Keys are visited 64 at a time,
// one key per lane for the scores; the softmax is accumulated online (running
// max and sum), so masked keys never enter and no score matrix is stored.
// Used for the fp32 path and for head dims the MFMA kernels do not take.
#include "qw_internal.h"

#include <math.h>

namespace qw {

namespace {
constexpr int MAX_HD = 128;

template <typename T>
__global__ void __launch_bounds__(256) attn_generic_kernel(AttnArgs a) {
  __shared__ float qs[4][MAX_HD];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wv;
  const bool active = gw < (int64_t)a.T * a.n_heads;
  const int t = active ? (int)(gw / a.n_heads) : 0, h = active ? (int)(gw % a.n_heads) : 0;
  const int hd = a.head_dim;
  const int g = a.n_heads / a.n_kv_heads, j = h / g;
  int b, pos;
  if (a.rag.cu) {
    b = ragged_seq(a.rag.cu, a.rag.n, t);
    pos = t - a.rag.cu[b];
  } else {
    b = t / a.rows_per_seq;
    pos = (a.pos0_dev ? a.pos0_dev[b] : a.pos0) + (t % a.rows_per_seq);
  }
  const int qd = a.n_heads * hd;
  const T *q = (const T *)a.q + (int64_t)t * qd + h * hd;
  for (int d = lane; d < hd; d += 64) qs[wv][d] = to_f32(q[d]) * a.softmax_scale;
  __syncthreads();
  if (!active) return;
  const T *K = (const T *)a.k_cache;
  const T *V = (const T *)a.v_cache;

  float m = -INFINITY, l = 0.f;
  float o0 = 0.f, o1 = 0.f;                   // dims lane and lane + 64
  const int n_keys = pos + 1;
  for (int c0 = 0; c0 < n_keys; c0 += 64) {
    const int tau = c0 + lane;
    float s = -INFINITY;
    if (tau < n_keys) {
      const T *kr = K + kv_offset(a.kv, a.n_kv_heads, hd, b, j, tau);
      float dot = 0.f;
      for (int d = 0; d < hd; ++d) dot = fmaf(qs[wv][d], to_f32(kr[d]), dot);
      s = dot;
    }
    const float cmax = wave_max(s);
    const float m_new = fmaxf(m, cmax);
    const float corr = __expf(m - m_new);     // 0 on the first chunk (m = -inf)
    const float p = (tau < n_keys) ? expf(s - m_new) : 0.f;
    l = l * corr + wave_sum(p);
    o0 *= corr;
    o1 *= corr;
    const int cnt = min(64, n_keys - c0);
    for (int u = 0; u < cnt; ++u) {
      const float pu = __shfl(p, u, 64);
      const T *vr = V + kv_offset(a.kv, a.n_kv_heads, hd, b, j, c0 + u);
      if (lane < hd) o0 = fmaf(pu, to_f32(vr[lane]), o0);
      if (lane + 64 < hd) o1 = fmaf(pu, to_f32(vr[lane + 64]), o1);
    }
    m = m_new;
  }
  T *o = (T *)a.o + (int64_t)t * qd + h * hd;
  const float inv = 1.0f / l;
  if (lane < hd) o[lane] = from_f32<T>(o0 * inv);
  if (lane + 64 < hd) o[lane + 64] = from_f32<T>(o1 * inv);
}
}  // namespace

hipError_t launch_attention_generic(hipStream_t s, bool f16_mode, const AttnArgs &a) {
  if (a.T <= 0) return hipSuccess;
  if (a.head_dim > MAX_HD) return hipErrorInvalidValue;
  const int64_t waves = (int64_t)a.T * a.n_heads;
  dim3 grid((unsigned)((waves + 3) / 4));
  if (f16_mode)
    QW_LAUNCH((attn_generic_kernel<f16>), dim3(grid), dim3(256), 0, s, a);
  else
    QW_LAUNCH((attn_generic_kernel<float>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qw
