// Sampling of the next token and the end-of-sequence rule.
//
// "augur" lists temperature, top-k and top-p sampling as not yet built and
// EOS stopping as part of generation; the speedrun harness stops on the
// end-of-stream token.  The pages give no formulas for the sampling, so the
// plain reading is taken: keep the top_k largest logits (ties: lower index
// first), weight them by exp((l - l_max) / temperature), keep the shortest
// prefix of that order whose weight reaches top_p of the total, and pick by
// the inverse cumulative distribution of one uniform draw u in [0, 1).  The
// draw is counter-based (Philox-4x64-10, Salmon et al., SC 2011): counter
// (n, sequence, 0, 0) under key (seed, 0), n = tokens in the sequence before
// the one being chosen, so a run with the cache and one without draw alike.
//
// One workgroup of 1024 threads per sequence:
//   1. radix selection (four passes of 8-bit digit histograms, most
//      significant first) of the top_k-th largest logit as an order-keeping
//      32-bit key;
//   2. the candidates: every key above it, and the lowest-index keys equal
//      to it up to top_k in all;
//   3. a bitonic sort in LDS by (logit desc, index asc);
//   4. weights, an inclusive scan, the top-p cut and the pick.
#include "qw_internal.h"

#include <math.h>

namespace qw {
namespace {

constexpr int kSampleThreads = 1024;      // also the largest top_k

// A float as an unsigned key with the same order (NaN sorts below -inf).
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0u;
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// First 64-bit word of Philox-4x64-10 for counter (c0, c1, 0, 0), key (k0, 0).
__device__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t k0) {
  uint64_t c[4] = {c0, c1, 0, 0};
  uint64_t k[2] = {k0, 0};
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = 0xD2E7470EE14C6C93ull * c[0], hi0 = __umul64hi(0xD2E7470EE14C6C93ull, c[0]);
    const uint64_t lo1 = 0xCA5A826395121157ull * c[2], hi1 = __umul64hi(0xCA5A826395121157ull, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k[0], n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k[0] += 0x9E3779B97F4A7C15ull;
    k[1] += 0xBB67AE8584CAA73Bull;
  }
  return c[0];
}

// Inclusive sum over the block (16 waves), in LDS scratch of 16 floats.
__device__ float block_inclusive_scan(float v, float *s_w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) s_w[wave] = v;
  __syncthreads();
  float add = 0.f;
  for (int w = 0; w < wave; ++w) add += s_w[w];
  __syncthreads();
  return v + add;
}

__device__ int block_count(bool p, int *s_c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = __popcll(__ballot(p));
  if (lane == 0) s_c[wave] = c;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kSampleThreads / 64; ++w) t += s_c[w];
  __syncthreads();
  return t;
}

__global__ void __launch_bounds__(kSampleThreads) sample_kernel(const float *__restrict__ logits, int64_t row_stride,
                                                                int V, float inv_temp, int top_k, float top_p,
                                                                uint64_t seed, const int *pos_dev,
                                                                int32_t *next, int *finished, int eos) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const float *row = logits + (int64_t)b * row_stride;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_left;
  __shared__ uint64_t s_key[kSampleThreads];
  __shared__ float s_w[16];
  __shared__ int s_c[16], s_ngt, s_neq;
  const int k = min(top_k, V);

  // 1. the k-th largest key, digit by digit
  uint32_t prefix = 0, mask = 0, left = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int d = tid; d < 256; d += kSampleThreads) hist[d] = 0;
    __syncthreads();
    for (int v = tid; v < V; v += kSampleThreads) {
      const uint32_t key = order_key(row[v]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + hist[d] >= left) break;
        cum += hist[d];
      }
      s_prefix = prefix | ((uint32_t)d << shift);
      s_left = left - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    left = s_left;
    mask |= 255u << shift;
  }
  const uint32_t T = prefix;          // the k-th largest key; `left` of the keys equal to it are taken

  // 2. candidates: keys above T (any order) and the first `left` equal to T
  // in index order; each as (key << 32) | ~index, so one descending sort
  // orders by logit desc, then index asc
  if (tid == 0) {
    s_ngt = 0;
    s_neq = 0;
  }
  s_key[tid] = 0;                     // padding sorts last
  __syncthreads();
  const int n_gt = k - (int)left;
  for (int base = 0; base < V; base += kSampleThreads) {
    const int v = base + tid;
    const uint32_t key = v < V ? order_key(row[v]) : 0u;
    const bool gt = v < V && key > T, eq = v < V && key == T;
    // rank of this equal key among the chunk's equal keys (index order)
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t bal = __ballot(eq);
    const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_c[wave] = __popcll(bal);
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s_c[w];
    const int eq_base = s_neq;
    if (gt) {
      const int slot = atomicAdd(&s_ngt, 1);
      s_key[slot] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)v;
    }
    if (eq) {
      const int r = eq_base + before + in_wave;
      if (r < (int)left) s_key[n_gt + r] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)v;
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kSampleThreads / 64; ++w) tot += s_c[w];
      s_neq = eq_base + tot;
    }
    __syncthreads();
  }

  // 3. bitonic sort, descending
  for (int size = 2; size <= kSampleThreads; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = tid ^ stride;
      if (partner > tid) {
        const uint64_t a = s_key[tid], c = s_key[partner];
        const bool desc = (tid & size) == 0;
        if (desc ? (a < c) : (a > c)) {
          s_key[tid] = c;
          s_key[partner] = a;
        }
      }
      __syncthreads();
    }
  }

  // 4. weights, cumulative sums, the top-p prefix and the pick
  const int idx = (int)~(uint32_t)(s_key[min(tid, k - 1)] & 0xFFFFFFFFu);
  const int idx0 = (int)~(uint32_t)(s_key[0] & 0xFFFFFFFFu);
  const float l0 = row[idx0];
  const float w = tid < k ? __expf((row[idx] - l0) * inv_temp) : 0.f;
  const float C = block_inclusive_scan(w, s_w);
  __shared__ float s_total, s_cm;
  if (tid == k - 1) s_total = C;
  __syncthreads();
  const float thr = top_p * s_total;
  const int m = min(k, 1 + block_count(tid < k && C < thr, s_c));
  if (tid == m - 1) s_cm = C;
  __syncthreads();
  const int n = pos_dev[b];           // tokens the sequence holds before the one chosen here
  const uint64_t word = philox_word0((uint64_t)n, (uint64_t)b, seed);
  const float u = (float)(word >> 40) * (1.0f / 16777216.0f);
  const float r = u * s_cm;
  const int j = min(m - 1, block_count(tid < m && C <= r, s_c));
  if (tid == j) {
    int tok = idx;
    if (finished) {
      if (finished[b]) tok = eos;
      else if (tok == eos) finished[b] = 1;
    }
    next[b] = tok;
  }
}

// The end-of-sequence rule after a greedy choice: a finished sequence emits
// eos again; one that emits eos is finished.
__global__ void __launch_bounds__(64) eos_kernel(int32_t *next, int *finished, int eos, int B) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= B) return;
  if (finished[b]) next[b] = eos;
  else if (next[b] == eos) finished[b] = 1;
}

__global__ void __launch_bounds__(64) fill_int_kernel(int *p, int v, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_sample(hipStream_t s, const float *logits, int64_t row_stride, int B, int V, float temperature,
                         int top_k, float top_p, uint64_t seed, const int *pos_dev, int32_t *next, int *finished,
                         int eos) {
  if (B <= 0) return hipSuccess;
  if (top_k < 1 || top_k > kSampleThreads || !(temperature > 0.f)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(kSampleThreads), 0, s, logits, row_stride, V, 1.0f / temperature,
                     top_k, top_p, seed, pos_dev, next, finished, eos);
  return hipGetLastError();
}

hipError_t launch_eos(hipStream_t s, int32_t *next, int *finished, int eos, int B) {
  if (B <= 0) return hipSuccess;
  eos_kernel<<<(B + 63) / 64, 64, 0, s>>>(next, finished, eos, B);
  return hipGetLastError();
}

hipError_t launch_fill_int(hipStream_t s, int *p, int v, int n) {
  if (n <= 0) return hipSuccess;
  fill_int_kernel<<<(n + 63) / 64, 64, 0, s>>>(p, v, n);
  return hipGetLastError();
}

}  // namespace qw
