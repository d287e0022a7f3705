// Row-wise kernels of the decoder forward and the set-up kernels of qw_create.
//
//  embed      token id -> residual row ("augur": full forward pass starts from
//             the embedding table; "LLM Speedrun: Architecture", harness
//             listing's Embedding: the table is [vocab, hidden]).
//  rmsnorm    "LLM Speedrun: Architecture", section "Normalization": each row
//             divided by sqrt(mean(x^2) + eps), times the norm weight.
//  rope_cache q/k/v bias ("Introducing bias"), split-half RoPE on q and k
//             ("Split-half RoPE implementation"), and the write of k and v
//             into the preallocated cache ("augur": preallocated KV-cache).
//  argmax     greedy choice: lowest index of the largest logit.
#include "qw_internal.h"

#include <math.h>

namespace qw {

// ---------------------------------------------------------------- embed
// Row r is token t = r % rows_per_seq of sequence b = r / rows_per_seq, whose
// id sits at ids[b * ids_stride + t].
template <typename T>
__global__ void __launch_bounds__(256) embed_kernel(const int32_t *__restrict__ ids, int rows_per_seq,
                                                    int64_t ids_stride, const T *__restrict__ emb,
                                                    float emb_scale, int hidden, int vocab,
                                                    float *__restrict__ x, int *__restrict__ bad) {
  const int r = blockIdx.x;
  int id = ids[(int64_t)(r / rows_per_seq) * ids_stride + r % rows_per_seq];
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) atomicOr(bad, kFlagBadId);
    id = 0;
  }
  const T *src = emb + (int64_t)id * hidden;
  float *dst = x + (int64_t)r * hidden;
  for (int c = threadIdx.x; c < hidden; c += blockDim.x) dst[c] = to_f32(src[c]) * emb_scale;
}

hipError_t launch_embed(hipStream_t s, bool f16_mode, const int32_t *ids, int rows, int rows_per_seq,
                        int64_t ids_stride, const void *emb, float emb_scale, int hidden, int vocab, float *x,
                        int *bad) {
  if (rows <= 0) return hipSuccess;
  if (rows_per_seq < 1) return hipErrorInvalidValue;
  if (f16_mode)
    QW_LAUNCH((embed_kernel<f16>), dim3(rows), dim3(256), 0, s, ids, rows_per_seq, ids_stride, (const f16 *)emb,
              emb_scale, hidden, vocab, x, bad);
  else
    QW_LAUNCH((embed_kernel<float>), dim3(rows), dim3(256), 0, s, ids, rows_per_seq, ids_stride,
              (const float *)emb, emb_scale, hidden, vocab, x, bad);
  return hipGetLastError();
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- rmsnorm
// One wave per row; fp32 statistics; the product is rounded once to T.
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float *__restrict__ x, int rows, int row_stride,
                                                      int hidden, const float *__restrict__ w, float eps,
                                                      T *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (int64_t)r * row_stride);
  const int n4 = hidden >> 2;
  float ss = 0.f;
  for (int c = lane; c < n4; c += 64) {
    float4 v = xr[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)hidden + eps);
  const float4 *w4 = reinterpret_cast<const float4 *>(w);
  T *o = out + (int64_t)r * hidden;
  for (int c = lane; c < n4; c += 64) {
    float4 v = xr[c], g = w4[c];
    o[4 * c + 0] = from_f32<T>(v.x * inv * g.x);
    o[4 * c + 1] = from_f32<T>(v.y * inv * g.y);
    o[4 * c + 2] = from_f32<T>(v.z * inv * g.z);
    o[4 * c + 3] = from_f32<T>(v.w * inv * g.w);
  }
}

// The same norm with f16 output in the unit-tiled layout (a GEMM operand).
// One workgroup of 16 waves per 16-row block, so a block's tiles are written
// from one XCD's L2 (four-row workgroups put each tile's rows on four XCDs,
// and their partial-line writes cost 60% more time).  Lane (i, g) of wave w
// takes row i and values 8g .. 8g + 7 of the 32-value units w, w + 16, ...
// (at most U of them), held in registers between the two passes: every load
// is issued at once, and each store of a wave is one whole 1 KB tile.  The
// row's sum of squares is added over the lanes of the row, then over the 16
// waves in a fixed order.
template <int U>
__global__ void __launch_bounds__(1024) rmsnorm_tiled_kernel(const float *__restrict__ x, int rows, int row_stride,
                                                             int hidden, const float *__restrict__ w, float eps,
                                                             f16 *__restrict__ out) {
  __shared__ float s_ss[16][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int r = blockIdx.x * 16 + i;
  const bool live = r < rows;
  const float *xr = x + (int64_t)(live ? r : rows - 1) * row_stride + 8 * g;
  const int units = hidden >> 5;
  float4 a[U], b[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int t = wave + 16 * j;
    if (t < units) {
      a[j] = *reinterpret_cast<const float4 *>(xr + 32 * t);
      b[j] = *reinterpret_cast<const float4 *>(xr + 32 * t + 4);
    } else {
      a[j] = b[j] = float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < U; ++j)
    ss += a[j].x * a[j].x + a[j].y * a[j].y + a[j].z * a[j].z + a[j].w * a[j].w + b[j].x * b[j].x +
          b[j].y * b[j].y + b[j].z * b[j].z + b[j].w * b[j].w;
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  if (g == 0) s_ss[wave][i] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) tot += s_ss[v][i];
  const float inv = 1.0f / sqrtf(tot / (float)hidden + eps);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int t = wave + 16 * j;
    if (t >= units) break;
    const float4 wa = *reinterpret_cast<const float4 *>(w + 32 * t + 8 * g);
    const float4 wb = *reinterpret_cast<const float4 *>(w + 32 * t + 8 * g + 4);
    f16x8_t v;
    v[0] = (f16)(a[j].x * inv * wa.x);
    v[1] = (f16)(a[j].y * inv * wa.y);
    v[2] = (f16)(a[j].z * inv * wa.z);
    v[3] = (f16)(a[j].w * inv * wa.w);
    v[4] = (f16)(b[j].x * inv * wb.x);
    v[5] = (f16)(b[j].y * inv * wb.y);
    v[6] = (f16)(b[j].z * inv * wb.z);
    v[7] = (f16)(b[j].w * inv * wb.w);
    if (live) *reinterpret_cast<f16x8_t *>(out + tile_off(r, 32 * t + 8 * g, hidden)) = v;
  }
}

hipError_t launch_rmsnorm(hipStream_t s, bool f16_mode, const float *x, int rows, int row_stride, int hidden,
                          const float *w, float eps, void *out, bool tiled) {
  if (rows <= 0) return hipSuccess;
  if (tiled && (!f16_mode || hidden % 32 || hidden > kRmsTiledMaxHidden)) return hipErrorInvalidValue;
  if (tiled) {
    // units of 32 values per wave (16 waves)
    const int per_wave = (hidden / 32 + 15) / 16;
    const dim3 grid((rows + 15) / 16);
    if (per_wave <= 2)
      QW_LAUNCH(rmsnorm_tiled_kernel<2>, grid, dim3(1024), 0, s, x, rows, row_stride, hidden, w, eps, (f16 *)out);
    else if (per_wave <= 4)
      QW_LAUNCH(rmsnorm_tiled_kernel<4>, grid, dim3(1024), 0, s, x, rows, row_stride, hidden, w, eps, (f16 *)out);
    else if (per_wave <= 8)
      QW_LAUNCH(rmsnorm_tiled_kernel<8>, grid, dim3(1024), 0, s, x, rows, row_stride, hidden, w, eps, (f16 *)out);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  dim3 grid((rows + 3) / 4);
  if (f16_mode)
    QW_LAUNCH((rmsnorm_kernel<f16>), dim3(grid), dim3(256), 0, s, x, rows, row_stride, hidden, w, eps, (f16 *)out);
  else
    QW_LAUNCH((rmsnorm_kernel<float>), dim3(grid), dim3(256), 0, s, x, rows, row_stride, hidden, w, eps, (float *)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bias + RoPE + cache write
// One block per row.  Work item i enumerates (head, pair) over the q heads,
// then the k heads (both rotated), then the v heads (copied).
// Rows of equal-length sequences (row t is position t % rows_per_seq of
// sequence t / rows_per_seq, after pos0 or pos0_dev[b]), or ragged ones
// (sequence s holds rows cu[s] .. cu[s+1]-1 from position 0).
template <typename T>
__global__ void __launch_bounds__(256) rope_cache_kernel(RopeCacheArgs a) {
  const int t = blockIdx.x;
  const int half = a.head_dim >> 1;
  int b, pos;
  if (a.rag.cu) {
    b = ragged_seq(a.rag.cu, a.rag.n, t);
    pos = t - a.rag.cu[b];
  } else {
    b = t / a.rows_per_seq;
    pos = (a.pos0_dev ? a.pos0_dev[b] : a.pos0) + (t % a.rows_per_seq);
  }
  const int qd = a.n_heads * a.head_dim, kvd = a.n_kv_heads * a.head_dim;
  const int ncols = qd + 2 * kvd;
  const float *row = a.qkv + (int64_t)t * ncols;
  const float2 *cs = a.rope + (int64_t)pos * half;
  const int n_items = (a.n_heads + 2 * a.n_kv_heads) * half;
  for (int it = threadIdx.x; it < n_items; it += blockDim.x) {
    const int head = it / half, i = it % half;
    const int c0 = head * a.head_dim + i, c1 = c0 + half;   // column in qkv
    float re = row[c0] + a.bias[c0];
    float im = row[c1] + a.bias[c1];
    if (head < a.n_heads + a.n_kv_heads) {                  // q or k: rotate
      const float2 r = cs[i];
      const float nre = re * r.x - im * r.y;
      const float nim = im * r.x + re * r.y;
      re = nre;
      im = nim;
    }
    if (head < a.n_heads) {
      T *q = (T *)a.q_out + (int64_t)t * qd;
      q[c0] = from_f32<T>(re);
      q[c1] = from_f32<T>(im);
    } else {
      const bool is_k = head < a.n_heads + a.n_kv_heads;
      const int j = is_k ? head - a.n_heads : head - a.n_heads - a.n_kv_heads;
      T *cache = (T *)(is_k ? a.k_cache : a.v_cache);
      T *dst = cache + kv_offset(a.kv, a.n_kv_heads, a.head_dim, b, j, pos);
      dst[i] = from_f32<T>(re);
      dst[i + half] = from_f32<T>(im);
    }
  }
}

// The same in f16 mode, four consecutive rotation pairs per thread: float4
// reads of the projections, biases and (cos, sin), 8-byte writes (half a
// head a multiple of 4).  The arithmetic of each element is unchanged.
__global__ void __launch_bounds__(256) rope_cache4_kernel(RopeCacheArgs a) {
  const int t = blockIdx.x;
  const int half = a.head_dim >> 1;
  int b, pos;
  if (a.rag.cu) {
    b = ragged_seq(a.rag.cu, a.rag.n, t);
    pos = t - a.rag.cu[b];
  } else {
    b = t / a.rows_per_seq;
    pos = (a.pos0_dev ? a.pos0_dev[b] : a.pos0) + (t % a.rows_per_seq);
  }
  const int qd = a.n_heads * a.head_dim, kvd = a.n_kv_heads * a.head_dim;
  const int ncols = qd + 2 * kvd;
  const float *row = a.qkv + (int64_t)t * ncols;
  const float2 *cs = a.rope + (int64_t)pos * half;
  const int n4 = (a.n_heads + 2 * a.n_kv_heads) * half / 4;
  for (int it4 = threadIdx.x; it4 < n4; it4 += blockDim.x) {
    const int it = 4 * it4, head = it / half, i = it % half;
    const int c0 = head * a.head_dim + i, c1 = c0 + half;
    const float4 x0 = *reinterpret_cast<const float4 *>(row + c0), x1 = *reinterpret_cast<const float4 *>(row + c1);
    const float4 b0 = *reinterpret_cast<const float4 *>(a.bias + c0), b1 = *reinterpret_cast<const float4 *>(a.bias + c1);
    float re[4] = {x0.x + b0.x, x0.y + b0.y, x0.z + b0.z, x0.w + b0.w};
    float im[4] = {x1.x + b1.x, x1.y + b1.y, x1.z + b1.z, x1.w + b1.w};
    if (head < a.n_heads + a.n_kv_heads) {
      const float4 r01 = *reinterpret_cast<const float4 *>(cs + i), r23 = *reinterpret_cast<const float4 *>(cs + i + 2);
      const float cr[4] = {r01.x, r01.z, r23.x, r23.z}, sr[4] = {r01.y, r01.w, r23.y, r23.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float nre = re[k] * cr[k] - im[k] * sr[k];
        const float nim = im[k] * cr[k] + re[k] * sr[k];
        re[k] = nre;
        im[k] = nim;
      }
    }
    f16 *dst;
    if (head < a.n_heads) {
      dst = (f16 *)a.q_out + (int64_t)t * qd + c0;
    } else {
      const bool is_k = head < a.n_heads + a.n_kv_heads;
      const int j = is_k ? head - a.n_heads : head - a.n_heads - a.n_kv_heads;
      dst = (f16 *)(is_k ? a.k_cache : a.v_cache) + kv_offset(a.kv, a.n_kv_heads, a.head_dim, b, j, pos) + i;
    }
    typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
    const f16x4v lo = {(f16)re[0], (f16)re[1], (f16)re[2], (f16)re[3]};
    const f16x4v hi = {(f16)im[0], (f16)im[1], (f16)im[2], (f16)im[3]};
    *reinterpret_cast<f16x4v *>(dst) = lo;
    *reinterpret_cast<f16x4v *>(dst + half) = hi;
  }
}

hipError_t launch_rope_cache(hipStream_t s, bool f16_mode, const RopeCacheArgs &a) {
  if (a.T <= 0) return hipSuccess;
  if (f16_mode && (a.head_dim / 2) % 4 == 0)
    QW_LAUNCH((rope_cache4_kernel), dim3(a.T), dim3(256), 0, s, a);
  else if (f16_mode)
    QW_LAUNCH((rope_cache_kernel<f16>), dim3(a.T), dim3(256), 0, s, a);
  else
    QW_LAUNCH((rope_cache_kernel<float>), dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- argmax
// One block per row.  Ties go to the lowest index; NaN never wins.
__global__ void __launch_bounds__(256) argmax_kernel(const float *__restrict__ logits, int vocab, int64_t stride,
                                                     int32_t *__restrict__ next_ids, int *pos_dev, int pos_add,
                                                     int *flag) {
  const float *row = logits + (int64_t)blockIdx.x * stride;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  bool finite = true;
  for (int v = threadIdx.x; v < vocab; v += blockDim.x) {
    const float x = row[v];
    if (x > best) { best = x; bi = v; }      // v increases, so the first max is kept
    finite = finite && (fabsf(x) <= 3.4e38f);
  }
  if (!finite) atomicOr(flag, kFlagNonFinite);
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  __shared__ float sb[4];
  __shared__ int si[4];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sb[wv] = best; si[wv] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < bi)) { best = sb[w]; bi = si[w]; }
    next_ids[blockIdx.x] = (bi == 0x7fffffff) ? 0 : bi;     // all-NaN row: 0
    if (pos_dev) pos_dev[blockIdx.x] += pos_add;
  }
}

hipError_t launch_argmax(hipStream_t s, const float *logits, int rows, int vocab, int64_t row_stride,
                         int32_t *next_ids, int *pos_dev, int pos_add, int *flag) {
  if (rows <= 0) return hipSuccess;
  QW_LAUNCH((argmax_kernel), dim3(rows), dim3(256), 0, s, logits, vocab, row_stride, next_ids, pos_dev, pos_add,
            flag);
  return hipGetLastError();
}


// Copies around the captured decode graph: caller ids into the staging row the
// graph reads, and the graph's next ids (and logits, when asked) out to the
// caller's buffers.
__global__ void __launch_bounds__(256) copy_i32_kernel(int32_t *dst, const int32_t *src, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) stage_out_kernel(int32_t *next_dst, const int32_t *next_src, int b,
                                                        float *logits_dst, const float *logits_src, int64_t n) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid < b) next_dst[tid] = next_src[tid];
  for (int64_t i = tid; i < n; i += (int64_t)gridDim.x * blockDim.x) logits_dst[i] = logits_src[i];
}

hipError_t launch_copy_i32(hipStream_t s, int32_t *dst, const int32_t *src, int n) {
  copy_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(dst, src, n);
  return hipGetLastError();
}

hipError_t launch_stage_out(hipStream_t s, int32_t *next_dst, const int32_t *next_src, int b, float *logits_dst,
                            const float *logits_src, int64_t n_logits) {
  const int64_t n = logits_dst ? n_logits : 0;
  const int64_t total = n > b ? n : b;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  stage_out_kernel<<<(unsigned)blocks, 256, 0, s>>>(next_dst, next_src, b, logits_dst, logits_src, n);
  return hipGetLastError();
}

// Generation bookkeeping: dst[b * dst_stride + dst_col] = src[b] for b < B
// (and, if seq is non-NULL, seq[b * seq_stride + seq_col] = src[b]).
__global__ void __launch_bounds__(64) put_column_kernel(int32_t *dst, int64_t dst_stride, int dst_col,
                                                        int32_t *seq, int64_t seq_stride, int seq_col,
                                                        const int32_t *src, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  dst[(int64_t)b * dst_stride + dst_col] = src[b];
  if (seq) seq[(int64_t)b * seq_stride + seq_col] = src[b];
}

hipError_t launch_put_column(hipStream_t s, int32_t *dst, int64_t dst_stride, int dst_col, int32_t *seq,
                             int64_t seq_stride, int seq_col, const int32_t *src, int B) {
  put_column_kernel<<<(B + 63) / 64, 64, 0, s>>>(dst, dst_stride, dst_col, seq, seq_stride, seq_col, src, B);
  return hipGetLastError();
}

// dst[r * dst_stride + c] = src[r * src_stride + c] for r < rows, c < n
// (int32 rows when bytes == 4 ... both callers move int32 or float rows).
__global__ void __launch_bounds__(256) copy_rows_kernel(uint32_t *dst, int64_t dst_stride, const uint32_t *src,
                                                        int64_t src_stride, int64_t n) {
  const int r = blockIdx.y;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x)
    dst[r * dst_stride + c] = src[r * src_stride + c];
}

hipError_t launch_copy_rows(hipStream_t s, void *dst, int64_t dst_stride, const void *src, int64_t src_stride,
                            int rows, int64_t n) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  int64_t bx = (n + 255) / 256;
  if (bx > 1024) bx = 1024;
  copy_rows_kernel<<<dim3((unsigned)bx, rows), 256, 0, s>>>((uint32_t *)dst, dst_stride, (const uint32_t *)src,
                                                             src_stride, n);
  return hipGetLastError();
}

struct PutChunk {
  int n;
  int idx[kPutChunk], val[kPutChunk];
};

__global__ void __launch_bounds__(256) put_ints_kernel(int *dst, PutChunk c) {
  const int k = threadIdx.x;
  if (k < c.n) dst[c.idx[k]] = c.val[k];
}

hipError_t launch_put_ints(hipStream_t s, int *dst, const int *idx, const int *val, int n) {
  for (int k0 = 0; k0 < n; k0 += kPutChunk) {
    PutChunk c;
    c.n = n - k0 < kPutChunk ? n - k0 : kPutChunk;
    for (int k = 0; k < c.n; ++k) {
      c.idx[k] = idx[k0 + k];
      c.val[k] = val[k0 + k];
    }
    put_ints_kernel<<<1, 256, 0, s>>>(dst, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ void __launch_bounds__(256) gather_last_rows_kernel(float *dst, const float *src, const int *cu, int H) {
  const int k = blockIdx.x;
  const float *row = src + (int64_t)(cu[k + 1] - 1) * H;
  for (int c = threadIdx.x; c < H; c += 256) dst[(int64_t)k * H + c] = row[c];
}

hipError_t launch_gather_last_rows(hipStream_t s, float *dst, const float *src, const int *cu, int n, int H) {
  if (n <= 0) return hipSuccess;
  gather_last_rows_kernel<<<n, 256, 0, s>>>(dst, src, cu, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------- set-up
// Element i of a weight tensor stored as kind (kWeightF32, kWeightBF16 or
// kWeightF16), as a float (exact for all three).
__device__ __forceinline__ float load_src(const void *p, int64_t i, int kind) {
  if (kind == kWeightBF16) return bf16_bits_to_f32(((const uint16_t *)p)[i]);
  if (kind == kWeightF16) return (float)((const f16 *)p)[i];
  return ((const float *)p)[i];
}

// Largest |value| as float bits.  Magnitudes are compared as unsigned bit
// patterns (the same order for non-negative floats), which keeps an inf or
// NaN as the maximum so that qw_create can reject it.
__global__ void __launch_bounds__(256) absmax_kernel(const void *src, int64_t n, int kind, unsigned *out) {
  unsigned m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    m = max(m, __float_as_uint(fabsf(load_src(src, i, kind))));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(out, m);
}

hipError_t launch_absmax(hipStream_t s, int src_kind, const void *src, int64_t n, unsigned *out_bits) {
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  absmax_kernel<<<blocks, 256, 0, s>>>(src, n, src_kind, out_bits);
  return hipGetLastError();
}

template <typename D>
__global__ void __launch_bounds__(256) convert_kernel(const void *src, int64_t n, int kind, D *dst, float scale) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = from_f32<D>(load_src(src, i, kind) * scale);
}

hipError_t launch_convert(hipStream_t s, int src_kind, const void *src, int64_t n, bool dst_f16, void *dst,
                          int64_t dst_offset, float scale) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 16384) blocks = 16384;
  if (dst_f16)
    convert_kernel<f16><<<blocks, 256, 0, s>>>(src, n, src_kind, (f16 *)dst + dst_offset, scale);
  else
    convert_kernel<float><<<blocks, 256, 0, s>>>(src, n, src_kind, (float *)dst + dst_offset, scale);
  return hipGetLastError();
}

template <typename D>
__global__ void __launch_bounds__(256) convert_gu_kernel(const void *gate, const void *up, int inter, int hidden,
                                                         int kind, D *dst, float scale) {
  const int64_t n = 2LL * inter * hidden;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t drow = i / hidden;
    const int c = (int)(i % hidden);
    const int64_t blk = drow / (2 * GU_BLOCK);
    const int within = (int)(drow % (2 * GU_BLOCK));
    const bool is_up = within >= GU_BLOCK;
    const int64_t f = blk * GU_BLOCK + (is_up ? within - GU_BLOCK : within);
    dst[i] = from_f32<D>(load_src(is_up ? up : gate, f * hidden + c, kind) * scale);
  }
}

hipError_t launch_convert_gu(hipStream_t s, int src_kind, const void *gate, const void *up, int inter, int hidden,
                             bool dst_f16, void *dst, float scale) {
  const int64_t n = 2LL * inter * hidden;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 16384) blocks = 16384;
  if (dst_f16)
    convert_gu_kernel<f16><<<blocks, 256, 0, s>>>(gate, up, inter, hidden, src_kind, (f16 *)dst, scale);
  else
    convert_gu_kernel<float><<<blocks, 256, 0, s>>>(gate, up, inter, hidden, src_kind, (float *)dst, scale);
  return hipGetLastError();
}

// dst[c][r] = src[r][c] * scale for a [rows, cols] source (f16 destination):
// the down projection's [I, H] copy that the decode MLP reads row by row.
// 32 x 32 tiles through LDS so both sides are read and written along rows.
__global__ void __launch_bounds__(256) convert_t_kernel(const void *src, int rows, int cols, int kind, f16 *dst,
                                                        float scale) {
  __shared__ float t[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    t[y][tx] = (r < rows && c < cols) ? load_src(src, (int64_t)r * cols + c, kind) * scale : 0.f;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (c < cols && r < rows) dst[(int64_t)c * rows + r] = (f16)t[tx][y];
  }
}

hipError_t launch_convert_t(hipStream_t s, int src_kind, const void *src, int rows, int cols, void *dst,
                            float scale) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  convert_t_kernel<<<grid, 256, 0, s>>>(src, rows, cols, src_kind, (f16 *)dst, scale);
  return hipGetLastError();
}

// Unit-tiled copy of an f16 weight matrix (layout in qw_internal.h): one
// thread per 16 bytes of the destination, read as 16 bytes of one source row.
__global__ void __launch_bounds__(256) tile_units_kernel(const f16 *W, int N, int K, f16 *Wt, int64_t n8) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;      // 16-byte piece c of Wt
  if (c >= n8) return;
  const int64_t tile = c >> 6;
  const int l = (int)(c & 63), i = l & 15, g = l >> 4;
  const int units = K >> 5;
  const int row = (int)(tile / units) * 16 + i, k = (int)(tile % units) * 32 + 8 * g;
  f16x8_t v = {};
  if (row < N) v = *reinterpret_cast<const f16x8_t *>(W + (int64_t)row * K + k);
  *reinterpret_cast<f16x8_t *>(Wt + c * 8) = v;
}

hipError_t launch_tile_units(hipStream_t s, const void *W, int N, int K, void *Wt) {
  if (N <= 0 || K <= 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  const int64_t n8 = (int64_t)(N + kTileRows - 1) / kTileRows * kTileRows * K / 8;
  tile_units_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>((const f16 *)W, N, K, (f16 *)Wt, n8);
  return hipGetLastError();
}

// RoPE table: entry (pos, i) = (cos, sin) of pos * theta^(-2i/hd), evaluated in
// double and rounded once to float ("Rotary Positional Embeddings RoPE").
__global__ void __launch_bounds__(256) rope_table_kernel(float2 *table, int max_seq, int head_dim, double theta) {
  const int half = head_dim / 2;
  const int64_t n = (int64_t)max_seq * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(e / half), i = (int)(e % half);
    const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)head_dim);
    table[e] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

hipError_t launch_rope_table(hipStream_t s, float2 *table, int max_seq, int head_dim, double theta) {
  const int64_t n = (int64_t)max_seq * (head_dim / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  rope_table_kernel<<<blocks, 256, 0, s>>>(table, max_seq, head_dim, theta);
  return hipGetLastError();
}

}  // namespace qw
