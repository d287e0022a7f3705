// Kernels of one decode step (one new token per sequence, B <= 32 sequences).
//
// What a step computes is the decoder block of "LLM Speedrun: Architecture"
// (sections "Attention", "Grouped Query Attention GQA", "Split-half RoPE
// implementation", "Introducing bias", "Decoding") for one row per sequence,
// reading past keys and values from the preallocated cache ("augur").  How it
// is laid out is specific to this GPU:
//
//  * Kernel boundaries are the only cheap device-wide synchronisation here,
//    and a device-scope fence per workgroup is expensive, so no kernel waits
//    on another workgroup.  Projections split K over workgroups and add their
//    partial sums with 64-bit integer atomics on a fixed-point copy of the
//    value (32 fractional bits).  Integer addition is associative, so the
//    result does not depend on arrival order (deterministic), and no fence
//    is needed: the consumer is the next kernel.
//  * The consumer of each fixed-point sum finishes the step it belongs to:
//    attention converts the q/k/v sums, adds the bias, applies RoPE and writes
//    k and v into the cache; the down projection converts the gate/up sums and
//    applies silu(gate) * up while loading its operand; the RMSNorm kernel
//    converts the residual stream.
//  * The residual stream of the decode rows lives in fixed point ([B, H]
//    int64), so o_proj and down_proj add into it atomically.
#include "qw_internal.h"

#include <math.h>

namespace qw {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float FIX_ONE = 4294967296.0f;        // 2^32
constexpr float FIX_INV = 2.3283064365386963e-10f;  // 2^-32
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ long long to_fix(float v) {
  v = fminf(fmaxf(v, -1.0e9f), 1.0e9f);
  return __float2ll_rn(v * FIX_ONE);
}
__device__ __forceinline__ float from_fix(long long q) { return (float)q * FIX_INV; }
__device__ __forceinline__ void fix_add(long long *p, float v) {
  atomicAdd(reinterpret_cast<unsigned long long *>(p), (unsigned long long)to_fix(v));
}
__device__ __forceinline__ f16x8 load8(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

// ---------------------------------------------------------------- begin / norm / end
// x_fix[b] = embedding row of ids[b] (exact value, fixed point)
__global__ void __launch_bounds__(256) dec_embed_kernel(const int32_t *ids, const f16 *emb, float emb_scale, int H,
                                                        int V, long long *x_fix, int *bad) {
  const int b = blockIdx.x;
  int id = ids[b];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(bad, 1);
    id = 0;
  }
  const f16 *row = emb + (int64_t)id * H;
  for (int c = threadIdx.x; c < H; c += blockDim.x) x_fix[(int64_t)b * H + c] = to_fix((float)row[c] * emb_scale);
}

// u[b] = f16(x[b] / sqrt(mean(x[b]^2) + eps) * w), and clears `zero_buf`
// (the fixed-point accumulator the next projection adds into).
__global__ void __launch_bounds__(256) dec_norm_kernel(const long long *x_fix, int H, const float *w, float eps, f16 *u,
                                                       long long *zero_buf, int zero_per_row) {
  const int b = blockIdx.x;
  __shared__ float red[4];
  const long long *xr = x_fix + (int64_t)b * H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += 256) {
    const float v = from_fix(xr[c]);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += 256) u[(int64_t)b * H + c] = (f16)(from_fix(xr[c]) * inv * w[c]);
  if (zero_buf)
    for (int c = threadIdx.x; c < zero_per_row; c += 256) zero_buf[(int64_t)b * zero_per_row + c] = 0;
}

// Reduce the LM head's per-block (max, index) pairs: lowest index among equal
// maxima.  Advances the device-side position.
__global__ void __launch_bounds__(256) dec_end_kernel(const float *pv, const int *pi, int nblk, int32_t *next,
                                                      int *pos_dev) {
  const int b = blockIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int k = threadIdx.x; k < nblk; k += 256) {
    const float v = pv[(int64_t)b * nblk + k];
    const int i = pi[(int64_t)b * nblk + k];
    if (v > best || (v == best && i < bi)) { best = v; bi = i; }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  __shared__ float sb[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sb[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sb[w] > best || (sb[w] == best && si[w] < bi)) { best = sb[w]; bi = si[w]; }
    next[b] = (bi == 0x7fffffff) ? 0 : bi;
    if (b == 0) *pos_dev += 1;
  }
}

// ---------------------------------------------------------------- projections
// out[b, n] (+)= sum_k act[b, k] * W[n, k] * scale for b < M <= 16 * NB.
// One wave = 16 weight rows x a K slice; a workgroup = 4 waves = 64 rows;
// gridDim.y = K slices.  See the header comment for the fixed-point output.
enum class DecAct : int { F16 = 0, SwiGLUFix = 1 };
enum class DecOut : int { FixAdd = 0, Logits = 1 };

template <int NB, DecAct AM, DecOut OM>
__global__ void __launch_bounds__(256) dec_gemv_kernel(DecGemvArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 15, g = lane >> 4;
  const int nblk = blockIdx.x, split = blockIdx.y;
  const int row = nblk * 64 + wave * 16 + i;
  const bool row_ok = row < a.N;
  const f16 *W = (const f16 *)a.W + (int64_t)(row_ok ? row : 0) * a.K;
  const int units = a.K >> 5;
  const int u0 = split * a.units_per_split;
  const int u1 = min(units, u0 + a.units_per_split);

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f16x8 zero = {};

  // 8 consecutive activations of batch row b at column k, as f16
  auto act8 = [&](int b, int k) -> f16x8 {
    if constexpr (AM == DecAct::F16) {
      return load8((const f16 *)a.act + (int64_t)b * a.lda + k);
    } else {
      // k indexes features; gate/up of feature f sit in GU_BLOCK-interleaved rows
      const long long *row2 = a.act_fix + (int64_t)b * a.lda;
      const int blk = k / GU_BLOCK, w = k % GU_BLOCK;
      const long long *gp = row2 + blk * 2 * GU_BLOCK + w;
      const long long *up = gp + GU_BLOCK;
      f16x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gt = from_fix(gp[e]), uv = from_fix(up[e]);
        r[e] = (f16)(silu_f(gt) * uv);
      }
      return r;
    }
  };

  int u = u0;
  for (; u + 4 <= u1; u += 4) {
    const int kb = u * 32 + g * 32;            // lane group g: k = kb .. kb + 31
    f16x8 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = row_ok ? load8(W + kb + c * 8) : zero;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + i;
      const bool b_ok = b < a.M;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x8 x = b_ok ? act8(b, kb + c * 8) : zero;
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[c], x, acc[nb], 0, 0, 0);
      }
    }
  }
  for (; u < u1; ++u) {
    const int kb = u * 32 + g * 8;
    const f16x8 w = row_ok ? load8(W + kb) : zero;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + i;
      const f16x8 x = (b < a.M) ? act8(b, kb) : zero;
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w, x, acc[nb], 0, 0, 0);
    }
  }

  // accumulator: lane (i, g) holds rows 4g..4g+3 (of the wave's 16) of batch column i
  const int nw = nblk * 64 + wave * 16 + 4 * g;
  if constexpr (OM == DecOut::FixAdd) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + i;
      if (b >= a.M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (nw + r < a.N) fix_add(a.out_fix + (int64_t)b * a.ldo + nw + r, acc[nb][r] * a.scale);
    }
  } else {
    // logits (optional copy) and this block's (max, lowest index) per batch row
    __shared__ float s_v[4][16 * NB];
    __shared__ int s_i[4][16 * NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int b = nb * 16 + i;
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = nw + r;
        const float v = acc[nb][r] * a.scale;
        if (n < a.N && b < a.M) {
          if (a.logits) a.logits[(int64_t)b * a.ldo + n] = v;
          if (v > best) { best = v; bi = n; }     // n increases with r
        }
      }
      // lanes i, i+16, i+32, i+48 share batch column i
#pragma unroll
      for (int off = 16; off < 64; off <<= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      if (g == 0) {
        s_v[wave][b] = best;
        s_i[wave][b] = bi;
      }
    }
    __syncthreads();
    if (tid < a.M) {
      float best = s_v[0][tid];
      int bi = s_i[0][tid];
      for (int w = 1; w < 4; ++w)
        if (s_v[w][tid] > best || (s_v[w][tid] == best && s_i[w][tid] < bi)) { best = s_v[w][tid]; bi = s_i[w][tid]; }
      a.arg_v[(int64_t)tid * gridDim.x + nblk] = best;
      a.arg_i[(int64_t)tid * gridDim.x + nblk] = bi;
    }
  }
}

template <int NB>
hipError_t launch_gemv_nb(hipStream_t s, const DecGemvArgs &a, dim3 grid) {
  if (a.logits_mode) {
    dec_gemv_kernel<NB, DecAct::F16, DecOut::Logits><<<grid, 256, 0, s>>>(a);
  } else if (a.act_fix) {
    dec_gemv_kernel<NB, DecAct::SwiGLUFix, DecOut::FixAdd><<<grid, 256, 0, s>>>(a);
  } else {
    dec_gemv_kernel<NB, DecAct::F16, DecOut::FixAdd><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention
// grid (n_kv_heads, B), 64 * NW threads (NW = 16 waves for g <= 4, else 8 so
// that the per-lane state of g heads fits in registers).  Prologue: q (the group's g heads), the
// new k and v from the fixed-point q/k/v sums + bias, RoPE at `pos`; k and v
// are written to the cache.  Body: keys 0..pos-1 from the cache, key pos from
// LDS; online softmax in the exp2 domain; merge of all lanes and waves.
template <int HD, int G, int NW>
__global__ void __launch_bounds__(64 * NW) dec_attn_kernel(DecAttnArgs a) {
  constexpr int LPK = HD / 8;        // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per load
  constexpr int KPB = NW * KPW;
  constexpr int HALF = HD / 2;
  __shared__ float s_q[G][HD];
  __shared__ float s_k[HD], s_v[HD];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_o[NW][G][HD];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = lane / LPK, dl = lane % LPK, d0 = dl * 8;
  const int j = blockIdx.x, b = blockIdx.y;
  const int pos = *a.pos_dev;
  const int nq = a.n_kv_heads * G;
  const int qd = nq * HD, kvd = a.n_kv_heads * HD;
  const int ncols = qd + 2 * kvd;
  const long long *acc = a.qkv_fix + (int64_t)b * ncols;
  const float2 *cs = a.rope + (int64_t)pos * HALF;
  const float qscale = a.softmax_scale * LOG2E;

  // prologue: (G + 1) rotated heads (q heads of the group, then k) and v
  for (int e = tid; e < (G + 1) * HALF + HD; e += 64 * NW) {
    if (e < (G + 1) * HALF) {
      const int hh = e / HALF, i = e % HALF;
      const int c0 = (hh < G) ? (j * G + hh) * HD + i : qd + j * HD + i;
      const float re = from_fix(acc[c0]) + a.bias[c0];
      const float im = from_fix(acc[c0 + HALF]) + a.bias[c0 + HALF];
      const float2 r = cs[i];
      const float nre = re * r.x - im * r.y, nim = im * r.x + re * r.y;
      if (hh < G) {
        s_q[hh][i] = (float)(f16)nre * qscale;       // q is rounded to f16 like the prefill path
        s_q[hh][i + HALF] = (float)(f16)nim * qscale;
      } else {
        s_k[i] = (float)(f16)nre;
        s_k[i + HALF] = (float)(f16)nim;
      }
    } else {
      const int d = e - (G + 1) * HALF;
      const int c = qd + kvd + j * HD + d;
      s_v[d] = (float)(f16)(from_fix(acc[c]) + a.bias[c]);
    }
  }
  __syncthreads();
  const int64_t head_base = ((int64_t)b * a.n_kv_heads + j) * a.max_seq * HD;
  f16 *Kc = (f16 *)a.k_cache + head_base;
  f16 *Vc = (f16 *)a.v_cache + head_base;
  if (tid < HD) {
    Kc[(int64_t)pos * HD + tid] = (f16)s_k[tid];
    Vc[(int64_t)pos * HD + tid] = (f16)s_v[tid];
  }

  float q[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[hh][e] = s_q[hh][d0 + e];
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }

  auto visit = [&](const float *kf, const float *vf) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(q[hh][e], kf[e], s);
#pragma unroll
      for (int off = LPK / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      const float mn = fmaxf(m[hh], s);
      const float corr = exp2f(m[hh] - mn);
      const float p = exp2f(s - mn);
      l[hh] = l[hh] * corr + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(p, vf[e], o[hh][e] * corr);
      m[hh] = mn;
    }
  };

  // cached keys 0 .. pos-1, two loads in flight per lane
  for (int kb = wave * KPW; kb < pos; kb += 2 * KPB) {
    const int t0 = kb + slot, t1 = kb + KPB + slot;
    f16x8 k0 = {}, v0 = {}, k1 = {}, v1 = {};
    if (t0 < pos) {
      k0 = load8(Kc + (int64_t)t0 * HD + d0);
      v0 = load8(Vc + (int64_t)t0 * HD + d0);
    }
    if (t1 < pos) {
      k1 = load8(Kc + (int64_t)t1 * HD + d0);
      v1 = load8(Vc + (int64_t)t1 * HD + d0);
    }
    if (t0 < pos) {
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { kf[e] = (float)k0[e]; vf[e] = (float)v0[e]; }
      visit(kf, vf);
    }
    if (t1 < pos) {
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { kf[e] = (float)k1[e]; vf[e] = (float)v1[e]; }
      visit(kf, vf);
    }
  }
  // the new key (position pos), handled by slot 0 of wave 0
  if (wave == 0 && slot == 0) {
    float kf[8], vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { kf[e] = s_k[d0 + e]; vf[e] = s_v[d0 + e]; }
    visit(kf, vf);
  }

  // merge the KPW key slots of each wave
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[hh], off, 64);
      const float lo = __shfl_xor(l[hh], off, 64);
      const float mn = fmaxf(m[hh], mo);
      const float ca = (m[hh] == -INFINITY) ? 0.f : exp2f(m[hh] - mn);
      const float cb = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[hh] = l[hh] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[hh][e], off, 64);
        o[hh][e] = o[hh][e] * ca + oo * cb;
      }
      m[hh] = mn;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (dl == 0) {
        s_m[wave][hh] = m[hh];
        s_l[wave][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][hh][d0 + e] = o[hh][e];
    }
  }
  __syncthreads();
  f16 *out = (f16 *)a.o + (int64_t)b * qd;
  for (int e = tid; e < G * HD; e += 64 * NW) {
    const int hh = e / HD, d = e % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = (s_m[w][hh] == -INFINITY) ? 0.f : exp2f(s_m[w][hh] - M);
      L += s_l[w][hh] * c;
      O += s_o[w][hh][d] * c;
    }
    out[(j * G + hh) * HD + d] = (f16)(O / L);
  }
}

template <int HD>
hipError_t launch_attn_hd(hipStream_t s, const DecAttnArgs &a, dim3 grid, int g) {
  switch (g) {
    case 1: dec_attn_kernel<HD, 1, 16><<<grid, 1024, 0, s>>>(a); break;
    case 2: dec_attn_kernel<HD, 2, 16><<<grid, 1024, 0, s>>>(a); break;
    case 3: dec_attn_kernel<HD, 3, 16><<<grid, 1024, 0, s>>>(a); break;
    case 4: dec_attn_kernel<HD, 4, 16><<<grid, 1024, 0, s>>>(a); break;
    case 5: dec_attn_kernel<HD, 5, 8><<<grid, 512, 0, s>>>(a); break;
    case 6: dec_attn_kernel<HD, 6, 8><<<grid, 512, 0, s>>>(a); break;
    case 7: dec_attn_kernel<HD, 7, 8><<<grid, 512, 0, s>>>(a); break;
    case 8: dec_attn_kernel<HD, 8, 8><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int head_dim, int group, int hidden, int q_dim, int inter) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) && group >= 1 && group <= 8 && hidden % 32 == 0 &&
         q_dim % 32 == 0 && inter % GU_BLOCK == 0;
}

int dec_gemv_splits(int N, int K, int M, int target_groups) {
  const int nblk = (N + 63) / 64;
  const int units = K / 32;
  int splits = (target_groups + nblk - 1) / nblk;
  int max_splits = (units + 3) / 4;            // at least 128 k per slice
  // keep the atomic traffic (8 bytes per output per slice) under ~1/8 of the weight bytes
  const int atomic_cap = (K * 2) / (8 * 8 * (M < 1 ? 1 : M));
  if (atomic_cap >= 1 && max_splits > atomic_cap) max_splits = atomic_cap;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

hipError_t launch_dec_embed(hipStream_t s, const int32_t *ids, int B, const void *emb, float emb_scale, int H, int V,
                            long long *x_fix, int *bad) {
  dec_embed_kernel<<<B, 256, 0, s>>>(ids, (const f16 *)emb, emb_scale, H, V, x_fix, bad);
  return hipGetLastError();
}

hipError_t launch_dec_norm(hipStream_t s, const long long *x_fix, int B, int H, const float *w, float eps, void *u,
                           long long *zero_buf, int zero_per_row) {
  dec_norm_kernel<<<B, 256, 0, s>>>(x_fix, H, w, eps, (f16 *)u, zero_buf, zero_per_row);
  return hipGetLastError();
}

hipError_t launch_dec_end(hipStream_t s, const float *arg_v, const int *arg_i, int nblk, int B, int32_t *next,
                          int *pos_dev) {
  dec_end_kernel<<<B, 256, 0, s>>>(arg_v, arg_i, nblk, next, pos_dev);
  return hipGetLastError();
}

hipError_t launch_dec_gemv(hipStream_t s, const DecGemvArgs &in) {
  DecGemvArgs a = in;
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.M > 32 || (a.K & 31) || (a.lda & 7)) return hipErrorInvalidValue;
  const int units = a.K / 32;
  int splits = a.logits_mode ? 1 : (a.splits < 1 ? 1 : a.splits);
  a.units_per_split = (units + splits - 1) / splits;
  splits = (units + a.units_per_split - 1) / a.units_per_split;
  dim3 grid((a.N + 63) / 64, splits);
  return a.M <= 16 ? launch_gemv_nb<1>(s, a, grid) : launch_gemv_nb<2>(s, a, grid);
}

hipError_t launch_dec_attention(hipStream_t s, const DecAttnArgs &a) {
  const int g = a.n_heads / a.n_kv_heads;
  dim3 grid(a.n_kv_heads, a.batch);
  switch (a.head_dim) {
    case 32: return launch_attn_hd<32>(s, a, grid, g);
    case 64: return launch_attn_hd<64>(s, a, grid, g);
    case 128: return launch_attn_hd<128>(s, a, grid, g);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qw
